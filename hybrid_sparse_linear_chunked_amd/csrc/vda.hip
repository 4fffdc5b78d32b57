// Video Delta Attention (VDA) branch of the VDN hybrid layer (gfx950).
//
// The memory is updated once per frame, all of the frame's tokens jointly solving
// one update that is non-expansive (besthub article "VDN-H3 Generates 14-Second
// 768p Video ...", section Video Delta Attention (VDA)).  Form implemented:
//     S_t = (S_{t-1} + beta_t B_t) A_t^-1,  A_t = I + beta_t G_t,
//     G_t = K_t K_t^T,  B_t = V_t K_t^T   (K_t, V_t: d x N, the frame's tokens).
// Both directions apply the same per-frame affine map S -> S M_t + C_t with
// M_t = A_t^-1 and C_t = beta_t B_t M_t, so the maps are built for every frame in
// parallel (factor_kernel) and the serial part (scan_kernel) is one small GEMM
// per frame.  The forward state of chunk c is the state after frames 1..5c-6
// (ascending), the backward state the state after frames F-2 down to 5(c+2)
// (sd114.wiki article "VDN-Minimax-H3 ...", section 双向线性注意力分支: the states
// cover the frames before / after the window and never the window or anchors).
// The readout adds g (.) ((S_fwd + S_bwd) q) to the softmax output.
#include "common.h"
#include "kernels.h"

namespace vdn {

// ============================================================ Grams (fp32 path)
// grid (F, H), 256 threads; G = K^T K and B = V^T K over the frame's tokens
// (K, V: N x D token-major), frames 1..F-2 only.
template <int D>
__global__ __launch_bounds__(256) void gram_f32_kernel(const float* __restrict__ k,
                                                       const float* __restrict__ v, int F, int N,
                                                       int H, float* __restrict__ G,
                                                       float* __restrict__ B) {
  const int f = blockIdx.x, h = blockIdx.y;
  if (f == 0 || f == F - 1) return;
  constexpr int TN = 16;
  constexpr int PER = 4;                          // entries per thread per pass
  __shared__ float Ks[TN][D], Vs[TN][D];
  const size_t rs = (size_t)H * D;
  const size_t base = ((size_t)f * H + h) * D * D;
  for (int e0 = 0; e0 < D * D; e0 += 256 * PER) {
    float g[PER], bb[PER];
#pragma unroll
    for (int x = 0; x < PER; ++x) g[x] = bb[x] = 0.f;
    for (int n0 = 0; n0 < N; n0 += TN) {
      __syncthreads();
      for (int c = threadIdx.x; c < TN * D; c += 256) {
        const int n = c / D, ch = c % D;
        const bool ok = n0 + n < N;
        const size_t off = ((size_t)f * N + n0 + n) * rs + (size_t)h * D + ch;
        Ks[n][ch] = ok ? k[off] : 0.f;
        Vs[n][ch] = ok ? v[off] : 0.f;
      }
      __syncthreads();
#pragma unroll
      for (int x = 0; x < PER; ++x) {
        const int e = e0 + threadIdx.x + 256 * x;
        if (e < D * D) {
          const int r = e / D, c = e % D;
          for (int n = 0; n < TN; ++n) {
            g[x] += Ks[n][r] * Ks[n][c];
            bb[x] += Vs[n][r] * Ks[n][c];
          }
        }
      }
    }
#pragma unroll
    for (int x = 0; x < PER; ++x) {
      const int e = e0 + threadIdx.x + 256 * x;
      if (e < D * D) {
        G[base + e] = g[x];
        B[base + e] = bb[x];
      }
    }
  }
}

// ============================================================ per-frame affine maps
// grid (F-2, H), 512 threads (8 waves; two workgroups per CU); frame t =
// blockIdx.x + 1.
// In:  G = K K^T, B = V K^T of frame t.   Out (in place): G <- M = A^-1,
// B <- C = beta B M, with A = I + beta G.
// The matrix lives in LDS (fp32, pitch D + 1) in 32 x 32 blocks, NB = D / 32 per side.
//   1. Blocked Cholesky A = L L^T, right-looking, with T_k = L_kk^-1 in place of the
//      diagonal block: for k = 0 .. NB-1,
//        - one wave turns the diagonal block A_kk into T_k (a column step at a time,
//          32 steps, no workgroup barrier; L_kk itself is never needed);
//        - L_ik = A_ik T_k^T for i > k (in place), and U_kj = T_k L_kj for j < k (in
//          place of L_kj, which no later step reads);
//        - A_ij -= L_ik L_jk^T for NB > i >= j > k.
//   2. Y = L^-1 by blocks: Y_kk = T_k, Y_ik = -sum_{j=k}^{i-1} U_ij Y_jk (i > k), in
//      order of i - k; Y_ik is stored transposed in the free upper block (k, i).
//   3. M = Y^T Y, block (a, b) = sum over R >= max(a, b) of Y_Ra^T Y_Rb; M goes to G
//      and, in LDS, over A.
//   4. C = beta B M with B read from global memory and M from LDS.
// Every block product is 16 fp32 MFMAs (32x32x2); a wave owns whole blocks.
constexpr int FACTOR_THREADS = 512;
constexpr int FACTOR_NW = FACTOR_THREADS / 64;

// acc += X Z over a 32-deep reduction, X[r][m] = xp[r * xr + m * xm], Z[m][c] =
// zp[m * zm + c * zc] (lane j: row / column j, half hf: odd or even m)
__device__ inline floatx16 block_mma(floatx16 acc, const float* xp, int xr, int xm, const float* zp, int zm, int zc,
                                     int j, int hf) {
#pragma unroll
  for (int s = 0; s < 16; ++s) {
    const int m = 2 * s + hf;
    acc = mfma_f32(xp[j * xr + m * xm], zp[m * zm + j * zc], acc);
  }
  return acc;
}
// element r of a 32 x 32 accumulator is row 8 (r / 4) + 4 hf + r % 4, column j
__device__ inline int acc_row(int r, int hf) { return 8 * (r >> 2) + 4 * hf + (r & 3); }

// Lanes of one wave exchanging values through LDS: the stores before this point
// are visible to every lane's loads after it (LDS serves a wave's instructions in
// order; the fences keep the compiler from moving or forwarding the accesses
// across it, which per-lane program order alone would allow).
__device__ inline void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
}

// One wave: the 32 x 32 diagonal block at Ab (pitch LP; lower triangle read) is
// replaced by T = L^-1, L its Cholesky factor (zeros above the diagonal).  Lane
// (i, hh) holds row i, columns 16 hh .. 16 hh + 15 of the block and of T; step p
// broadcasts column p of the block and row p of T through cb / rb (in-order LDS
// within the wave).  As in a right-looking step with d = A_pp (after p steps):
// L_ip = A_ip / sqrt(d), so both rank-1 updates take the column times 1 / d, and
// row p of T is final once scaled by 1 / sqrt(d).
template <int LP>
__device__ inline void diag_inverse_factor(float* Ab, float* cb, float* rb, int lane) {
  const int i = lane & 31, hh = lane >> 5;
  float a[16], y[16];
#pragma unroll
  for (int x = 0; x < 16; ++x) {
    a[x] = Ab[i * LP + 16 * hh + x];
    y[x] = (16 * hh + x == i) ? 1.f : 0.f;
  }
#pragma unroll
  for (int p = 0; p < 32; ++p) {
    if (hh == (p >> 4)) cb[i] = a[p & 15];
    if (i == p) {
#pragma unroll
      for (int x = 0; x < 16; ++x) rb[16 * hh + x] = y[x];
    }
    wave_lds_sync();
    // the lane's 16 entries of the broadcast column and row, read together
    float cv[16], rv[16];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float4 c4 = *reinterpret_cast<const float4*>(cb + 16 * hh + 4 * q);
      const float4 r4 = *reinterpret_cast<const float4*>(rb + 16 * hh + 4 * q);
      cv[4 * q] = c4.x; cv[4 * q + 1] = c4.y; cv[4 * q + 2] = c4.z; cv[4 * q + 3] = c4.w;
      rv[4 * q] = r4.x; rv[4 * q + 1] = r4.y; rv[4 * q + 2] = r4.z; rv[4 * q + 3] = r4.w;
    }
    const float d = cb[p];                       // the pivot, >= 1 (A = I + beta G)
    const float inv_d = __builtin_amdgcn_rcpf(d);
    const float rsq = __builtin_amdgcn_rsqf(d);
    const float f = cb[i] * inv_d;
    if (i > p) {
#pragma unroll
      for (int x = 0; x < 16; ++x) {
        if (16 * hh + x > p) a[x] -= f * cv[x];
        y[x] -= f * rv[x];
      }
    } else if (i == p) {
#pragma unroll
      for (int x = 0; x < 16; ++x) y[x] *= rsq;
    }
    wave_lds_sync();   // every lane's reads of this step before the next step's stores
  }
#pragma unroll
  for (int x = 0; x < 16; ++x) Ab[i * LP + 16 * hh + x] = y[x];
}

template <int D>
__global__ __launch_bounds__(FACTOR_THREADS, 4)
void factor_kernel(float* __restrict__ G, float* __restrict__ Bm, const float* __restrict__ beta, int F, int H) {
  constexpr int NB = D / 32;
  constexpr int LP = D + 1;
  constexpr int NW = FACTOR_NW;
  constexpr int NBLK = NB * NB;
  constexpr int PER_WAVE = (NBLK + NW - 1) / NW;
  extern __shared__ float sm[];
  float* As = sm;                 // [D][LP]: A, then L / U and T_k, then Y; then M
  float* cb = As + D * LP;        // [32] column broadcast of the diagonal steps
  float* rb = cb + 32;            // [32] row broadcast
  auto blk = [&](int r, int c) { return As + 32 * r * LP + 32 * c; };

  const int t = blockIdx.x + 1, h = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int j = lane & 31, hf = lane >> 5;
  const float b = beta[(size_t)t * H + h];
  float* Gp = G + ((size_t)t * H + h) * D * D;
  float* Bp = Bm + ((size_t)t * H + h) * D * D;

  for (int e = tid; e < D * D; e += FACTOR_THREADS) {
    const int r = e / D, c = e - r * D;
    As[r * LP + c] = b * Gp[e] + (r == c ? 1.f : 0.f);
  }
  __syncthreads();

  // ---- 1. blocked Cholesky, T_k in the diagonal blocks
  for (int k = 0; k < NB; ++k) {
    if (w == 0) diag_inverse_factor<LP>(blk(k, k), cb, rb, lane);
    __syncthreads();
    // tasks 0 .. k-1: U_kj = T_k L_kj; tasks k .. NB-2: L_ik = A_ik T_k^T, i = task + 1
    for (int task = w; task < NB - 1; task += NW) {
      floatx16 acc = floatx16{};
      float* out;
      if (task < k) {
        out = blk(k, task);
        acc = block_mma(acc, blk(k, k), LP, 1, out, LP, 1, j, hf);
      } else {
        out = blk(task + 1, k);
        acc = block_mma(acc, out, LP, 1, blk(k, k), 1, LP, j, hf);
      }
      // (the wave's own reads of `out` are complete: every MFMA above consumed them)
#pragma unroll
      for (int r = 0; r < 16; ++r) out[acc_row(r, hf) * LP + j] = acc[r];
    }
    __syncthreads();
    // A_ij -= L_ik L_jk^T, NB > i >= j > k; task = pair index in row-major order
    const int m = NB - 1 - k;
    for (int task = w; task < m * (m + 1) / 2; task += NW) {
      int i = 0;
      while ((i + 1) * (i + 2) / 2 <= task) ++i;
      const int jj = task - i * (i + 1) / 2;
      float* out = blk(k + 1 + i, k + 1 + jj);
      floatx16 acc = floatx16{};
      acc = block_mma(acc, blk(k + 1 + i, k), LP, 1, blk(k + 1 + jj, k), 1, LP, j, hf);
#pragma unroll
      for (int r = 0; r < 16; ++r) out[acc_row(r, hf) * LP + j] -= acc[r];
    }
    __syncthreads();
  }

  // ---- 2. Y = L^-1: Y_ik (i = k + dl) = -sum_{jj=k}^{i-1} U_i,jj Y_jj,k, stored
  // transposed in block (k, i); Y_kk = T_k sits in the diagonal block as [row][col]
  for (int dl = 1; dl < NB; ++dl) {
    for (int k = w; k < NB - dl; k += NW) {
      const int i = k + dl;
      floatx16 acc = floatx16{};
      acc = block_mma(acc, blk(i, k), LP, 1, blk(k, k), LP, 1, j, hf);
      for (int jj = k + 1; jj < i; ++jj) acc = block_mma(acc, blk(i, jj), LP, 1, blk(k, jj), 1, LP, j, hf);
      float* out = blk(k, i);
#pragma unroll
      for (int r = 0; r < 16; ++r) out[j * LP + acc_row(r, hf)] = -acc[r];
    }
    __syncthreads();
  }

  // ---- 3. M = Y^T Y: block (ba, bb) = sum_{R >= max(ba, bb)} Y_R,ba^T Y_R,bb, where
  // Y_R,c[r][x] is blk(c, c)[r][x] for R = c and blk(c, R)[x][r] for R > c
  floatx16 macc[PER_WAVE];
#pragma unroll
  for (int x = 0; x < PER_WAVE; ++x) {
    macc[x] = floatx16{};
    const int bk = w * PER_WAVE + x;
    if (bk < NBLK) {
      const int ba = bk / NB, bb = bk % NB;
      for (int R = ba > bb ? ba : bb; R < NB; ++R) {
        const float* xa = R == ba ? blk(ba, ba) : blk(ba, R);
        const int xr = R == ba ? 1 : LP, xm = R == ba ? LP : 1;
        const float* zb = R == bb ? blk(bb, bb) : blk(bb, R);
        const int zm = R == bb ? LP : 1, zc = R == bb ? 1 : LP;
        macc[x] = block_mma(macc[x], xa, xr, xm, zb, zm, zc, j, hf);
      }
    }
  }
  __syncthreads();   // every read of Y done
#pragma unroll
  for (int x = 0; x < PER_WAVE; ++x) {
    const int bk = w * PER_WAVE + x;
    if (bk < NBLK) {
      const int ba = bk / NB, bb = bk % NB;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = 32 * ba + acc_row(r, hf);
        As[row * LP + 32 * bb + j] = macc[x][r];
        Gp[row * D + 32 * bb + j] = macc[x][r];
      }
    }
  }
  __syncthreads();

  // ---- 4. C = beta B M  (C[a][b] = beta sum_k B[a][k] M[k][b]).  Lane (j, hf)
  // reads 16 bytes of row j of B at a time, k = 8 u + 4 hf .. + 3, and MFMA 4 u + e
  // takes k = 8 u + 4 hf + e on both operands (the reduction in another order).
  floatx16 acc[PER_WAVE];
#pragma unroll
  for (int x = 0; x < PER_WAVE; ++x) {
    const int bk = w * PER_WAVE + x;
    acc[x] = floatx16{};
    if (bk < NBLK) {
      const int ba = bk / NB, bb = bk % NB;
      const float* brow = Bp + (size_t)(32 * ba + j) * D + 4 * hf;
      for (int u = 0; u < D / 8; ++u) {
        const float4 a4 = *reinterpret_cast<const float4*>(brow + 8 * u);
        const float* mcol = As + (8 * u + 4 * hf) * LP + 32 * bb + j;
        acc[x] = mfma_f32(a4.x, mcol[0], acc[x]);
        acc[x] = mfma_f32(a4.y, mcol[LP], acc[x]);
        acc[x] = mfma_f32(a4.z, mcol[2 * LP], acc[x]);
        acc[x] = mfma_f32(a4.w, mcol[3 * LP], acc[x]);
      }
    }
  }
  __syncthreads();   // every read of B done before C overwrites it
#pragma unroll
  for (int x = 0; x < PER_WAVE; ++x) {
    const int bk = w * PER_WAVE + x;
    if (bk < NBLK) {
      const int ba = bk / NB, bb = bk % NB;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = 32 * ba + acc_row(r, hf);
        Bp[row * D + 32 * bb + j] = b * acc[x][r];
      }
    }
  }
}

// ============================================================ serial scan
// grid (D/32 row blocks, 2 directions, H), D/32 waves.  Each workgroup carries
// 32 rows of the state through every frame of its direction: the rows of
// S <- S M + C evolve independently.  Wave w computes output columns
// [32w, 32w+32) as S_new^T = M S^T + C^T with fp32 MFMA (M is symmetric); its A
// operand is rows 32w.. of M_t, which the wave reads from global memory into
// registers one step ahead (no shared copy of M); the state goes between waves
// through LDS in the MFMA's own output layout, double-buffered, one barrier per
// step.
template <int D>
__global__ __launch_bounds__(2 * D) void scan_kernel(const float* __restrict__ Mg,
                                                     const float* __restrict__ Cg, int F, int H,
                                                     float* __restrict__ Sf, float* __restrict__ Sb) {
  constexpr int NW = D / 32;
  constexpr int NA = NW * 4;                // float4 pieces of this lane's A operand per step
  __shared__ float Sx[2][NW * 16 * 64];

  const int rb = blockIdx.x, dir = blockIdx.y, h = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, j = lane & 31, hf = lane >> 5;
  const int C = num_chunks(F);
  const int row = 32 * rb + j;
  float* Sout = dir == 0 ? Sf : Sb;

  auto snap = [&](int c, const floatx16& s) {
    float* dst = Sout + (((size_t)c * H + h) * D + row) * D + 32 * w + 4 * hf;
#pragma unroll
    for (int g = 0; g < 4; ++g)
      *reinterpret_cast<float4*>(dst + 8 * g) = make_float4(s[4 * g], s[4 * g + 1], s[4 * g + 2], s[4 * g + 3]);
  };
  // A chunk's state is zero when its set of frames is empty, and also when the
  // chunk holds no non-anchor frame (the last chunk when F = 5m + 1): no query
  // reads such a state.
  auto live = [&](int c) { return nq_end(c, F) > nq_first(c); };
  const floatx16 zero = floatx16{};
  for (int c = 0; c < C; ++c) {
    const bool empty = dir == 0 ? (c <= 1) : (5 * c + 10 > F - 2);
    if (empty || !live(c)) snap(c, zero);
  }
  int t0, nsteps, tstep;
  if (dir == 0) {
    t0 = 1;
    nsteps = 5 * (C - 1) - 6;          // frames 1 .. 5(C-1)-6
    tstep = 1;
  } else {
    t0 = F - 2;
    nsteps = F - 2 - 10 + 1;           // frames F-2 down to 10
    tstep = -1;
  }
  if (nsteps <= 0) return;

  for (int x = threadIdx.x; x < NW * 16 * 64; x += 2 * D) Sx[0][x] = 0.f;
  // lane (j, hf) of wave w feeds M[32w + j][32 wb + 8 g + 4 hf .. +3] for k-slots
  // s = 16 wb + 4 g + 0..3 of the MFMA chain
  float4 ma[NA], mn[NA];
  auto load_m = [&](int t, float4* dst) {
    const float* src = Mg + (((size_t)t * H + h) * D + 32 * w + j) * D + 4 * hf;
#pragma unroll
    for (int x = 0; x < NA; ++x) dst[x] = *reinterpret_cast<const float4*>(src + 32 * (x >> 2) + 8 * (x & 3));
  };
  // C_t entries of this lane's outputs initialise the accumulator; like M_t they
  // are loaded one step ahead
  float4 creg[4];
  auto load_c = [&](int t) {
    const float* cp = Cg + (((size_t)t * H + h) * D + row) * D + 32 * w + 4 * hf;
#pragma unroll
    for (int g = 0; g < 4; ++g) creg[g] = *reinterpret_cast<const float4*>(cp + 8 * g);
  };
  load_m(t0, mn);
  load_c(t0);
  __syncthreads();
  floatx16 acc = floatx16{};
  for (int step = 0; step < nsteps; ++step) {
    const int t = t0 + tstep * step, cur = step & 1;
#pragma unroll
    for (int x = 0; x < NA; ++x) ma[x] = mn[x];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      acc[4 * g + 0] = creg[g].x;
      acc[4 * g + 1] = creg[g].y;
      acc[4 * g + 2] = creg[g].z;
      acc[4 * g + 3] = creg[g].w;
    }
    if (step + 1 < nsteps) {
      load_m(t + tstep, mn);
      load_c(t + tstep);
    }
    const float* sx = Sx[cur];
#pragma unroll
    for (int s = 0; s < D / 2; ++s) {
      const int wb = s >> 4, e = s & 15;
      const float4 m4 = ma[4 * wb + (e >> 2)];
      const float av = (e & 3) == 0 ? m4.x : (e & 3) == 1 ? m4.y : (e & 3) == 2 ? m4.z : m4.w;
      acc = mfma_f32(av, sx[(wb * 16 + e) * 64 + lane], acc);
    }
    float* sxn = Sx[cur ^ 1];
#pragma unroll
    for (int e = 0; e < 16; ++e) sxn[(w * 16 + e) * 64 + lane] = acc[e];
    __syncthreads();     // the new state is visible; every read of the old buffer is done
    if (dir == 0) {
      if (t % 5 == 4) {
        const int c = (t + 6) / 5;
        if (c <= C - 1 && live(c)) snap(c, acc);
      }
    } else {
      if (t % 5 == 0 && t >= 10 && live((t - 10) / 5)) snap((t - 10) / 5, acc);
    }
  }
}

// ============================================================ readout weights
// W[c][h] = diag(g_h) (S_fwd[c][h] + S_bwd[c][h]) (g = 1 when gate is null),
// rounded to bf16 for the bf16 MFMA readout (relative error <= 2^-9 per entry);
// fp32 path: fp32.
__global__ void wprep_kernel(const float* __restrict__ Sf, const float* __restrict__ Sb,
                             const float* __restrict__ gate, int C, int H, int D, int bf16,
                             void* __restrict__ W) {
  const size_t n = (size_t)C * H * D * D;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) {
    const int dv = (i / D) % D;
    const int h = (i / ((size_t)D * D)) % H;
    const float g = gate ? gate[(size_t)h * D + dv] : 1.f;
    const float x = g * (Sf[i] + Sb[i]);
    if (bf16) static_cast<uint16_t*>(W)[i] = f32_to_bf16_bits(x);
    else static_cast<float*>(W)[i] = x;
  }
}

// ============================================================ readout (bf16)
// grid (RX, C, H), 256 threads.  Tiles of 64 tokens of chunk c's non-anchor
// frames, the RX workgroups of a (chunk, head) striding over them.
// O_lin^T = W q^T with W (its bf16 part) in LDS and q as the MFMA B operand; wave
// w takes tokens 32*(w & 1) .. +32 of the tile and output rows (value dims)
// 64*(w >> 1) .. +64.  ACC: O += O_lin, else O = O_lin.
//
// Global memory is touched only by whole-row accesses: the q and O tiles come in
// by 16-byte direct loads to LDS (lane L of a load takes 16 bytes of row L/RPL),
// and the result goes out from LDS by 16-byte stores in the same pattern.  A
// per-lane layout that follows the MFMA operands instead spreads every 64-lane
// access over 32 rows, which leaves the address unit, not HBM, as the limit.
// Tile rows are 2*D bytes; 16-byte chunks are XOR-swizzled per row (swz_rows) so
// the MFMA-order reads and writes of 16 consecutive rows hit distinct banks.
template <int D>
struct ReadoutCfg {
  static constexpr int TT = 64;                 // tokens per tile
  static constexpr int RB = 2 * D;              // bytes per token row
  static constexpr int RPL = RB / 16;           // 16-byte pieces per row
  static constexpr int RPI = 1024 / RB;         // rows per 1 KiB direct load
  static constexpr int LOADS = TT / RPI;        // direct loads per tile (q or O)
  static constexpr int P = D + 8;               // W row pitch in LDS (elements)
  static constexpr int NAB = D / 64 > 0 ? D / 64 : 1;   // 32-row output blocks per wave
  static constexpr int NWR = D / (32 * NAB);    // waves along the output rows
  static_assert(NWR * 2 <= 4, "4 waves cover 2 token halves x the output rows");
  static constexpr int TILE_BYTES = TT * RB;
};

template <int D, bool ACC>
__global__ __launch_bounds__(256, 2) void readout_kernel(const uint16_t* __restrict__ q,
                                                      const uint16_t* __restrict__ Wb, int F,
                                                      int N, int H, uint16_t* __restrict__ O) {
  using Cfg = ReadoutCfg<D>;
  constexpr int P = Cfg::P, RB = Cfg::RB, RPL = Cfg::RPL, RPI = Cfg::RPI, NAB = Cfg::NAB;
  __shared__ __attribute__((aligned(16))) uint16_t Ws[D * P];
  __shared__ __attribute__((aligned(16))) unsigned char qt[Cfg::TILE_BYTES];
  __shared__ __attribute__((aligned(16))) unsigned char ot[Cfg::TILE_BYTES];
  const int c = blockIdx.y, h = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, j = lane & 31, hf = lane >> 5;
  const int tok_begin = nq_first(c) * N, tok_end = nq_end(c, F) * N;
  if (tok_end <= tok_begin) return;
  {
    const uint16_t* src = Wb + ((size_t)c * H + h) * D * D;
    for (int x = tid; x < D * D / 8; x += 256) {
      const int r = (8 * x) / D, col = (8 * x) % D;
      *reinterpret_cast<uint4*>(&Ws[r * P + col]) = *reinterpret_cast<const uint4*>(src + 8 * x);
    }
  }
  const size_t rs = (size_t)H * D;                 // token stride (elements)
  const int ntile = (tok_end - tok_begin + Cfg::TT - 1) / Cfg::TT;
  const int tr = 32 * (w & 1);                     // this wave's first token row in the tile
  const int ab0 = NAB * (w >> 1);                  // this wave's first 32-row output block
  // direct-load lane pattern: row L / RPL of the 1 KiB block, logical chunk (L % RPL) ^ swz
  const int lrow = lane / RPL, lpos = lane % RPL;

  for (int tile = blockIdx.x; tile < ntile; tile += gridDim.x) {
    const int t0 = tok_begin + tile * Cfg::TT;
    // ---- q and O rows of the tile -> LDS (rows past the chunk repeat its last row);
    // the buffer base (wave-uniform) is the tile's first row, lanes add row offsets
    const size_t base = ((size_t)t0 * rs + (size_t)h * D) * 2;
    const uint32_t span = (uint32_t)(Cfg::TT * rs * 2);
    const __amdgpu_buffer_rsrc_t qrs = make_rsrc(reinterpret_cast<const unsigned char*>(q) + base, span);
    const __amdgpu_buffer_rsrc_t ors = make_rsrc(reinterpret_cast<const unsigned char*>(O) + base, span);
    for (int i = w; i < Cfg::LOADS; i += 4) {
      const int r = RPI * i + lrow;
      const int tok = min(t0 + r, tok_end - 1);
      const uint32_t off = (uint32_t)((tok - t0) * rs * 2) + 16u * (lpos ^ swz_rows(r, RB));
      __builtin_amdgcn_raw_ptr_buffer_load_lds(qrs, (lds_void_ptr)(qt + 1024 * i), 16, off, 0, 0, 0);
      if (ACC) __builtin_amdgcn_raw_ptr_buffer_load_lds(ors, (lds_void_ptr)(ot + 1024 * i), 16, off, 0, 0, 0);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();     // tile (and, on the first pass, W) in LDS

    // ---- O_lin^T for this wave's 32 tokens x 32*NAB output rows (d = 32: two waves)
    if ((w >> 1) < Cfg::NWR) {
    floatx16 acc[NAB];
#pragma unroll
    for (int x = 0; x < NAB; ++x) acc[x] = floatx16{};
    const int r = tr + j;
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      const bf16x8 qb = *reinterpret_cast<const bf16x8*>(qt + r * RB + 16 * ((2 * s + hf) ^ swz_rows(r, RB)));
#pragma unroll
      for (int x = 0; x < NAB; ++x) {
        const bf16x8 wa = *reinterpret_cast<const bf16x8*>(&Ws[(32 * (ab0 + x) + j) * P + 16 * s + 8 * hf]);
        acc[x] = mfma_bf16(wa, qb, acc[x]);
      }
    }
    // ---- O tile in LDS <- O (+) O_lin: accumulator element 4g + i of block ab is
    // output row 32*ab + 8g + 4*hf + i, i.e. bytes 8*hf.. of chunk 4*ab + g
#pragma unroll
    for (int x = 0; x < NAB; ++x)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        unsigned char* cell = ot + r * RB + 16 * ((4 * (ab0 + x) + g) ^ swz_rows(r, RB)) + 8 * hf;
        float x0 = acc[x][4 * g], x1 = acc[x][4 * g + 1], x2 = acc[x][4 * g + 2], x3 = acc[x][4 * g + 3];
        if (ACC) {
          const uint2 old = *reinterpret_cast<const uint2*>(cell);
          x0 += __uint_as_float(old.x << 16);
          x1 += __uint_as_float(old.x & 0xffff0000u);
          x2 += __uint_as_float(old.y << 16);
          x3 += __uint_as_float(old.y & 0xffff0000u);
        }
        *reinterpret_cast<uint2*>(cell) = make_uint2(pack_bf16x2(x0, x1), pack_bf16x2(x2, x3));
      }
    }
    __syncthreads();     // O tile complete

    // ---- O tile -> global, whole rows
    for (int i = w; i < Cfg::LOADS; i += 4) {
      const int rr = RPI * i + lrow;
      const int tok = t0 + rr;
      if (tok < tok_end) {
        const uint4 vv = *reinterpret_cast<const uint4*>(ot + 1024 * i + 16 * lane);   // row rr, position lpos
        const int chunk = lpos ^ swz_rows(rr, RB);
        *reinterpret_cast<uint4*>(O + (size_t)tok * rs + (size_t)h * D + 8 * chunk) = vv;
      }
    }
    __syncthreads();     // tile buffers free for the next tile
  }
}

// ============================================================ readout (fp32)
// One thread per output element of a non-anchor frame.
template <bool ACC>
__global__ void readout_f32_kernel(const float* __restrict__ q, const float* __restrict__ W, int F,
                                   int N, int H, int D, float* __restrict__ O) {
  const size_t total = (size_t)F * N * H * D;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += (size_t)gridDim.x * blockDim.x) {
    const int dv = i % D;
    const int h = (i / D) % H;
    const size_t tok = i / ((size_t)H * D);
    const int f = static_cast<int>(tok / N);
    if (f == 0 || f == F - 1) continue;
    const int c = f / kChunk;
    const float* wr = W + (((size_t)c * H + h) * D + dv) * D;
    const float* qr = q + tok * H * D + (size_t)h * D;
    float s = 0.f;
    for (int kk = 0; kk < D; ++kk) s += wr[kk] * qr[kk];
    O[i] = ACC ? O[i] + s : s;
  }
}

__global__ void fill_zero_kernel(uint32_t* p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) p[i] = 0u;
}

// ============================================================ launchers
hipError_t launch_gram_f32(const float* k, const float* v, int F, int N, int H, int D, float* G,
                           float* B, hipStream_t st) {
  const dim3 grid(F, H);
  switch (D) {
    case 32: hipLaunchKernelGGL(gram_f32_kernel<32>, grid, dim3(256), 0, st, k, v, F, N, H, G, B); break;
    case 64: hipLaunchKernelGGL(gram_f32_kernel<64>, grid, dim3(256), 0, st, k, v, F, N, H, G, B); break;
    case 128: hipLaunchKernelGGL(gram_f32_kernel<128>, grid, dim3(256), 0, st, k, v, F, N, H, G, B); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int D>
static hipError_t factor_d(float* G, float* B, const float* beta, int F, int H, hipStream_t st) {
  const size_t lds = ((size_t)D * (D + 1) + 64) * sizeof(float);
  static std::atomic<unsigned long long> attr_done{0};
  hipError_t e = set_max_lds_once(reinterpret_cast<const void*>(&factor_kernel<D>), (int)lds, &attr_done);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(factor_kernel<D>, dim3(F - 2, H), dim3(FACTOR_THREADS), lds, st, G, B, beta, F, H);
  return hipGetLastError();
}

hipError_t launch_factor(float* G, float* B, const float* beta, int F, int H, int D, hipStream_t st) {
  if (F < 3) return hipSuccess;
  switch (D) {
    case 32: return factor_d<32>(G, B, beta, F, H, st);
    case 64: return factor_d<64>(G, B, beta, F, H, st);
    case 128: return factor_d<128>(G, B, beta, F, H, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_scan(const float* M, const float* Cm, int F, int H, int D, float* Sf, float* Sb,
                       hipStream_t st) {
  const dim3 grid(D / 32, 2, H);
  switch (D) {
    case 32: hipLaunchKernelGGL(scan_kernel<32>, grid, dim3(64), 0, st, M, Cm, F, H, Sf, Sb); break;
    case 64: hipLaunchKernelGGL(scan_kernel<64>, grid, dim3(128), 0, st, M, Cm, F, H, Sf, Sb); break;
    case 128: hipLaunchKernelGGL(scan_kernel<128>, grid, dim3(256), 0, st, M, Cm, F, H, Sf, Sb); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_wprep(const float* Sf, const float* Sb, const float* gate, int C, int H, int D,
                        int bf16, void* W, hipStream_t st) {
  const size_t n = (size_t)C * H * D * D;
  const unsigned blocks = (unsigned)((n + 255) / 256 < 8192 ? (n + 255) / 256 : 8192);
  hipLaunchKernelGGL(wprep_kernel, dim3(blocks), dim3(256), 0, st, Sf, Sb, gate, C, H, D, bf16, W);
  return hipGetLastError();
}

hipError_t launch_readout(int prec, const void* q, const void* W, int F, int N, int H, int D,
                          void* O, int accumulate, hipStream_t st) {
  const int C = num_chunks(F);
  if (prec == 0) {
    const size_t total = (size_t)F * N * H * D;
    const unsigned blocks = (unsigned)((total + 255) / 256 < 65536 ? (total + 255) / 256 : 65536);
    if (accumulate)
      hipLaunchKernelGGL(readout_f32_kernel<true>, dim3(blocks), dim3(256), 0, st,
                         static_cast<const float*>(q), static_cast<const float*>(W), F, N, H, D, static_cast<float*>(O));
    else
      hipLaunchKernelGGL(readout_f32_kernel<false>, dim3(blocks), dim3(256), 0, st,
                         static_cast<const float*>(q), static_cast<const float*>(W), F, N, H, D, static_cast<float*>(O));
    return hipGetLastError();
  }
  const int max_tiles = (kChunk * N + 127) / 128;
  const int rx = max_tiles < 16 ? max_tiles : 16;
  const dim3 grid(rx, C, H);
  const uint16_t* qq = static_cast<const uint16_t*>(q);
  const uint16_t* ww = static_cast<const uint16_t*>(W);
  uint16_t* oo = static_cast<uint16_t*>(O);
#define VDN_RO(DD)                                                                                        \
  if (D == DD) {                                                                                          \
    if (accumulate)                                                                                       \
      hipLaunchKernelGGL((readout_kernel<DD, true>), grid, dim3(256), 0, st, qq, ww, F, N, H, oo);        \
    else                                                                                                  \
      hipLaunchKernelGGL((readout_kernel<DD, false>), grid, dim3(256), 0, st, qq, ww, F, N, H, oo);       \
    return hipGetLastError();                                                                             \
  }
  VDN_RO(32) VDN_RO(64) VDN_RO(128)
#undef VDN_RO
  return hipErrorInvalidValue;
}

hipError_t launch_zero(void* p, size_t bytes, hipStream_t st) {
  const size_t n = bytes / 4;
  if (n == 0) return hipSuccess;
  const unsigned blocks = (unsigned)((n + 255) / 256 < 4096 ? (n + 255) / 256 : 4096);
  hipLaunchKernelGGL(fill_zero_kernel, dim3(blocks), dim3(256), 0, st, static_cast<uint32_t*>(p), n);
  return hipGetLastError();
}

}  // namespace vdn
