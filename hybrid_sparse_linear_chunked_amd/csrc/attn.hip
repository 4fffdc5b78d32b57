// Softmax branch of the VDN hybrid video-to-video attention layer (gfx950).
//
// What is computed (sd114.wiki article "VDN-Minimax-H3 ...", section
// 双向滑动窗口Softmax分支): five latent frames form a chunk; the tokens of a query
// frame of chunk c attend, with softmax(q.k / sqrt(d)), to every token of the
// frames of chunks c-1, c, c+1 and of the first and last frame; the first and
// last frame attend to every frame.  No causal mask.
//
// Kernels in this file
//   prep_kernel      one pass over k and v per (frame, head): writes v transposed
//                    into 64-key blocks (the P.V operand layout of attn_kernel) and,
//                    for non-anchor frames, the frame's Grams G = K K^T and
//                    B = V K^T in fp32 (the VDA branch's inputs) with bf16 MFMA.
//   attn_kernel      flash-style attention: a 128-query tile against the key
//                    frames of its chunk (or one slice of all frames for anchor
//                    query frames), K / V^T tiles double-buffered in LDS, online
//                    softmax in fp32 registers, 32x32 MFMA for Q.K^T and P.V
//                    (the fp32 layer).
//   attn_lds_kernel  the same for bf16 and fp8-q.k I/O with 256-query items from
//                    per-XCD queues, tiles moved global -> LDS by direct loads,
//                    and the linear readout + gated merge in its epilogue.
//   attn_pp_kernel   the full-fp8 path (q.k and P.V on E4M3 codes): two groups of
//                    waves that take turns on the matrix and vector units.
//   combine_kernel   log-sum-exp merge of the anchor rows' key slices.
//   amax / fp8_exp / quant   per-head E4M3 quantiser (power-of-two scales) of
//                    the fp8 Q.K^T variant.
#include <type_traits>

#include "attn_common.h"

namespace vdn {

// ============================================================ layouts
// v transposed ("vt"): bf16 [H][F][nb][D][64], nb = ceil(N / 64).  Block (h, f, b)
// holds the values of keys f*N + 64b + (0..63) (zero past the frame's end), one
// row of 64 keys per channel.  Inside each group of 16 keys the order is
//   position 16u + 8g + e  <->  key 16u + 8(e/4) + 4g + e%4   (g = 0, 1; e = 0..7),
// which is the key order in which a 32x32 MFMA output tile hands its scores to
// the next MFMA's B operand (see attn_kernel), so each lane's eight P.V operand
// values are 16 contiguous bytes.
__device__ inline int vt_pos_of_key(int n) {   // n in [0, 64)
  int u = n >> 4, r = n & 15;
  return 16 * u + 8 * ((r & 7) >> 2) + 4 * (r >> 3) + (r & 3);
}

// Four E4M3 ("FN": no infinities, max 448) codes, round to nearest even with
// subnormals, packed low byte first, by the hardware conversion.  Every caller's
// values are at most 448 in magnitude (their power-of-two scale is chosen so), and
// on that range the conversion equals the format's definition for every fp32
// input (checked on the device over all of them, both signs).
__device__ inline uint32_t e4m3x4(float x0, float x1, float x2, float x3) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(x0, x1, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(x2, x3, w, true);
  return static_cast<uint32_t>(w);
}

// v transposed as E4M3 codes ("vt8", fp8 P.V): bytes [H][F][nb][D][64], the same
// blocks and keys as vt, each row regrouped so that a lane half's 32 operand bytes
// are contiguous:
//   byte 32 hf + 8 u + e  <->  vt position 16 u + 8 hf + e   (hf = 0, 1; u = 0..3),
// i.e. lane half hf of a 64-deep P.V MFMA reads bytes 32 hf .. 32 hf + 31, the keys
// whose probabilities that lane half holds, in the same order.  code =
// E4M3(fp32(v * 2^-e_v)), e_v the head's power-of-two scale exponent.

// ============================================================ prep (bf16)
// grid (F, H), 512 threads.  LDS: K^T and V^T of one 64-token tile, keys permuted
// as in the vt layout (the Gram products only need both operands in the same
// token order).  With vt8 set, the V^T blocks go out as E4M3 codes in the vt8
// layout (scale exponents vexp [H]) instead of bf16 vt.
//
// The transpose happens in registers: a thread loads four token rows x 8
// channels (four 16-byte pieces, coalesced across the wave), regroups them into
// 8 channels x four tokens with 16-bit permutes, and writes 8-byte pieces to
// LDS.  The four tokens are the ones the vt permutation puts at consecutive
// positions, so the pieces land as whole runs of a V^T row.  The next tile's
// loads are in flight while this tile's V^T block is written out and its Gram
// MFMAs run.
template <int D>
__global__ __launch_bounds__(512) void prep_kernel(const uint16_t* __restrict__ k,
                                                   const uint16_t* __restrict__ v, int F, int N,
                                                   int H, uint16_t* __restrict__ vt,
                                                   float* __restrict__ G, float* __restrict__ B,
                                                   int do_grams, uint8_t* __restrict__ vt8,
                                                   const int* __restrict__ vexp) {
  constexpr int P = 64 + 8;                      // LDS row pitch (bf16)
  constexpr int NB = D / 32;                     // 32-channel blocks per side
  constexpr int NBLK = 2 * NB * NB;              // G blocks then B blocks
  constexpr int PER_WAVE = (NBLK + 7) / 8;
  constexpr int ACTIVE = 4 * D;                  // loading threads: 2 tensors x 8 key pieces x D/8 groups x 2 halves
  static_assert(ACTIVE <= 512, "one 4-token x 8-channel piece per loading thread");
  __shared__ __attribute__((aligned(16))) uint16_t KT[D * P];
  __shared__ __attribute__((aligned(16))) uint16_t VT[D * P];

  const int f = blockIdx.x, h = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int j = lane & 31, hf = lane >> 5;
  const int nb = (N + 63) / 64;
  const bool grams = do_grams && f > 0 && f < F - 1;
  const size_t rs = (size_t)H * D;               // token stride (elements)

  // this thread's piece: tensor, 8-position run pc of the permuted key order,
  // channel group cg, half th of the run (positions 8*pc + 4*th .. +4)
  const bool loader = tid < ACTIVE;
  const int isv = tid / (2 * D), rem = tid % (2 * D);
  const int pc = rem & 7, cg = (rem >> 3) % (D / 8), th = rem / D;
  const uint16_t* src = (isv ? v : k) + (size_t)f * N * rs + (size_t)h * D + 8 * cg;
  // key of position 8*pc + 4*th + e (inverse of vt_pos_of_key)
  const int key0 = 16 * (pc >> 1) + 4 * (pc & 1) + 8 * th;
  uint4 raw[4];
  auto load = [&](int b) {
    const int nvalid = min(64, N - 64 * b);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int n = key0 + e;
      raw[e] = (loader && n < nvalid) ? *reinterpret_cast<const uint4*>(src + (size_t)(64 * b + n) * rs)
                                      : make_uint4(0, 0, 0, 0);
    }
  };

  floatx16 acc[PER_WAVE];
#pragma unroll
  for (int x = 0; x < PER_WAVE; ++x) acc[x] = floatx16{};

  load(0);
  for (int b = 0; b < nb; ++b) {
    // ---- 4 tokens x 8 channels -> 8 channels x 4 tokens -> LDS
    if (loader) {
      uint16_t* T = isv ? VT : KT;
      const uint32_t r0[4] = {raw[0].x, raw[0].y, raw[0].z, raw[0].w};
      const uint32_t r1[4] = {raw[1].x, raw[1].y, raw[1].z, raw[1].w};
      const uint32_t r2[4] = {raw[2].x, raw[2].y, raw[2].z, raw[2].w};
      const uint32_t r3[4] = {raw[3].x, raw[3].y, raw[3].z, raw[3].w};
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        // channels 2m (low halves) and 2m+1 (high halves) of the four tokens
        const uint2 lo = make_uint2((r0[m] & 0xffffu) | (r1[m] << 16), (r2[m] & 0xffffu) | (r3[m] << 16));
        const uint2 hi = make_uint2((r0[m] >> 16) | (r1[m] & 0xffff0000u), (r2[m] >> 16) | (r3[m] & 0xffff0000u));
        *reinterpret_cast<uint2*>(&T[(8 * cg + 2 * m) * P + 8 * pc + 4 * th]) = lo;
        *reinterpret_cast<uint2*>(&T[(8 * cg + 2 * m + 1) * P + 8 * pc + 4 * th]) = hi;
      }
    }
    __syncthreads();
    if (b + 1 < nb) load(b + 1);
    // ---- V^T block out: D rows x 64 keys
    if (vt8 == nullptr) {
      uint16_t* dst = vt + (((size_t)h * F + f) * nb + b) * (size_t)(D * 64);
      for (int c = tid; c < D * 8; c += 512) {
        const int row = c >> 3, c8 = c & 7;
        *reinterpret_cast<uint4*>(dst + row * 64 + 8 * c8) =
            *reinterpret_cast<const uint4*>(&VT[row * P + 8 * c8]);
      }
    } else {
      // piece c: row, lane half hf, group u -> 8 codes at byte 32 hf + 8 u
      uint8_t* dst = vt8 + (((size_t)h * F + f) * nb + b) * (size_t)(D * 64);
      const int ne = -vexp[h];
      for (int c = tid; c < D * 8; c += 512) {
        const int row = c >> 3, hf8 = (c >> 2) & 1, u = c & 3;
        const uint4 x = *reinterpret_cast<const uint4*>(&VT[row * P + 16 * u + 8 * hf8]);
        const uint32_t wv[4] = {x.x, x.y, x.z, x.w};
        float y[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint32_t bits = (e & 1) ? (wv[e >> 1] & 0xffff0000u) : (wv[e >> 1] << 16);
          y[e] = __builtin_ldexpf(__uint_as_float(bits), ne);              // exact scaling
        }
        *reinterpret_cast<uint2*>(dst + row * 64 + 32 * hf8 + 8 * u) =
            make_uint2(e4m3x4(y[0], y[1], y[2], y[3]), e4m3x4(y[4], y[5], y[6], y[7]));
      }
    }
    if (grams) {
#pragma unroll
      for (int x = 0; x < PER_WAVE; ++x) {
        const int blk = w * PER_WAVE + x;
        if (blk < NBLK) {
          const bool isB = blk >= NB * NB;
          const int bb = isB ? blk - NB * NB : blk;
          const int bi = bb / NB, bj = bb % NB;
          const uint16_t* A = isB ? VT : KT;
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            bf16x8 a = *reinterpret_cast<const bf16x8*>(&A[(32 * bi + j) * P + 16 * u + 8 * hf]);
            bf16x8 bo = *reinterpret_cast<const bf16x8*>(&KT[(32 * bj + j) * P + 16 * u + 8 * hf]);
            acc[x] = mfma_bf16(a, bo, acc[x]);
          }
        }
      }
    }
    __syncthreads();
  }
  if (grams) {
#pragma unroll
    for (int x = 0; x < PER_WAVE; ++x) {
      const int blk = w * PER_WAVE + x;
      if (blk < NBLK) {
        const bool isB = blk >= NB * NB;
        const int bb = isB ? blk - NB * NB : blk;
        const int bi = bb / NB, bj = bb % NB;
        float* dst = (isB ? B : G) + ((size_t)f * H + h) * D * D;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = 32 * bi + 8 * (r >> 2) + 4 * hf + (r & 3);
          dst[row * D + 32 * bj + j] = acc[x][r];
        }
      }
    }
  }
}

template <int D, int PREC>
struct AttnCfg {
  static constexpr bool F32 = PREC == 0;
  static constexpr bool FP8 = PREC == 2;
  // K tile pitch in elements of the K operand type
  static constexpr int KP = F32 ? D + 1 : (FP8 ? D + 16 : D + 8);
  static constexpr int K_BYTES = F32 ? BK * KP * 4 : (FP8 ? BK * KP : BK * KP * 2);
  // V tile: fp32 path [64 keys][D+1] floats; otherwise V^T [D][64+8] bf16
  static constexpr int VP = F32 ? D + 1 : BK + 8;
  static constexpr int V_BYTES = F32 ? BK * VP * 4 : D * VP * 2;
  static constexpr int STAGE = ((K_BYTES + V_BYTES) + 15) / 16 * 16;
  // 16-byte chunks of one tile in global memory
  static constexpr int K_CHUNKS = F32 ? BK * D / 4 : (FP8 ? BK * D / 16 : BK * D / 8);
  static constexpr int V_CHUNKS = F32 ? BK * D / 4 : D * BK / 8;
  static constexpr int K_PER_T = (K_CHUNKS + 255) / 256;
  static constexpr int V_PER_T = (V_CHUNKS + 255) / 256;
  static constexpr int QSTEPS = F32 ? D / 2 : (FP8 ? D / 64 : D / 16);
};

template <int D, int PREC>
__global__ __launch_bounds__(256, 2) void attn_kernel(AttnArgs a) {
  using Cfg = AttnCfg<D, PREC>;
  constexpr bool F32 = Cfg::F32, FP8 = Cfg::FP8;
  constexpr int NDB = D / 32;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int j = lane & 31, hf = lane >> 5;
  const int F = a.F, N = a.N, H = a.H;
  const size_t rs = (size_t)H * D;
  const int nb = (N + BK - 1) / BK;

  // ---------------- decode the work item
  int h, q_tok0, q_rows, split = -1, anchor_idx = 0;
  int kf_mode;          // 0: contiguous frames [k_f0, k_f1); 1: chunk key list
  int k_f0 = 0, k_f1 = 0, wf = 0, we = 0, nslots;
  // The dispatcher deals workgroups round-robin over the 8 XCDs (each with its own
  // L2).  Renumber so that every XCD runs one contiguous range of work items:
  // consecutive items share their key frames, so concurrent workgroups on an XCD
  // stream the same K / V^T tiles through that XCD's L2.
  int bid;
  {
    const int G = gridDim.x, b = blockIdx.x;
    const int x = b & 7, i8 = b >> 3, q8 = G >> 3, r8 = G & 7;
    bid = (x < r8 ? x * (q8 + 1) : r8 * (q8 + 1) + (x - r8) * q8) + i8;
  }
  if (bid < a.n_anchor_items) {
    // anchor items: query tile fastest, then anchor frame, then key slice, then
    // head, so items reading the same key slice are adjacent
    int r = bid;
    const int qt = r % a.qt_anchor;
    r /= a.qt_anchor;
    anchor_idx = r % a.na;
    r /= a.na;
    split = r % a.nsplit;
    h = r / a.nsplit;
    const int qf = anchor_idx == 0 ? 0 : F - 1;
    q_tok0 = qf * N + qt * a.bq;
    q_rows = min(a.bq, N - qt * a.bq);
    kf_mode = 0;
    k_f0 = split * a.fs;
    k_f1 = min(F, k_f0 + a.fs);
    nslots = k_f1 - k_f0;
  } else {
    int r = bid - a.n_anchor_items;
    h = r / a.tiles_per_head;
    r -= h * a.tiles_per_head;
    const int C = num_chunks(F);
    int c = 0;
    for (; c < C; ++c) {
      const int nf = nq_end(c, F) - nq_first(c);
      const int t = nf > 0 ? (nf * N + a.bq - 1) / a.bq : 0;
      if (r < t) break;
      r -= t;
    }
    const int tok_begin = nq_first(c) * N, tok_end = nq_end(c, F) * N;
    q_tok0 = tok_begin + r * a.bq;
    q_rows = min(a.bq, tok_end - q_tok0);
    kf_mode = 1;
    wf = win_first(c);
    we = win_end(c, F);
    nslots = (wf > 0 ? 1 : 0) + (we - wf) + (we < F ? 1 : 0);
  }
  const int ntiles = nslots * nb;

  // ---------------- Q operand fragments (B operand of S^T = K Q^T), resident
  const int qi = 32 * w + j;                    // query row within the tile
  const bool qvalid = qi < q_rows;
  const size_t qoff = (size_t)(q_tok0 + qi) * rs + (size_t)h * D;
  bf16x8 qb[F32 || FP8 ? 1 : Cfg::QSTEPS];
  float qf[F32 ? Cfg::QSTEPS : 1];
  intx8 q8f[FP8 ? Cfg::QSTEPS : 1];
  if constexpr (F32) {
    const float* q = static_cast<const float*>(a.q);
#pragma unroll
    for (int s = 0; s < Cfg::QSTEPS; ++s) qf[s] = qvalid ? q[qoff + 2 * s + hf] : 0.f;
  } else if constexpr (FP8) {
#pragma unroll
    for (int s = 0; s < Cfg::QSTEPS; ++s) {
      if (qvalid) {
        const uint4* p = reinterpret_cast<const uint4*>(a.q8 + qoff + 64 * s + 32 * hf);
        uint4 x0 = p[0], x1 = p[1];
        q8f[s] = intx8{(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w, (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
      } else {
        q8f[s] = intx8{};
      }
    }
  } else {
    const uint16_t* q = static_cast<const uint16_t*>(a.q);
#pragma unroll
    for (int s = 0; s < Cfg::QSTEPS; ++s)
      qb[s] = qvalid ? *reinterpret_cast<const bf16x8*>(q + qoff + 16 * s + 8 * hf) : bf16x8{};
  }
  // fp8: the q codes carry the base-2 temperature, a score is 2^(e_q + e_k) times
  // the code products
  const float scale = FP8 ? __builtin_ldexpf(1.f, a.fexp[h] + a.fexp[H + h]) : a.scale_log2;

  // ---------------- tile loader
  auto tile_frame = [&](int t, int& f, int& b) {
    const int s = t / nb;
    b = t - s * nb;
    f = kf_mode == 0 ? k_f0 + s : chunk_key_frame(s, wf, we, F);
  };
  uint4 kreg[Cfg::K_PER_T];
  uint4 vreg[Cfg::V_PER_T];
  auto load_tile = [&](int t) {
    int f, b;
    tile_frame(t, f, b);
    const int nvalid = min(BK, N - BK * b);
    const size_t tok0 = (size_t)f * N + BK * b;
#pragma unroll
    for (int x = 0; x < Cfg::K_PER_T; ++x) {
      const int c = tid + 256 * x;
      kreg[x] = make_uint4(0, 0, 0, 0);
      if (c < Cfg::K_CHUNKS) {
        constexpr int CPR = Cfg::K_CHUNKS / BK;   // chunks per key row
        const int n = c / CPR, cc = c % CPR;
        if (n < nvalid) {
          if constexpr (F32)
            kreg[x] = *reinterpret_cast<const uint4*>(static_cast<const float*>(a.k) + (tok0 + n) * rs + (size_t)h * D + 4 * cc);
          else if constexpr (FP8)
            kreg[x] = *reinterpret_cast<const uint4*>(a.k8 + (tok0 + n) * rs + (size_t)h * D + 16 * cc);
          else
            kreg[x] = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.k) + (tok0 + n) * rs + (size_t)h * D + 8 * cc);
        }
      }
    }
#pragma unroll
    for (int x = 0; x < Cfg::V_PER_T; ++x) {
      const int c = tid + 256 * x;
      vreg[x] = make_uint4(0, 0, 0, 0);
      if (c < Cfg::V_CHUNKS) {
        if constexpr (F32) {
          constexpr int CPR = D / 4;
          const int n = c / CPR, cc = c % CPR;
          if (n < nvalid)
            vreg[x] = *reinterpret_cast<const uint4*>(static_cast<const float*>(a.v) + (tok0 + n) * rs + (size_t)h * D + 4 * cc);
        } else {
          const uint16_t* src = a.vt + (((size_t)h * F + f) * nb + b) * (size_t)(D * BK);
          vreg[x] = *reinterpret_cast<const uint4*>(src + 8 * c);
        }
      }
    }
  };
  auto store_tile = [&](int stage) {
    unsigned char* base = smem + stage * Cfg::STAGE;
#pragma unroll
    for (int x = 0; x < Cfg::K_PER_T; ++x) {
      const int c = tid + 256 * x;
      if (c < Cfg::K_CHUNKS) {
        constexpr int CPR = Cfg::K_CHUNKS / BK;
        const int n = c / CPR, cc = c % CPR;
        if constexpr (F32) {
          float* Ks = reinterpret_cast<float*>(base);
          Ks[n * Cfg::KP + 4 * cc + 0] = __uint_as_float(kreg[x].x);
          Ks[n * Cfg::KP + 4 * cc + 1] = __uint_as_float(kreg[x].y);
          Ks[n * Cfg::KP + 4 * cc + 2] = __uint_as_float(kreg[x].z);
          Ks[n * Cfg::KP + 4 * cc + 3] = __uint_as_float(kreg[x].w);
        } else if constexpr (FP8) {
          *reinterpret_cast<uint4*>(base + n * Cfg::KP + 16 * cc) = kreg[x];
        } else {
          *reinterpret_cast<uint4*>(base + 2 * (n * Cfg::KP + 8 * cc)) = kreg[x];
        }
      }
    }
    unsigned char* vb = base + Cfg::K_BYTES;
#pragma unroll
    for (int x = 0; x < Cfg::V_PER_T; ++x) {
      const int c = tid + 256 * x;
      if (c < Cfg::V_CHUNKS) {
        if constexpr (F32) {
          constexpr int CPR = D / 4;
          const int n = c / CPR, cc = c % CPR;
          float* Vs = reinterpret_cast<float*>(vb);
          Vs[n * Cfg::VP + 4 * cc + 0] = __uint_as_float(vreg[x].x);
          Vs[n * Cfg::VP + 4 * cc + 1] = __uint_as_float(vreg[x].y);
          Vs[n * Cfg::VP + 4 * cc + 2] = __uint_as_float(vreg[x].z);
          Vs[n * Cfg::VP + 4 * cc + 3] = __uint_as_float(vreg[x].w);
        } else {
          const int row = c >> 3, c8 = c & 7;
          *reinterpret_cast<uint4*>(vb + 2 * (row * Cfg::VP + 8 * c8)) = vreg[x];
        }
      }
    }
  };

  // ---------------- running softmax state (per lane: query j; both halves agree on m)
  floatx16 o[NDB];
#pragma unroll
  for (int x = 0; x < NDB; ++x) o[x] = floatx16{};
  float m_run = -INFINITY, l_run = 0.f;

  load_tile(0);
  store_tile(0);
  __syncthreads();

  for (int t = 0; t < ntiles; ++t) {
    const int stage = t & 1;
    if (t + 1 < ntiles) load_tile(t + 1);
    const unsigned char* base = smem + stage * Cfg::STAGE;
    int nvalid;
    {
      int f, b;
      tile_frame(t, f, b);
      nvalid = min(BK, N - BK * b);
    }

    // S^T = K Q^T for two 32-key blocks
    floatx16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s[kb] = floatx16{};
      const int krow = 32 * kb + j;
      if constexpr (F32) {
        const float* Ks = reinterpret_cast<const float*>(base);
#pragma unroll
        for (int st = 0; st < Cfg::QSTEPS; ++st)
          s[kb] = mfma_f32(Ks[krow * Cfg::KP + 2 * st + hf], qf[st], s[kb]);
      } else if constexpr (FP8) {
#pragma unroll
        for (int st = 0; st < Cfg::QSTEPS; ++st) {
          const uint4* p = reinterpret_cast<const uint4*>(base + krow * Cfg::KP + 64 * st + 32 * hf);
          uint4 x0 = p[0], x1 = p[1];
          intx8 ka = {(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w, (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
          s[kb] = mfma_fp8_scaled(ka, q8f[st], s[kb], 127, 127);   // (scales applied in the exponent)
        }
      } else {
        const uint16_t* Ks = reinterpret_cast<const uint16_t*>(base);
#pragma unroll
        for (int st = 0; st < Cfg::QSTEPS; ++st) {
          bf16x8 ka = *reinterpret_cast<const bf16x8*>(&Ks[krow * Cfg::KP + 16 * st + 8 * hf]);
          s[kb] = mfma_bf16(ka, qb[st], s[kb]);
        }
      }
    }
    // Online softmax in log2 units.  Scores are scaled inside the exp2 argument
    // (one FMA).  The running max m_run is raised only when a tile's max exceeds it
    // by more than kLazy (wave-uniform decision), so O and l are rescaled rarely;
    // in between, p = 2^(x - m_run) <= 2^kLazy, which bf16 P and fp32 sums hold
    // exactly as well as values <= 1.  The result O / l does not depend on m_run.
    if (nvalid < BK) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = 32 * kb + 8 * (r >> 2) + 4 * hf + (r & 3);
          if (key >= nvalid) s[kb][r] = -INFINITY;
        }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; r += 2) mx = fmaxf(mx, fmaxf(s[kb][r], s[kb][r + 1]));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float mt = mx * scale;
    if (__any(mt > m_run + kLazy)) {
      const float m_new = fmaxf(m_run, mt);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int x = 0; x < NDB; ++x) o[x] *= alpha;
    }
    const float neg_m = -m_run;
    float psum = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = __builtin_amdgcn_exp2f(fmaf(s[kb][r], scale, neg_m));
        s[kb][r] = p;
        psum += p;
      }
    l_run += psum;

    // O^T += V^T P^T
    if constexpr (F32) {
      const float* Vs = reinterpret_cast<const float*>(base + Cfg::K_BYTES);
#pragma unroll
      for (int u = 0; u < 32; ++u) {
        const int kb = u >> 4, r = u & 15;
        const int key = 32 * kb + 8 * (r >> 2) + 4 * hf + (r & 3);
#pragma unroll
        for (int db = 0; db < NDB; ++db)
          o[db] = mfma_f32(Vs[key * Cfg::VP + 32 * db + j], s[kb][r], o[db]);
      }
    } else {
      const uint16_t* Vs = reinterpret_cast<const uint16_t*>(base + Cfg::K_BYTES);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int kb = u >> 1, e0 = 8 * (u & 1);
        bf16x8 pb;
#pragma unroll
        for (int e = 0; e < 8; ++e) pb[e] = (__bf16)s[kb][e0 + e];
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          bf16x8 va = *reinterpret_cast<const bf16x8*>(&Vs[(32 * db + j) * Cfg::VP + 16 * u + 8 * hf]);
          o[db] = mfma_bf16(va, pb, o[db]);
        }
      }
    }

    if (t + 1 < ntiles) store_tile(stage ^ 1);
    __syncthreads();
  }

  // ---------------- epilogue
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  if (!qvalid) return;
  if (split < 0) {
    const float inv = 1.f / l_tot;
    const size_t ooff = (size_t)(q_tok0 + qi) * rs + (size_t)h * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int dd = 32 * db + 8 * g + 4 * hf;
        const float x0 = o[db][4 * g + 0] * inv, x1 = o[db][4 * g + 1] * inv;
        const float x2 = o[db][4 * g + 2] * inv, x3 = o[db][4 * g + 3] * inv;
        if constexpr (F32) {
          *reinterpret_cast<float4*>(static_cast<float*>(a.O) + ooff + dd) = make_float4(x0, x1, x2, x3);
        } else {
          uint2 pk = make_uint2(pack_bf16x2(x0, x1), pack_bf16x2(x2, x3));
          *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.O) + ooff + dd) = pk;
        }
      }
  } else {
    const int n = q_tok0 - (anchor_idx == 0 ? 0 : (F - 1) * N) + qi;
    const size_t row = (((size_t)split * H + h) * a.na + anchor_idx) * N + n;
    float* po = a.part_O + row * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int dd = 32 * db + 8 * g + 4 * hf;
        *reinterpret_cast<float4*>(po + dd) =
            make_float4(o[db][4 * g + 0], o[db][4 * g + 1], o[db][4 * g + 2], o[db][4 * g + 3]);
      }
    if (hf == 0) {
      a.part_ml[2 * row + 0] = m_run;
      a.part_ml[2 * row + 1] = l_tot;
    }
  }
}

// Work item when the layer has extra tokens.  Per head, per key split: the anchor
// frames' query tiles, then the extra tokens' query tiles (anchor_idx = na); then
// the chunk items as in decode_item.  The key list of a chunk item, and of the last
// split of a split item, ends with the extra tokens: their slot is returned in
// *xslot (-1 if none), after the it.nslots video frames.
__device__ inline Item decode_item_x(const AttnArgs& a, int* xslot) {
  Item it;
  const int F = a.F, N = a.N;
  const int G = a.na * a.qt_anchor + a.qt_x;             // split-item query tiles per split
  const int na_h = G * a.nsplit;                         // split items per head
  // dispatch order: the split items of every head first (15 or so key frames
  // each, dealt round-robin over the XCDs), then the chunk items (the extra
  // tokens' keys only: a few tiles each), so no long item starts last
  const int b = blockIdx.x, nsp = a.H * na_h;
  int hh, li;
  if (b < nsp) {
    hh = b / na_h;
    li = b - hh * na_h;
  } else {
    hh = (b - nsp) / a.tiles_per_head;
    li = na_h + (b - nsp) - hh * a.tiles_per_head;
  }
  it.wf = it.we = it.k_f0 = 0;
  it.h = hh;
  if (li < na_h) {
    it.split = li / G;
    const int g = li - it.split * G;
    if (g < a.na * a.qt_anchor) {
      it.anchor_idx = g / a.qt_anchor;
      const int qt = g - it.anchor_idx * a.qt_anchor;
      it.q_tok0 = (it.anchor_idx == 0 ? 0 : F - 1) * N + qt * a.bq;
      it.q_rows = min(a.bq, N - qt * a.bq);
    } else {
      it.anchor_idx = a.na;
      const int qt = g - a.na * a.qt_anchor;
      it.q_tok0 = F * N + qt * a.bq;
      it.q_rows = min(a.bq, a.T - qt * a.bq);
    }
    it.mode = 0;
    it.k_f0 = it.split * a.fs;
    it.nslots = min(F, it.k_f0 + a.fs) - it.k_f0;
    *xslot = it.split == a.nsplit - 1 ? it.nslots : -1;
  } else {
    int rr = li - na_h;
    it.split = -1;
    it.anchor_idx = 0;
    const int C = num_chunks(F);
    int c = 0;
    for (; c < C; ++c) {
      const int nf = nq_end(c, F) - nq_first(c);
      const int t = nf > 0 ? (nf * N + a.bq - 1) / a.bq : 0;
      if (rr < t) break;
      rr -= t;
    }
    const int tok_begin = nq_first(c) * N, tok_end = nq_end(c, F) * N;
    it.q_tok0 = tok_begin + rr * a.bq;
    it.q_rows = min(a.bq, tok_end - it.q_tok0);
    it.mode = 1;
    it.wf = win_first(c);
    it.we = win_end(c, F);
    it.nslots = 0;           // the extra tokens only: the video frames follow in a second pass
    *xslot = 0;
  }
  return it;
}


// XT: the layer has extra tokens; this instantiation runs the split items with
// them and, for chunk items, the extra tokens' keys alone, leaving the softmax
// state in px.  XI: the chunk items' video pass that starts from that state.
// SPLIT: chunk items write O_soft and g (.) O_lin side by side (token stride 2 H D,
// the output projection's input) instead of their sum.
template <int D, int PREC, int NW, bool XT, bool SPLIT, bool XI = false>
// (two waves per SIMD: d = 128 needs ~240 registers)
__global__ __launch_bounds__(64 * NW, 2) void attn_lds_kernel(AttnArgs a) {
  using Cfg = LdsCfg<D, PREC>;
  constexpr bool FP8 = Cfg::FP8;
  constexpr int NDB = D / 32;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];

  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int j = lane & 31, hf = lane >> 5;
  const int F = a.F, N = a.N, H = a.H;
  const size_t rs = (size_t)H * D;                 // token stride in elements
  const int nb = (N + BK - 1) / BK;
  // the item is wave-uniform; say so, so that tile bookkeeping stays in SGPRs
  int xs = -1;                 // with extra tokens: their slot in the key list
  Item it0;
  if constexpr (XT) {
    it0 = decode_item_x(a, &xs);
  } else if (a.qctr != nullptr) {
    // the item from the queues: one thread takes it, and the LDS word after the
    // tile stages hands it to the other waves
    int* slot = reinterpret_cast<int*>(smem + kLdsStages * Cfg::STAGE);
    if (tid == 0) *slot = acquire_item(a);
    __syncthreads();
    const int pk = __builtin_amdgcn_readfirstlane(*slot);
    if (pk < 0) return;      // every queue empty (the grid's spare workgroups)
    const int M = a.na * a.qt_anchor * a.nsplit + a.tiles_per_head;
    const int hh = pk / M;
    it0 = decode_item_at(a, hh, pk - hh * M);
  } else {
    it0 = decode_item(a);
  }
  const Item it = uniform_item(it0);
  const int xslot = XT ? __builtin_amdgcn_readfirstlane(xs) : -1;
  // the second wave of every SIMD issues first when both are ready: a fixed order
  // for the two waves that share the matrix core (measured 0.5-1 % faster than
  // the hardware's default arbitration; the reverse order gains the same)
  if (w >= NW / 2) __builtin_amdgcn_s_setprio(1);
  const int h = it.h;
  const int ntiles = it.nslots * nb + (XT && xslot >= 0 ? a.nbx : 0);

  // ---- Q operand fragments, resident for the whole item
  const int qi = 32 * w + j;
  const bool qvalid = qi < it.q_rows;
  const size_t qoff = (size_t)(it.q_tok0 + qi) * rs + (size_t)h * D;
  bf16x8 qb[FP8 ? 1 : Cfg::QSTEPS];
  intx8 q8f[FP8 ? Cfg::QSTEPS : 1];
  if constexpr (FP8) {
#pragma unroll
    for (int s = 0; s < Cfg::QSTEPS; ++s) {
      if (qvalid) {
        const uint4* p = reinterpret_cast<const uint4*>(a.q8 + qoff + 64 * s + 32 * hf);
        const uint4 x0 = p[0], x1 = p[1];
        q8f[s] = intx8{(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w, (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
      } else {
        q8f[s] = intx8{};
      }
    }
  } else {
    const uint16_t* q = static_cast<const uint16_t*>(a.q);
#pragma unroll
    for (int s = 0; s < Cfg::QSTEPS; ++s)
      qb[s] = qvalid ? *reinterpret_cast<const bf16x8*>(q + qoff + 16 * s + 8 * hf) : bf16x8{};
  }
  // The MFMAs deliver scores in log2 units directly.  bf16: the Q operand carries
  // the factor log2(e)/sqrt(d) (rounded once to bf16).  fp8: the q codes carry it
  // (applied before quantisation), and the power-of-two scales of the q and k
  // codes are the MFMA's E8M0 operand scales (sq for Q, sk for K)
  int sq = 0, sk = 0;
  if constexpr (FP8) {
    sq = a.fexp[h] + 127;
    sk = a.fexp[H + h] + 127;
  } else {
    const float scale = a.scale_log2;
#pragma unroll
    for (int s = 0; s < Cfg::QSTEPS; ++s)
#pragma unroll
      for (int e = 0; e < 8; ++e) qb[s][e] = (__bf16)((float)qb[s][e] * scale);
  }

  // ---- global -> LDS tile loads
  const unsigned char* kbase = FP8 ? reinterpret_cast<const unsigned char*>(a.k8)
                                   : static_cast<const unsigned char*>(a.k);
  auto frame_of = [&](int slot) {
    // The two forms of the lookup (and the two epilogue shapes below) make the
    // compiler lay out the tile loop differently, and the attention kernel's speed
    // and L2-miss traffic follow the layout; each path takes the combination
    // measured fastest for it (same-box A/B: bf16 at the 768p workload 247.6 vs
    // 252.4 ms, 255 vs 515 GB past L2; fp8 q.k at the long stream 425.7 vs 441.0 ms,
    // 308 vs 807 GB).
    if constexpr (PREC == 2) return it.mode == 0 ? it.k_f0 + slot : chunk_key_frame_sel(slot, it.wf, it.we, F);
    else return it.mode == 0 ? it.k_f0 + slot : chunk_key_frame(slot, it.wf, it.we, F);
  };
  // Per-lane byte offsets of this lane's 16-byte pieces inside a K tile (rows of
  // the token-major k tensor) and a V^T block; the tile base is wave-uniform.
  // (Kept in a struct: clang drops the host launch stub of a kernel template
  // whose lambda captures local arrays sized by a dependent constant.)
  // load ii of a tile is issued by wave ii % NW as its load ii / NW; lane L of
  // load ii fills LDS chunk q = 64 ii + L, i.e. row q / pitch, chunk q % pitch
  // (the padding chunk re-reads the row's last chunk; rows past a V^T block's
  // end, in its last partial load, re-read its last row)
  constexpr int KX = (Cfg::K_INSTR + NW - 1) / NW, VX = (Cfg::V_INSTR + NW - 1) / NW;
  const size_t krs = rs * (FP8 ? 1 : 2);             // token stride in bytes
  LaneOffsets<KX, VX> lo;
  uint32_t* koff = lo.koff;
  uint32_t* voff = lo.voff;
#pragma unroll
  for (int x = 0; x < KX; ++x) {
    const int q = 64 * (x * NW + w) + lane;
    const int row = q / (Cfg::KCH + 1), c = min(q % (Cfg::KCH + 1), Cfg::KCH - 1);
    koff[x] = (uint32_t)(row * krs) + 16u * c;
  }
#pragma unroll
  for (int x = 0; x < VX; ++x) {
    const int q = 64 * (x * NW + w) + lane;
    const int row = min(q / (Cfg::VCH + 1), D - 1), c = min(q % (Cfg::VCH + 1), Cfg::VCH - 1);
    voff[x] = (uint32_t)(row * (16 * Cfg::VCH) + 16 * c);
  }
  // loads [x0, x1) of this wave's share of a tile: K loads first, then V^T loads
  constexpr int LPT = KX + VX;
  auto issue_range = [&](int stage, int f, int b, int x0, int x1) {
    unsigned char* sbase = smem + stage * Cfg::STAGE;
    const int nvalid = min(BK, (XT && f == F ? a.T : N) - BK * b);
    // buffer loads to LDS (MUBUF): unlike the FLAT-encoded global_load_lds they
    // leave the compiler free to wait for LDS reads one by one (lgkmcnt(n))
    const unsigned char* kt = kbase + (((size_t)f * N + BK * b) * rs + (size_t)h * D) * (FP8 ? 1 : 2);
    // the resource ends with the frame: rows past its end read as zeros (their
    // scores are masked)
    const __amdgpu_buffer_rsrc_t krsrc = make_rsrc(kt, (uint32_t)(nvalid * krs));
#pragma unroll
    for (int x = 0; x < KX; ++x) {
      if (x < x0 || x >= x1) continue;
      if (x * NW + w >= Cfg::K_INSTR) break;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(krsrc, (lds_void_ptr)(sbase + 1024 * (x * NW + w)), 16, koff[x], 0, 0, 0);
    }
    const unsigned char* vsrc =
        XT && f == F ? reinterpret_cast<const unsigned char*>(a.vtx + ((size_t)h * a.nbx + b) * (size_t)(D * BK))
                     : reinterpret_cast<const unsigned char*>(a.vt) + (((size_t)h * F + f) * nb + b) * (size_t)(D * BK * 2);
    const __amdgpu_buffer_rsrc_t vrsrc = make_rsrc(vsrc, (uint32_t)(D * BK * 2));
#pragma unroll
    for (int x = 0; x < VX; ++x) {
      if (KX + x < x0 || KX + x >= x1) continue;
      if (x * NW + w >= Cfg::V_INSTR) break;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(vrsrc, (lds_void_ptr)(sbase + Cfg::K_BYTES + 1024 * (x * NW + w)), 16,
                                               voff[x], 0, 0, 0);
    }
  };
  // Tile cursors: ld_* is the next tile to load, b the 64-key block of tile t.
  // Tiles go through NSTG LDS stages and are loaded NSTG/2 tiles ahead; a
  // workgroup barrier every NSTG/2 tiles publishes the loads of the next group
  // of tiles and frees the stages of the previous one.
  constexpr int NSTG = kLdsStages, AHEAD = NSTG / 2;
  int ld_slot = 0, ld_b = 0, ld_f = frame_of(0);
  auto next_load = [&]() {
    if (++ld_b == nb) {
      ld_b = 0;
      ld_f = frame_of(++ld_slot);
    }
  };

  floatx16 o[NDB];
#pragma unroll
  for (int x = 0; x < NDB; ++x) o[x] = floatx16{};
  // running max m (log2 units).  The Q.K^T accumulators start at -m, so the
  // MFMAs leave s - m and the exponent needs no VALU op; m is finite from the
  // start and the first tile sets it to that tile's maximum
  float m_run = 0.f, l_run = 0.f;
  floatx16 nm = floatx16{};      // -m in every element: the first Q.K^T accumulator input
  if constexpr (XI) {
    // start from the state after the extra tokens' keys (l on the first half-wave
    // only: the two halves' partial sums are added at the end)
    if (qvalid) {
      const float* ps = a.px + ((size_t)h * F * N + it.q_tok0 + qi) * (D + 4);
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const float4 x4 = *reinterpret_cast<const float4*>(ps + 32 * db + 8 * g + 4 * hf);
          o[db][4 * g + 0] = x4.x;
          o[db][4 * g + 1] = x4.y;
          o[db][4 * g + 2] = x4.z;
          o[db][4 * g + 3] = x4.w;
        }
      m_run = ps[D];
      l_run = hf == 0 ? ps[D + 1] : 0.f;
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) nm[r] = -m_run;
  }

  // with extra tokens, tiles t >= t_x (the last ones of the key list, when the
  // item has them) are the extra tokens' 64-key blocks t - t_x, frame index F;
  // the frame cursor above walks the video frames only
  const int t_x = it.nslots * nb;
#pragma unroll
  for (int x = 0; x < AHEAD; ++x) {
    if (x < ntiles) {
      if (XT && x >= t_x) {
        issue_range(x, F, x - t_x, 0, LPT);
      } else {
        issue_range(x, ld_f, ld_b, 0, LPT);
        next_load();
      }
    }
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  int b = 0;
  for (int t = 0; t < ntiles; ++t) {
    const int stage = t & (NSTG - 1);
    const bool ld = t + AHEAD < ntiles;      // load tile t + AHEAD during this tile
    int ldf = ld_f, ldb = ld_b;
    int nvalid;
    if constexpr (XT) {
      if (t + AHEAD >= t_x) {
        ldf = F;
        ldb = t + AHEAD - t_x;
      } else if (ld) {
        next_load();
      }
      if (t >= t_x) {
        nvalid = min(BK, a.T - BK * (t - t_x));
      } else {
        nvalid = min(BK, N - BK * b);
        if (++b == nb) b = 0;
      }
    } else {
      if (ld) next_load();
      nvalid = min(BK, N - BK * b);
      if (++b == nb) b = 0;
    }
    const unsigned char* sbase = smem + stage * Cfg::STAGE;

    // ---- S^T = K Q^T.  Operand fragments come from LDS in batches, double
    // buffered: each batch's reads are issued before the previous batch's
    // MFMAs, so one batch is in flight while the matrix core works.
    const unsigned char* vbase = sbase + Cfg::K_BYTES;
    constexpr int NQK = 2 * Cfg::QSTEPS, QB = NQK < kQkBatch ? NQK : kQkBatch, NQB = NQK / QB;
    typename LdsCfg<D, PREC>::KFrag kf[2][QB];
    bf16x8 va[2][NDB];
    floatx16 s[2] = {nm, nm};
#pragma unroll
    for (int x = 0; x < QB; ++x) kf[0][x] = Cfg::kfrag(sbase, x, j, hf);
#pragma unroll
    for (int bt = 0; bt < NQB; ++bt) {
      if (VDN_LDS_WAITALL) lds_wait_all();
      if (bt + 1 < NQB) {
#pragma unroll
        for (int x = 0; x < QB; ++x) kf[(bt + 1) & 1][x] = Cfg::kfrag(sbase, (bt + 1) * QB + x, j, hf);
      } else {
#pragma unroll
        for (int db = 0; db < NDB; ++db) va[0][db] = Cfg::vfrag(vbase, 0, db, j, hf);
      }
      // this batch's share of the next tile's loads: spread over the batches so
      // the address unit works through them while the MFMAs run, instead of
      // every wave queueing its loads at once
      if (ld) issue_range((t + AHEAD) & (NSTG - 1), ldf, ldb, bt * LPT / NQB, (bt + 1) * LPT / NQB);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int x = 0; x < QB; ++x) {
        const int i = bt * QB + x, st = i >> 1, kb = i & 1;
        if constexpr (FP8) s[kb] = mfma_fp8_scaled(kf[bt & 1][x], q8f[st], s[kb], sk, sq);
        else s[kb] = mfma_bf16(kf[bt & 1][x], qb[st], s[kb]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }

    // ---- online softmax (see attn_kernel): maxima, lazy raise
    if (nvalid < BK) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = 32 * kb + 8 * (r >> 2) + 4 * hf + (r & 3);
          if (key >= nvalid) s[kb][r] = -INFINITY;
        }
    }
    float mx = __builtin_fmaxf(s[0][0], s[1][0]);
#pragma unroll
    for (int e = 1; e < 16; ++e) mx = __builtin_fmaxf(__builtin_fmaxf(mx, s[0][e]), s[1][e]);
    // (a row's maximum is split over the two lanes of a pair, both in this wave:
    // the wave-wide test gives the same answer on the per-lane parts, so the pair
    // combine runs only when the maximum is raised)
    {
      // scores are s - m already: raise m by the excess (on the first tile, by the
      // tile maximum whatever its sign; nothing is accumulated yet to rescale)
      const bool first = !XI && t == 0;     // nothing accumulated yet
      if (first || __any(mx > kLazy)) {
        mx = pair_max(mx);
        const float dm = first ? mx : __builtin_fmaxf(mx, 0.f);
        if (!first) {
          const float alpha = __builtin_amdgcn_exp2f(-dm);
          l_run *= alpha;
#pragma unroll
          for (int x = 0; x < NDB; ++x) o[x] *= alpha;
        }
        m_run += dm;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) s[kb][r] -= dm;
#pragma unroll
        for (int r = 0; r < 16; ++r) nm[r] = -m_run;
      }
      asm volatile("" : "+v"(nm));   // keep it in registers rather than rebuild it every tile
    }
    // exponent of a score: the scores are already s - m in log2 units
    auto expo = [&](float x) { return __builtin_amdgcn_exp2f(x); };

    // ---- O^T += V^T P^T, one group of 16 keys per batch; the probabilities of
    // the next group are formed on the VALU while this group's MFMAs run, and
    // the row sum l takes the same bf16 values, two per v_dot2_f32_bf16
    const bf16x2 ones = {(__bf16)1.f, (__bf16)1.f};
    float psum = 0.f;
    bf16x8 pb[2];
#pragma unroll
    for (int e = 0; e < 8; ++e) pb[0][e] = (__bf16)expo(s[0][e]);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if (VDN_LDS_WAITALL) lds_wait_all();
      if (u + 1 < 4) {
#pragma unroll
        for (int db = 0; db < NDB; ++db) va[(u + 1) & 1][db] = Cfg::vfrag(vbase, u + 1, db, j, hf);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int db = 0; db < NDB; ++db) o[db] = mfma_bf16(va[u & 1][db], pb[u & 1], o[db]);
      if (u + 1 < 4) {
        const int kb = (u + 1) >> 1, e0 = 8 * ((u + 1) & 1);
#pragma unroll
        for (int e = 0; e < 8; ++e)
          pb[(u + 1) & 1][e] = (__bf16)expo(s[kb][e0 + e]);
      }
#pragma unroll
      for (int e = 0; e < 8; e += 2)
        psum = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{pb[u & 1][e], pb[u & 1][e + 1]}, ones, psum, false);
      // a fixed interleave: each MFMA followed by two exponentials and two other
      // VALU ops (left to the scheduler, the order follows unrelated code elsewhere
      // in the kernel, and some orders measured up to 3 % slower)
#pragma unroll
      for (int x = 0; x < NDB; ++x) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x400, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    l_run += psum;

    if ((t & (AHEAD - 1)) == AHEAD - 1 || t + 1 == ntiles) {
      __builtin_amdgcn_s_waitcnt(0);   // this wave's loads of the next tiles landed
      __syncthreads();                 // ... and every other wave's; all reads of this group done
    }
  }

  // ---- epilogue
  const float l_tot = pair_sum(l_run);
  // Linear-branch readout and gated merge, fused (besthub article "VDN-H3
  // Generates 14-Second 768p Video ...", Hybrid Attention Architecture: the gated
  // linear output is added to the softmax output): every query row of a chunk
  // item lies in one chunk c, whose readout weights W = g (.) (S_fwd + S_bwd) come
  // into the LDS stages (free since the last tile's barrier) by the same padded
  // direct loads as a K tile; then O^T = O_soft^T + W Q^T with Q as the B operand
  // it already is.  Anchor query frames (split items) take no linear term.
  constexpr int WCH = D / 8;                         // 16-byte chunks per bf16 W row
  constexpr int WP = 16 * (WCH + 1);                 // LDS pitch of a W row
  constexpr int W_INSTR = (D * (WCH + 1) + 63) / 64; // wave-wide direct loads for W
  static_assert(1024 * W_INSTR <= kLdsStages * Cfg::STAGE, "W fits in the LDS stages");
  // The arguments only the epilogue needs (output pointers, readout weights) are
  // read here, from the kernel's argument segment behind an empty asm statement,
  // so that they are not loaded at entry and held in scalar registers through the
  // tile loop.
  using KArgs = const __attribute__((address_space(4))) AttnArgs*;
  KArgs kargs = (KArgs)__builtin_amdgcn_kernarg_segment_ptr();
  asm volatile("" : "+s"(kargs));
  if constexpr (XT) {
    if (it.split < 0) {
      // chunk item over the extra tokens' keys: leave the state for the video pass
      if (qvalid) {
        float* ps = kargs->px + ((size_t)h * F * N + it.q_tok0 + qi) * (D + 4);
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int g = 0; g < 4; ++g)
            *reinterpret_cast<float4*>(ps + 32 * db + 8 * g + 4 * hf) =
                make_float4(o[db][4 * g + 0], o[db][4 * g + 1], o[db][4 * g + 2], o[db][4 * g + 3]);
        if (hf == 0) {
          ps[D] = m_run;
          ps[D + 1] = l_tot;
        }
      }
      return;
    }
  }
  const uint16_t* Wp = kargs->W;
  const bool lin = it.split < 0 && Wp != nullptr;    // workgroup-uniform
  // fp8 q.k: q rows as stored (the resident fragments are E4M3 codes), loaded
  // beside the W tile
  bf16x8 q8r[FP8 ? D / 16 : 1];
  if (lin) {
    const int chunk = it.q_tok0 / N / kChunk;      // chunk of the item's first (and every) row
    const uint16_t* wsrc = Wp + ((size_t)chunk * H + h) * (size_t)(D * D);
    // rows past D (the last partial load at D = 32) read as zeros and are never used
    const __amdgpu_buffer_rsrc_t wrsrc = make_rsrc(wsrc, (uint32_t)(D * D * 2));
#pragma unroll
    for (int x = 0; x < (W_INSTR + NW - 1) / NW; ++x) {
      if (x * NW + w >= W_INSTR) break;
      const int q = 64 * (x * NW + w) + lane;
      const int row = q / (WCH + 1), c = min(q % (WCH + 1), WCH - 1);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(wrsrc, (lds_void_ptr)(smem + 1024 * (x * NW + w)), 16,
                                               (uint32_t)(row * 2 * D + 16 * c), 0, 0, 0);
    }
    if constexpr (FP8) {
      const uint16_t* qrow = static_cast<const uint16_t*>(kargs->q) + (size_t)(it.q_tok0 + qi) * rs + (size_t)h * D;
#pragma unroll
      for (int s = 0; s < D / 16; ++s)
        q8r[s] = qvalid ? *reinterpret_cast<const bf16x8*>(qrow + 16 * s + 8 * hf) : bf16x8{};
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }
  // (all lanes take part in the MFMAs: lane j also supplies row j of W; rows of
  // Q past the item's end are zeros)
  float inv = 1.f / l_tot;
  if constexpr (SPLIT) {
    if (lin) {
      constexpr int QS = D / 16;
      bf16x8 qr[QS];
      float us;
      if constexpr (FP8) {
#pragma unroll
        for (int s = 0; s < QS; ++s) qr[s] = q8r[s];
        us = 1.f;
      } else {
#pragma unroll
        for (int s = 0; s < QS; ++s) qr[s] = qb[s];
        us = 1.f / kargs->scale_log2;
      }
      // token stride 2 H D: O_soft at h D, g (.) O_lin at H D + h D
      uint16_t* ao = static_cast<uint16_t*>(kargs->O) + (size_t)(it.q_tok0 + qi) * (2 * rs) + (size_t)h * D;
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        floatx16 acc = floatx16{};
#pragma unroll
        for (int s = 0; s < QS; ++s)
          acc = mfma_bf16(*reinterpret_cast<const bf16x8*>(smem + (32 * db + j) * WP + 16 * (2 * s + hf)), qr[s], acc);
        if (qvalid) {
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int dd = 32 * db + 8 * g + 4 * hf;
            const floatx16& c = o[db];
            *reinterpret_cast<uint2*>(ao + dd) =
                make_uint2(pack_bf16x2(c[4 * g + 0] * inv, c[4 * g + 1] * inv),
                           pack_bf16x2(c[4 * g + 2] * inv, c[4 * g + 3] * inv));
            *reinterpret_cast<uint2*>(ao + rs + dd) =
                make_uint2(pack_bf16x2(acc[4 * g + 0] * us, acc[4 * g + 1] * us),
                           pack_bf16x2(acc[4 * g + 2] * us, acc[4 * g + 3] * us));
          }
        }
      }
      return;
    }
  }
  if (lin) {
    // Q in bf16 as the B operand: the bf16 path's resident fragments carry the
    // factor log2(e)/sqrt(d) (rounded to bf16 with it), taken back out of the
    // product; the fp8 path reads q.  (A version that read q rows in the bf16 path
    // too, for a single rounding of q, compiled the tile loop differently and ran
    // 1.9 % slower with twice the L2-miss traffic, same-box A/B; the fragments'
    // extra rounding is at most 2^-9 relative per q entry.)
    constexpr int QS = D / 16;
    bf16x8 qr[QS];
    float us;
    if constexpr (FP8) {
#pragma unroll
      for (int s = 0; s < QS; ++s) qr[s] = q8r[s];
      us = 1.f;
    } else {
#pragma unroll
      for (int s = 0; s < QS; ++s) qr[s] = qb[s];
      us = 1.f / kargs->scale_log2;
    }
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      floatx16 acc = floatx16{};
#pragma unroll
      for (int s = 0; s < QS; ++s)
        acc = mfma_bf16(*reinterpret_cast<const bf16x8*>(smem + (32 * db + j) * WP + 16 * (2 * s + hf)), qr[s], acc);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        if constexpr (FP8) o[db][r] = fmaf(o[db][r], inv, acc[r]);
        else o[db][r] = fmaf(acc[r], us, o[db][r] * inv);
      }
    }
    inv = 1.f;
  }
  if (!qvalid) return;
  if (it.split < 0) {
    const size_t ooff = (size_t)(it.q_tok0 + qi) * rs + (size_t)h * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int dd = 32 * db + 8 * g + 4 * hf;
        const uint2 pk = make_uint2(pack_bf16x2(o[db][4 * g + 0] * inv, o[db][4 * g + 1] * inv),
                                    pack_bf16x2(o[db][4 * g + 2] * inv, o[db][4 * g + 3] * inv));
        *reinterpret_cast<uint2*>(static_cast<uint16_t*>(kargs->O) + ooff + dd) = pk;
      }
  } else {
    size_t row;
    if constexpr (XT) {
      // rows per head: the anchor frames' N each, then the T extra tokens
      const int na = kargs->na, R = na * N + kargs->T;
      const int rr = it.anchor_idx < na
                         ? it.anchor_idx * N + it.q_tok0 - (it.anchor_idx == 0 ? 0 : (F - 1) * N) + qi
                         : na * N + it.q_tok0 - F * N + qi;
      row = ((size_t)it.split * H + h) * R + rr;
    } else {
      const int n = it.q_tok0 - (it.anchor_idx == 0 ? 0 : (F - 1) * N) + qi;
      row = (((size_t)it.split * H + h) * kargs->na + it.anchor_idx) * N + n;
    }
    float* po = kargs->part_O + row * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int dd = 32 * db + 8 * g + 4 * hf;
        *reinterpret_cast<float4*>(po + dd) =
            make_float4(o[db][4 * g + 0], o[db][4 * g + 1], o[db][4 * g + 2], o[db][4 * g + 3]);
      }
    if (hf == 0) {
      kargs->part_ml[2 * row + 0] = m_run;
      kargs->part_ml[2 * row + 1] = l_tot;
    }
  }
}

// ============================================================ attention, full fp8, two groups of waves
// With P.V on E4M3 codes a tile costs about as much vector work (the softmax of
// 64 keys: maxima, exponentials, E4M3 conversions) as matrix work (Q.K^T and P.V
// on E4M3 codes, the row sums), and a wave's vector instructions do not issue
// under its own MFMAs (accumulators in VGPRs): the two waves that share a SIMD
// have to take turns on the two units.  With one barrier per tile
// (attn_lds_kernel) they start every tile together and their softmaxes collide.
// Here the workgroup advances in segments separated by one barrier; in segment k
//   waves 0-3 (one per SIMD): P.V of tile k-1 and Q.K^T of tile k, then the
//                             softmax of tile k;
//   waves 4-7:                the softmax of tile k-1, then P.V of tile k-1 and
//                             Q.K^T of tile k,
// so in each half of a segment one wave of a SIMD issues MFMAs while the other
// runs its softmax.  Every wave takes its tiles in order with the same arithmetic
// as attn_lds_kernel (the outputs are bitwise equal).  Segment k reads tiles k-1
// and k and loads tile k+1 (four LDS stages).  The compiler makes a wave wait for
// its own direct loads before its next LDS read, so waves 4-7 issue all of a
// tile's loads at the start of a segment, before their softmax, and their first
// operand read comes a softmax later.  Plain video layer (no extra tokens, no
// split output).

// The softmax of one 64-key tile: scores s (already s - m in log2 units) of the
// wave's 32 queries, lazy running-max raise (rescaling o and the row sums), then
// the E4M3 probabilities in pf.  Cursor: tile sm_t, its 64-key block sm_b of the
// frame.
template <int NDB>
__device__ __forceinline__ void pp_softmax(floatx16 (&s)[2], floatx16 (&o)[NDB], floatx16& nm, floatx16& lsum,
                                           intx8& pf, float& m_run, int& sm_t, int& sm_b, int N, int nb, int hf) {
  const int nvalid = min(BK, N - BK * sm_b);
  if (++sm_b == nb) sm_b = 0;
  if (nvalid < BK) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = 32 * kb + 8 * (r >> 2) + 4 * hf + (r & 3);
        if (key >= nvalid) s[kb][r] = -INFINITY;
      }
  }
  float mx = __builtin_fmaxf(s[0][0], s[1][0]);
#pragma unroll
  for (int e = 1; e < 16; ++e) mx = __builtin_fmaxf(__builtin_fmaxf(mx, s[0][e]), s[1][e]);
  const bool first = sm_t == 0;
  if (first || __any(mx > kLazy)) {
    mx = pair_max(mx);
    const float dm = first ? mx : __builtin_fmaxf(mx, 0.f);
    if (!first) {
      const float alpha = __builtin_amdgcn_exp2f(-dm);
      lsum *= alpha;
#pragma unroll
      for (int x = 0; x < NDB; ++x) o[x] *= alpha;
    }
    m_run += dm;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) s[kb][r] -= dm;
#pragma unroll
    for (int r = 0; r < 16; ++r) nm[r] = -m_run;
  }
  asm volatile("" : "+v"(nm));
  // lane (j, hf) holds keys 32 kb + 8 (r / 4) + 4 hf + r % 4: bytes 16 kb + r.  (Each
  // word starts from zero in a fresh register: converting into the old word, which
  // the previous P.V MFMAs may still be reading, measured 14 % slower.)
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const int kb = t >> 2, r0 = 4 * (t & 3);
    const float p0 = __builtin_amdgcn_exp2f(s[kb][r0]), p1 = __builtin_amdgcn_exp2f(s[kb][r0 + 1]);
    const float p2 = __builtin_amdgcn_exp2f(s[kb][r0 + 2]), p3 = __builtin_amdgcn_exp2f(s[kb][r0 + 3]);
    int wd = __builtin_amdgcn_cvt_pk_fp8_f32(p0, p1, 0, false);
    wd = __builtin_amdgcn_cvt_pk_fp8_f32(p2, p3, wd, true);
    pf[t] = wd;
  }
  ++sm_t;
}

template <int D>
__global__ __launch_bounds__(512, 2) void attn_pp_kernel(AttnArgs a) {
  using Cfg = LdsCfg<D, 3>;
  constexpr int NW = 8, NDB = D / 32, NSTG = 4, NQK = 2 * Cfg::QSTEPS;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];

  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int j = lane & 31, hf = lane >> 5;
  const bool lead = w < NW / 2;          // matrix half of a segment first
  // waves 4-7 (softmax first) issue first when both waves of a SIMD are ready
  // (same-box A/B at the long stream: 306.0 ms against 352.5 with no priority and
  // 354.1 with waves 0-3 first; priorities switched with the phase: 335-355 ms)
  if (!lead) __builtin_amdgcn_s_setprio(1);
  const int F = a.F, N = a.N, H = a.H;
  const size_t rs = (size_t)H * D;       // token stride (elements; one byte each as codes)
  const int nb = (N + BK - 1) / BK;
  // the item from the queues (one thread takes it, one LDS word hands it over)
  int* slot = reinterpret_cast<int*>(smem + NSTG * Cfg::STAGE);
  if (tid == 0) *slot = acquire_item(a);
  __syncthreads();
  const int pk = __builtin_amdgcn_readfirstlane(*slot);
  if (pk < 0) return;
  const int Mi = a.na * a.qt_anchor * a.nsplit + a.tiles_per_head;
  const int hh0 = pk / Mi;
  const Item it = uniform_item(decode_item_at(a, hh0, pk - hh0 * Mi));
  const int h = it.h;
  const int ntiles = it.nslots * nb;

  // ---- Q operand fragments (E4M3 codes carrying log2(e)/sqrt(d)), resident
  const int qi = 32 * w + j;
  const bool qvalid = qi < it.q_rows;
  const size_t qoff = (size_t)(it.q_tok0 + qi) * rs + (size_t)h * D;
  intx8 q8f[Cfg::QSTEPS];
#pragma unroll
  for (int st = 0; st < Cfg::QSTEPS; ++st) {
    if (qvalid) {
      const uint4* p = reinterpret_cast<const uint4*>(a.q8 + qoff + 64 * st + 32 * hf);
      const uint4 x0 = p[0], x1 = p[1];
      q8f[st] = intx8{(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w, (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
    } else {
      q8f[st] = intx8{};
    }
  }
  const int sq = a.fexp[h] + 127, sk = a.fexp[H + h] + 127, sv = a.fexp[2 * H + h] + 127;

  // ---- global -> LDS tile loads by waves 4-7: load ii of a tile is issued by wave
  // 4 + ii % 4 as its load ii / 4; lane L of load ii fills LDS chunk 64 ii + L (the
  // padded rows of attn_lds_kernel)
  auto frame_of = [&](int fslot) {
    return it.mode == 0 ? it.k_f0 + fslot : chunk_key_frame(fslot, it.wf, it.we, F);
  };
  constexpr int NL = NW / 2;
  const int wl = w & (NL - 1);
  constexpr int KX = (Cfg::K_INSTR + NL - 1) / NL, VX = (Cfg::V_INSTR + NL - 1) / NL;
  // (the lambda reaches the offsets through pointers: clang drops the host launch
  // stub of a kernel template whose lambda captures an array sized by a dependent
  // constant)
  LaneOffsets<KX, VX> lo;
  uint32_t* koff = lo.koff;
  uint32_t* voff = lo.voff;
#pragma unroll
  for (int x = 0; x < KX; ++x) {
    const int q = 64 * (x * NL + wl) + lane;
    const int row = q / (Cfg::KCH + 1), c = min(q % (Cfg::KCH + 1), Cfg::KCH - 1);
    koff[x] = (uint32_t)(row * rs) + 16u * c;
  }
#pragma unroll
  for (int x = 0; x < VX; ++x) {
    const int q = 64 * (x * NL + wl) + lane;
    const int row = min(q / (Cfg::VCH + 1), D - 1), c = min(q % (Cfg::VCH + 1), Cfg::VCH - 1);
    voff[x] = (uint32_t)(row * (16 * Cfg::VCH) + 16 * c);
  }
  int ld_slot = 0, ld_b = 0, ld_f = frame_of(0), ldt = 0;
  // waves 4-7: their share of tile ldt, into its stage (every wave keeps the cursor)
  auto issue_tile = [&]() {
    if (!lead) {
      unsigned char* sbase = smem + (ldt & (NSTG - 1)) * Cfg::STAGE;
      const int nvalid = min(BK, N - BK * ld_b);
      const unsigned char* kt = a.k8 + ((size_t)ld_f * N + BK * ld_b) * rs + (size_t)h * D;
      // the resource ends with the frame: rows past its end read as zeros (masked)
      const __amdgpu_buffer_rsrc_t krsrc = make_rsrc(kt, (uint32_t)(nvalid * rs));
#pragma unroll
      for (int x = 0; x < KX; ++x) {
        if (x * NL + wl >= Cfg::K_INSTR) break;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(krsrc, (lds_void_ptr)(sbase + 1024 * (x * NL + wl)), 16, koff[x], 0,
                                                 0, 0);
      }
      const unsigned char* vsrc =
          reinterpret_cast<const unsigned char*>(a.vt) + (((size_t)h * F + ld_f) * nb + ld_b) * (size_t)(D * BK);
      const __amdgpu_buffer_rsrc_t vrsrc = make_rsrc(vsrc, (uint32_t)(D * BK));
#pragma unroll
      for (int x = 0; x < VX; ++x) {
        if (x * NL + wl >= Cfg::V_INSTR) break;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(vrsrc, (lds_void_ptr)(sbase + Cfg::K_BYTES + 1024 * (x * NL + wl)),
                                                 16, voff[x], 0, 0, 0);
      }
    }
    ++ldt;
    if (++ld_b == nb) {
      ld_b = 0;
      ld_f = frame_of(++ld_slot);
    }
  };

  issue_tile();                      // ntiles >= 1
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  floatx16 o[NDB];
#pragma unroll
  for (int x = 0; x < NDB; ++x) o[x] = floatx16{};
  float m_run = 0.f;
  floatx16 lsum = floatx16{};        // row sums from the all-ones MFMA (every element)
  floatx16 nm = floatx16{};          // -m in every element: the Q.K^T accumulator start
  floatx16 s[2];                     // scores of the tile whose softmax is next
  intx8 pf = intx8{};                // E4M3 probabilities of the tile whose P.V is next
  int sm_t = 0, sm_b = 0;            // softmax cursor: tile, its 64-key block in the frame
  // the row sums' all-ones A operand (E4M3 1.0 in every byte), kept in registers
  // rather than rebuilt every tile
  constexpr int kOne = 0x38383838;
  intx8 ones8 = intx8{kOne, kOne, kOne, kOne, kOne, kOne, kOne, kOne};

  for (int k = 0; k <= ntiles; ++k) {
    if (!lead && k + 1 < ntiles) issue_tile();     // tile k + 1
    if (!lead && k > 0) pp_softmax<NDB>(s, o, nm, lsum, pf, m_run, sm_t, sm_b, N, nb, hf);   // tile k - 1
    {
      // P.V of tile k - 1 (probabilities from the softmax before it): the V^T
      // operands read together, then the MFMAs; then Q.K^T of tile k into s
      const unsigned char* vbase = smem + ((k - 1) & (NSTG - 1)) * Cfg::STAGE + Cfg::K_BYTES;
      const unsigned char* kbase = smem + (k & (NSTG - 1)) * Cfg::STAGE;
      if (k > 0) {
        intx8 vf8[NDB];
#pragma unroll
        for (int db = 0; db < NDB; ++db) vf8[db] = Cfg::vfrag8(vbase, db, j, hf);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int db = 0; db < NDB; ++db) o[db] = mfma_fp8_scaled(vf8[db], pf, o[db], sv, 127);
        asm volatile("" : "+v"(ones8));
        lsum = mfma_fp8_scaled(ones8, pf, lsum, 127, 127);
        __builtin_amdgcn_sched_barrier(0);
      }
      if (k < ntiles) {
        intx8 kf[NQK];
#pragma unroll
        for (int i = 0; i < NQK; ++i) kf[i] = Cfg::kfrag(kbase, i, j, hf);
        s[0] = nm;
        s[1] = nm;
#pragma unroll
        for (int i = 0; i < NQK; ++i) s[i & 1] = mfma_fp8_scaled(kf[i], q8f[i >> 1], s[i & 1], sk, sq);
      }
    }
    if (lead && k < ntiles) pp_softmax<NDB>(s, o, nm, lsum, pf, m_run, sm_t, sm_b, N, nb, hf);   // tile k
    // end of the segment: this wave's loads of tile k + 1 have landed and its LDS
    // reads are done; the barrier publishes tile k + 1 and frees tile k - 1's stage.
    // (A plain s_barrier: __syncthreads' fence adds nothing here.)
    __builtin_amdgcn_s_waitcnt(0x0070);            // vmcnt(0) lgkmcnt(0)
    asm volatile("s_barrier" ::: "memory");
  }

  // ---- epilogue (as attn_lds_kernel's video path): readout + gated merge for
  // chunk items, the unnormalised state for the anchor rows' key slices
  const float l_tot = lsum[0];
  constexpr int WCH = D / 8;
  constexpr int WP = 16 * (WCH + 1);
  constexpr int W_INSTR = (D * (WCH + 1) + 63) / 64;
  static_assert(1024 * W_INSTR <= NSTG * Cfg::STAGE, "W fits in the LDS stages");
  using KArgs = const __attribute__((address_space(4))) AttnArgs*;
  KArgs kargs = (KArgs)__builtin_amdgcn_kernarg_segment_ptr();
  asm volatile("" : "+s"(kargs));
  const uint16_t* Wp = kargs->W;
  const bool lin = it.split < 0 && Wp != nullptr;   // workgroup-uniform
  float inv = 1.f / l_tot;
  if (lin) {
    const int chunk = it.q_tok0 / N / kChunk;
    const uint16_t* wsrc = Wp + ((size_t)chunk * H + h) * (size_t)(D * D);
    const __amdgpu_buffer_rsrc_t wrsrc = make_rsrc(wsrc, (uint32_t)(D * D * 2));
#pragma unroll
    for (int x = 0; x < (W_INSTR + NW - 1) / NW; ++x) {
      if (x * NW + w >= W_INSTR) break;
      const int q = 64 * (x * NW + w) + lane;
      const int row = q / (WCH + 1), c = min(q % (WCH + 1), WCH - 1);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(wrsrc, (lds_void_ptr)(smem + 1024 * (x * NW + w)), 16,
                                               (uint32_t)(row * 2 * D + 16 * c), 0, 0, 0);
    }
    // q rows as stored (the resident fragments are E4M3 codes)
    constexpr int QS = D / 16;
    bf16x8 qr[QS];
    const uint16_t* qrow = static_cast<const uint16_t*>(kargs->q) + qoff;
#pragma unroll
    for (int st = 0; st < QS; ++st) qr[st] = qvalid ? *reinterpret_cast<const bf16x8*>(qrow + 16 * st + 8 * hf) : bf16x8{};
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      floatx16 acc = floatx16{};
#pragma unroll
      for (int st = 0; st < QS; ++st)
        acc = mfma_bf16(*reinterpret_cast<const bf16x8*>(smem + (32 * db + j) * WP + 16 * (2 * st + hf)), qr[st], acc);
      // (the rounding order of attn_lds_kernel's full-fp8 epilogue)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[db][r] = fmaf(acc[r], 1.f, o[db][r] * inv);
    }
    inv = 1.f;
  }
  if (!qvalid) return;
  if (it.split < 0) {
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int dd = 32 * db + 8 * g + 4 * hf;
        const uint2 v2 = make_uint2(pack_bf16x2(o[db][4 * g + 0] * inv, o[db][4 * g + 1] * inv),
                                    pack_bf16x2(o[db][4 * g + 2] * inv, o[db][4 * g + 3] * inv));
        *reinterpret_cast<uint2*>(static_cast<uint16_t*>(kargs->O) + qoff + dd) = v2;
      }
  } else {
    const int n = it.q_tok0 - (it.anchor_idx == 0 ? 0 : (F - 1) * N) + qi;
    const size_t row = (((size_t)it.split * H + h) * kargs->na + it.anchor_idx) * N + n;
    float* po = kargs->part_O + row * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int dd = 32 * db + 8 * g + 4 * hf;
        *reinterpret_cast<float4*>(po + dd) =
            make_float4(o[db][4 * g + 0], o[db][4 * g + 1], o[db][4 * g + 2], o[db][4 * g + 3]);
      }
    if (hf == 0) {
      kargs->part_ml[2 * row + 0] = m_run;
      kargs->part_ml[2 * row + 1] = l_tot;
    }
  }
}

// ============================================================ combine
// One thread per (split-merged row, 4 channels).  Rows: [H][na * N + T], the
// anchor frames' tokens, then the extra tokens'.
// ostride: output elements per token (H D; 2 H D when the output holds O_soft and
// g (.) O_lin side by side, the second half then written as zeros: anchor rows have
// no linear term).
template <int D, bool F32OUT>
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ part_O,
                                                      const float* __restrict__ part_ml, int F,
                                                      int N, int T, int H, int na, int nsplit, void* O,
                                                      int ostride) {
  const int R = na * N + T;
  const size_t rows = (size_t)H * R;
  const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= rows * (D / 4)) return;
  const size_t row = idx / (D / 4);
  const int c4 = idx % (D / 4);
  const int h = row / R, rr = row % R;
  float m = -INFINITY;
  for (int s = 0; s < nsplit; ++s) m = fmaxf(m, part_ml[2 * (s * rows + row)]);
  float l = 0.f;
  float4 acc = make_float4(0, 0, 0, 0);
  for (int s = 0; s < nsplit; ++s) {
    const size_t r = s * rows + row;
    const float wgt = __builtin_amdgcn_exp2f(part_ml[2 * r] - m);
    l += wgt * part_ml[2 * r + 1];
    const float4 x = *reinterpret_cast<const float4*>(part_O + r * D + 4 * c4);
    acc.x += wgt * x.x;
    acc.y += wgt * x.y;
    acc.z += wgt * x.z;
    acc.w += wgt * x.w;
  }
  const float inv = 1.f / l;
  const size_t tok = rr < na * N ? (size_t)(rr < N ? 0 : F - 1) * N + rr % N : (size_t)F * N + (rr - na * N);
  const size_t off = tok * ostride + (size_t)h * D + 4 * c4;
  if constexpr (F32OUT) {
    *reinterpret_cast<float4*>(static_cast<float*>(O) + off) =
        make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
  } else {
    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(O) + off) =
        make_uint2(pack_bf16x2(acc.x * inv, acc.y * inv), pack_bf16x2(acc.z * inv, acc.w * inv));
    if (ostride != H * D) *reinterpret_cast<uint2*>(static_cast<uint16_t*>(O) + off + (size_t)H * D) = make_uint2(0, 0);
  }
}

// ============================================================ fp8 quantiser

__global__ void fill_u32_kernel(uint32_t* p, int n, uint32_t value) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = value;
}

hipError_t launch_fill_u32(uint32_t* p, int n, uint32_t value, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(fill_u32_kernel, dim3((n + 255) / 256), dim3(256), 0, st, p, n, value);
  return hipGetLastError();
}

// grid (ceil(F*N / 1024), H), 256 threads: max |x| over 1024 tokens of head h.
template <int D>
__global__ __launch_bounds__(256) void amax_kernel(const uint16_t* __restrict__ x, size_t ntok, int H,
                                                   uint32_t* __restrict__ amax_bits) {
  constexpr int CPR = D / 8;                       // 16-byte chunks per (token, head) row
  const int h = blockIdx.y;
  const size_t t0 = (size_t)blockIdx.x * 1024;
  float m = 0.f;
  for (int c = threadIdx.x; c < 1024 * CPR; c += 256) {
    const size_t t = t0 + c / CPR;
    if (t < ntok) {
      const uint4 val = *reinterpret_cast<const uint4*>(x + t * H * D + (size_t)h * D + 8 * (c % CPR));
      const uint32_t wv[4] = {val.x, val.y, val.z, val.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        m = fmaxf(m, fabsf(__uint_as_float(wv[e] << 16)));
        m = fmaxf(m, fabsf(__uint_as_float(wv[e] & 0xffff0000u)));
      }
    }
  }
  m = wave_max(m);
  __shared__ float red[4];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    // non-negative floats order like their bit patterns: the max is exact and
    // independent of the order in which blocks arrive
    atomicMax(&amax_bits[h], __float_as_uint(m));
  }
}

// The power-of-two scale exponent of a head: the smallest integer e with
// amax <= 448 * 2^e, clamped to [-127, 127] (an E8M0 scale byte is e + 127); 0 for
// amax = 0.  From the binary exponent of amax: amax = f 2^x with f in [0.5, 1),
// and 448 = 0.875 * 2^9, so e = x - 9 if f <= 0.875, else x - 8 (exact).
__device__ inline int fp8_scale_exponent(float amax) {
  if (!(amax > 0.f)) return 0;
  const int x = __builtin_amdgcn_frexp_expf(amax);
  const float f = __builtin_amdgcn_frexp_mantf(amax);
  const int e = f <= 0.875f ? x - 9 : x - 8;
  return e < -127 ? -127 : (e > 127 ? 127 : e);
}

// one thread per head: amax bits (from amax_kernel) -> scale exponent, in place;
// the amax is that of fp32(x * prescale)
__global__ void fp8_exp_kernel(uint32_t* __restrict__ bits, int H, float prescale) {
  const int h = blockIdx.x * blockDim.x + threadIdx.x;
  if (h < H) bits[h] = static_cast<uint32_t>(fp8_scale_exponent(__uint_as_float(bits[h]) * prescale));
}

// 8 elements per thread: code = E4M3(fp32(fp32(x * prescale) * 2^-e[h]))
template <int D>
__global__ __launch_bounds__(256) void quant_kernel(const uint16_t* __restrict__ x, size_t n8, int H,
                                                    const int* __restrict__ fexp, float prescale,
                                                    uint8_t* __restrict__ codes) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n8) return;
  const int h = static_cast<int>((i / (D / 8)) % H);
  const int ne = -fexp[h];
  const uint4 val = *reinterpret_cast<const uint4*>(x + 8 * i);
  const uint32_t wv[4] = {val.x, val.y, val.z, val.w};
  float y[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const uint32_t bits = (e & 1) ? (wv[e >> 1] & 0xffff0000u) : (wv[e >> 1] << 16);
    y[e] = __builtin_ldexpf(__uint_as_float(bits) * prescale, ne);  // one fp32 rounding, exact scaling
  }
  *reinterpret_cast<uint2*>(codes + 8 * i) = make_uint2(e4m3x4(y[0], y[1], y[2], y[3]), e4m3x4(y[4], y[5], y[6], y[7]));
}

// ============================================================ launchers
template <int D>
static hipError_t prep_d(const uint16_t* k, const uint16_t* v, int F, int N, int H, uint16_t* vt,
                         float* G, float* B, int grams, uint8_t* vt8, const int* vexp, hipStream_t st) {
  hipLaunchKernelGGL(prep_kernel<D>, dim3(F, H), dim3(512), 0, st, k, v, F, N, H, vt, G, B, grams, vt8, vexp);
  return hipGetLastError();
}

hipError_t launch_prep(const uint16_t* k, const uint16_t* v, int F, int N, int H, int D,
                       uint16_t* vt, float* G, float* B, int grams, hipStream_t st, uint8_t* vt8,
                       const int* vexp) {
  switch (D) {
    case 32: return prep_d<32>(k, v, F, N, H, vt, G, B, grams, vt8, vexp, st);
    case 64: return prep_d<64>(k, v, F, N, H, vt, G, B, grams, vt8, vexp, st);
    case 128: return prep_d<128>(k, v, F, N, H, vt, G, B, grams, vt8, vexp, st);
  }
  return hipErrorInvalidValue;
}

void attn_split_plan(int F, int* nsplit, int* fs) {
  // anchor query frames see all F key frames; slice them into pieces of about
  // the length of an interior chunk's key list (17 frames) for load balance
  int ns = (F + 14) / 15;
  if (ns < 1) ns = 1;
  int f = (F + ns - 1) / ns;
  *fs = f;
  *nsplit = (F + f - 1) / f;
}

template <typename KernelFn>
static hipError_t attn_launch(KernelFn fn, int lds, std::atomic<unsigned long long>* attr_done, AttnArgs a, hipStream_t st,
                              int threads, bool queue = false) {
  a.bq = 32 * (threads / 64);
  return attn_launch_items(fn, lds, attr_done, a, st, threads, queue);
}

// fp32 I/O: the register-staged kernel; bf16 and fp8: the direct-to-LDS kernel
template <int D>
static hipError_t attn_f32(const AttnArgs& a, hipStream_t st) {
  static std::atomic<unsigned long long> done{0};
  return attn_launch(&attn_kernel<D, 0>, 2 * AttnCfg<D, 0>::STAGE, &done, a, st, 256);
}
template <int D, int PREC>
static hipError_t attn_lds(const AttnArgs& a, hipStream_t st, bool split) {
  // the tile stages, then one word that hands a queued item to every wave
  constexpr int lds = kLdsStages * LdsCfg<D, PREC>::STAGE + 16;
  if constexpr (PREC == 3) {
    // fp8 P.V: the plain layer only (no extra tokens, no split output), by the
    // two-group kernel (4 LDS stages, 8 waves)
    if (split || a.T > 0) return hipErrorInvalidValue;
    static std::atomic<unsigned long long> done8{0};
    return attn_launch(&attn_pp_kernel<D>, 4 * LdsCfg<D, PREC>::STAGE + 16, &done8, a, st, 512, true);
  } else {
  if constexpr (D == 128) {
    // opt-in: the 64-queries-per-wave kernel (half the LDS reads per MFMA, one
    // wave per SIMD); slower than this one on the measured workloads
    if (!split && a.T == 0 && attn_w64_requested()) return launch_attn_w64(PREC, a, st);
  }
  if (split) {   // (no extra tokens in this form)
    static std::atomic<unsigned long long> done_s{0};
    return attn_launch(&attn_lds_kernel<D, PREC, kLdsWaves, false, true>, lds, &done_s, a, st, 64 * kLdsWaves, true);
  }
  if (a.T > 0) {
    // the split items, and the chunk items over the extra tokens' keys (state to
    // px); then the chunk items' video pass from that state
    static std::atomic<unsigned long long> done_x{0}, done_i{0};
    hipError_t e = attn_launch(&attn_lds_kernel<D, PREC, kLdsWaves, true, false>, lds, &done_x, a, st,
                               64 * kLdsWaves);
    if (e != hipSuccess) return e;
    AttnArgs b = a;
    b.na = 0;                // chunk items only
    b.T = 0;
    b.nbx = 0;
    return attn_launch(&attn_lds_kernel<D, PREC, kLdsWaves, false, false, true>, lds, &done_i, b, st,
                       64 * kLdsWaves, true);
  }
  static std::atomic<unsigned long long> done{0};
  return attn_launch(&attn_lds_kernel<D, PREC, kLdsWaves, false, false>, lds, &done, a, st, 64 * kLdsWaves, true);
  }
}

hipError_t launch_attn(int prec, const void* q, const void* k, const void* v, const uint16_t* vt,
                       const uint8_t* q8, const uint8_t* k8, const int* fexp, int F, int N, int H,
                       int D, void* O, float* part_O, float* part_ml, const uint16_t* W,
                       int T, const uint16_t* vtx, int split, float* px, int* qctr, hipStream_t st) {
  AttnArgs a;
  a.qctr = qctr;
  a.q = q; a.k = k; a.v = v; a.vt = vt; a.q8 = q8; a.k8 = k8; a.fexp = fexp;
  a.O = O; a.part_O = part_O; a.part_ml = part_ml;
  a.W = W;
  a.T = T;
  a.nbx = (T + BK - 1) / BK;
  a.vtx = vtx;
  a.px = px;
  // the fp32 kernel has neither the fused readout nor extra tokens
  if (prec == 0 && (W != nullptr || T != 0)) return hipErrorInvalidValue;
  if (T < 0 || (T > 0 && (vtx == nullptr || px == nullptr))) return hipErrorInvalidValue;
  // split output: the readout weights are needed, and no extra tokens
  if (split && (W == nullptr || T != 0 || prec == 0)) return hipErrorInvalidValue;
  a.F = F; a.N = N; a.H = H;
  attn_split_plan(F, &a.nsplit, &a.fs);
  a.na = F >= 2 ? 2 : 1;
  a.scale_log2 = softmax_temperature_log2(D);
  if (prec == 0) {
    if (D == 32) return attn_f32<32>(a, st);
    if (D == 64) return attn_f32<64>(a, st);
    if (D == 128) return attn_f32<128>(a, st);
  } else if (prec == 1) {
    if (D == 32) return attn_lds<32, 1>(a, st, split != 0);
    if (D == 64) return attn_lds<64, 1>(a, st, split != 0);
    if (D == 128) return attn_lds<128, 1>(a, st, split != 0);
  } else if (prec == 2) {
    if (D == 64) return attn_lds<64, 2>(a, st, split != 0);
    if (D == 128) return attn_lds<128, 2>(a, st, split != 0);
  } else if (prec == 3) {
    if (D == 64) return attn_lds<64, 3>(a, st, split != 0);
    if (D == 128) return attn_lds<128, 3>(a, st, split != 0);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_combine(int prec, const float* part_O, const float* part_ml, int F, int N, int T,
                          int H, int D, void* O, int split, hipStream_t st) {
  if (split && prec == 0) return hipErrorInvalidValue;
  const int ostride = (split ? 2 : 1) * H * D;
  int nsplit, fs;
  attn_split_plan(F, &nsplit, &fs);
  const int na = F >= 2 ? 2 : 1;
  const size_t threads = (size_t)H * ((size_t)na * N + T) * (D / 4);
  const dim3 grid((unsigned)((threads + 255) / 256));
#define VDN_COMB(DD)                                                                                   \
  if (D == DD) {                                                                                       \
    if (prec == 0)                                                                                     \
      hipLaunchKernelGGL((combine_kernel<DD, true>), grid, dim3(256), 0, st, part_O, part_ml, F, N, T, \
                         H, na, nsplit, O, ostride);                                                   \
    else                                                                                               \
      hipLaunchKernelGGL((combine_kernel<DD, false>), grid, dim3(256), 0, st, part_O, part_ml, F, N,   \
                         T, H, na, nsplit, O, ostride);                                                \
    return hipGetLastError();                                                                          \
  }
  VDN_COMB(32) VDN_COMB(64) VDN_COMB(128)
#undef VDN_COMB
  return hipErrorInvalidValue;
}

hipError_t launch_fp8_scale(const uint16_t* x, int F, int N, int H, int D, float prescale, int* fexp,
                            hipStream_t st) {
  const size_t ntok = (size_t)F * N;
  uint32_t* bits = reinterpret_cast<uint32_t*>(fexp);
  hipLaunchKernelGGL(fill_u32_kernel, dim3((H + 255) / 256), dim3(256), 0, st, bits, H, 0u);
  const dim3 g1((unsigned)((ntok + 1023) / 1024), H);
  switch (D) {
    case 64: hipLaunchKernelGGL(amax_kernel<64>, g1, dim3(256), 0, st, x, ntok, H, bits); break;
    case 128: hipLaunchKernelGGL(amax_kernel<128>, g1, dim3(256), 0, st, x, ntok, H, bits); break;
    default: return hipErrorInvalidValue;
  }
  hipLaunchKernelGGL(fp8_exp_kernel, dim3((H + 63) / 64), dim3(64), 0, st, bits, H, prescale);
  return hipGetLastError();
}

hipError_t launch_fp8_quant(const uint16_t* x, int F, int N, int H, int D, float prescale, uint8_t* codes,
                            int* fexp, hipStream_t st) {
  hipError_t e = launch_fp8_scale(x, F, N, H, D, prescale, fexp, st);
  if (e != hipSuccess) return e;
  const size_t n8 = (size_t)F * N * H * D / 8;
  const dim3 g2((unsigned)((n8 + 255) / 256));
  if (D == 64) hipLaunchKernelGGL(quant_kernel<64>, g2, dim3(256), 0, st, x, n8, H, fexp, prescale, codes);
  else hipLaunchKernelGGL(quant_kernel<128>, g2, dim3(256), 0, st, x, n8, H, fexp, prescale, codes);
  return hipGetLastError();
}

}  // namespace vdn
