// Output projections of the two branches, as one bf16 GEMM on the matrix cores:
//   Y[M, N] = A[M, K] B[N, K]^T,   fp32 accumulation, bf16 out,
// with A = [O_soft | g (.) O_lin] per token (K = 2 H d) and B = [W_s | W_l]
// (arXiv abstract page, Abstract; ananclaw note, section 一、方法拆解: separate
// output projections of the two branches, learnable gates between them).
//
// Workgroup tile 256 (M) x 256 (N), 8 waves, K in steps of 64.  Both operand tiles
// go global -> LDS by 16-byte direct loads (no staging registers) into rows with
// one 16-byte padding chunk each (144-byte pitch), so 16 consecutive rows read at
// one chunk hit 16 distinct bank groups; two LDS stages, one barrier per step,
// placed before the step's last 16-wide sub-step.  Inside a step the operand
// fragments of sub-step s + 1 are read while the MFMAs of sub-step s run; after
// the barrier the next step's first fragments are read, and the step after it
// starts loading into the stage just freed, during the last sub-step's MFMAs
// (4 % faster than a barrier at the end of the step, after which every wave
// waits for its first fragments with the matrix core idle).
// Each wave computes Y^T for 64 rows of B (N) x 128 rows of A (M): the MFMA's A
// operand is a 32-row block of B, its B operand a 32-row block of A, so each lane
// ends with 4 consecutive output columns (n) of one output row (m).  The tile
// goes back through LDS and leaves as whole 512-byte rows, 16 bytes a lane (3 %
// faster than each lane storing its 8-byte pieces).  Blocks walk the tile list
// XCD-contiguously, in groups of 4 M tiles x all N tiles (m fastest inside a
// group), so the ~32 tiles an XCD runs at once cover about 4 M x 8 N tiles and
// share its L2 for both operands' rows (3 % faster than all N tiles of one M tile
// in turn, which re-fetches every B tile for each M tile).
#include <hip/hip_runtime.h>

#include <cstdint>

#include "common.h"
#include "kernels.h"

namespace vdn {

namespace {

constexpr int PJ_TM = 256, PJ_TN = 256, PJ_TK = 64;   // workgroup tile
constexpr int PJ_NW = 8;                               // waves per workgroup
constexpr int PJ_PITCH = 16 * 9;                       // LDS row: 8 data chunks + 1 pad
constexpr int PJ_OPER = 256 * PJ_PITCH;                // one operand tile in LDS (36 KiB)
constexpr int PJ_STAGE = 2 * PJ_OPER;                  // A tile + B tile
constexpr int PJ_LOADS = 256 * 9 / 64;                 // 36 wave-wide direct loads per operand tile
constexpr int PJ_LX = (PJ_LOADS + PJ_NW - 1) / PJ_NW;  // per wave (the last partly idle)
constexpr int PJ_LDS = 2 * PJ_STAGE;                   // 144 KiB

// (the launcher checks K % 64 == 0, N % 8 == 0, M, N, K > 0 and 2*K*256 < 2^32)
// Next tile from the queues (one thread per workgroup), or -1 when all are empty:
// queue x holds the x-th of 8 contiguous runs of the tile list, qctr[x] its cursor
// (zero at launch).  A workgroup takes from its own XCD's queue first, then from
// the next non-empty one, so an XCD that runs ahead takes tiles from the others.
__device__ inline int acquire_tile(int* qctr, int T) {
  const int q8 = T >> 3, m8 = T & 7;
  const int x = __builtin_amdgcn_s_getreg((15 << 11) | 20) & 7;   // HW_REG_XCC_ID
  for (int k = 0; k < 8; ++k) {
    const int y = (x + k) & 7;
    const int n = q8 + (y < m8 ? 1 : 0);
    if (n == 0 || __hip_atomic_load(qctr + y, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= n) continue;
    const int i = __hip_atomic_fetch_add(qctr + y, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (i < n) return y * q8 + min(y, m8) + i;
  }
  return -1;
}

__global__ __launch_bounds__(64 * PJ_NW, 1) void proj_kernel(const uint16_t* __restrict__ A,
                                                             const uint16_t* __restrict__ B, int M, int N,
                                                             int K, uint16_t* __restrict__ Y, int* qctr) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int j = lane & 31, hf = lane >> 5;

  // this workgroup's tile: the XCDs take contiguous runs of the tile list, from
  // the queues when qctr is set (the LDS word after the stages hands the tile to
  // every wave), else the blocks one XCD receives (every 8th) take the run
  const int tn_count = (N + PJ_TN - 1) / PJ_TN, tm_count = (M + PJ_TM - 1) / PJ_TM;
  const int T = tm_count * tn_count;
  int t;
  if (qctr != nullptr) {
    int* slot = reinterpret_cast<int*>(smem + PJ_LDS);
    if (tid == 0) *slot = acquire_tile(qctr, T);
    __syncthreads();
    t = __builtin_amdgcn_readfirstlane(*slot);
    if (t < 0) return;       // every queue empty (the grid's spare workgroups)
  } else {
    const int b = blockIdx.x, q8 = T >> 3, m8 = T & 7, r = b & 7;
    t = r * q8 + min(r, m8) + (b >> 3);
  }
  // grouped order: G M tiles x all N tiles per group, m fastest inside a group
  // (the last group takes the M tiles left over)
  constexpr int G = 4;
  const int grp = t / (G * tn_count), gm0 = G * grp;
  const int gsz = min(G, tm_count - gm0);
  const int tg = t - grp * G * tn_count;              // position inside the group
  // (the division runs on the vector unit; the tile origin is block-uniform, and
  // the buffer resources built from it must live in scalar registers)
  const int m0 = __builtin_amdgcn_readfirstlane(PJ_TM * (gm0 + tg % gsz));
  const int n0 = __builtin_amdgcn_readfirstlane(PJ_TN * (tg / gsz));
  const int wn = w & 3, wm = w >> 2;                   // wave: B rows 64 wn.., A rows 128 wm..
  // waves w and w + 4 share a SIMD: a fixed higher priority for one of them lets
  // it run ahead rather than the two contending at every step (2 % faster)
  if (w >= 4) __builtin_amdgcn_s_setprio(1);

  // direct loads: load x of this wave fills LDS chunk q = 64 (x NW + w) + lane of
  // an operand tile, i.e. row q / 9, chunk q % 9 (the padding chunk re-reads the
  // row's last chunk)
  uint32_t off[PJ_LX];
#pragma unroll
  for (int x = 0; x < PJ_LX; ++x) {
    const int q = 64 * (x * PJ_NW + w) + lane;
    const int row = q / 9, c = min(q % 9, 7);
    off[x] = (uint32_t)row * (uint32_t)(2 * K) + 16u * c;
  }
  // rows past M (N) read zeros: a tile's resource ends right after its last valid
  // row's 128 bytes of the current K step
  const int va = min(PJ_TM, M - m0), vb = min(PJ_TN, N - n0);
  const uint32_t a_bytes = (uint32_t)(va - 1) * (uint32_t)(2 * K) + 2 * PJ_TK;
  const uint32_t b_bytes = (uint32_t)(vb - 1) * (uint32_t)(2 * K) + 2 * PJ_TK;
  const uint16_t* a_base = A + (size_t)m0 * K;
  const uint16_t* b_base = B + (size_t)n0 * K;
  auto issue = [&](int stage, int kk, int x0, int x1) {
    unsigned char* sb = smem + stage * PJ_STAGE;
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(a_base + (size_t)kk * PJ_TK, a_bytes);
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(b_base + (size_t)kk * PJ_TK, b_bytes);
#pragma unroll
    for (int x = 0; x < PJ_LX; ++x) {
      if (x < x0 || x >= x1) continue;
      if (x * PJ_NW + w >= PJ_LOADS) break;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_void_ptr)(sb + 1024 * (x * PJ_NW + w)), 16, off[x], 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_void_ptr)(sb + PJ_OPER + 1024 * (x * PJ_NW + w)), 16, off[x],
                                               0, 0, 0);
    }
  };

  floatx16 acc[2][4];
#pragma unroll
  for (int nb = 0; nb < 2; ++nb)
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) acc[nb][mb] = floatx16{};

  const int nk = K / PJ_TK;
  constexpr int NS = PJ_TK / 16;                       // 16-wide K sub-steps per step
  // loads of a step issued right after the barrier two steps before, the rest in
  // the first sub-step of the step before (measured best of 0-5 after the barrier,
  // and of spreading the rest over two sub-steps)
  constexpr int LH = PJ_LX / 2;
  // steps 0 and 1 first (the loop loads step kk + 2 once step kk's stage is free)
  issue(0, 0, 0, PJ_LX);
  if (nk > 1) issue(1, 1, 0, PJ_LX);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  bf16x8 wf[2][2], af[2][4];
  auto read = [&](const unsigned char* sa, int s, int buf) {
    const unsigned char* sw = sa + PJ_OPER;
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
      wf[buf][nb] = *reinterpret_cast<const bf16x8*>(sw + (64 * wn + 32 * nb + j) * PJ_PITCH + 16 * (2 * s + hf));
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
      af[buf][mb] = *reinterpret_cast<const bf16x8*>(sa + (128 * wm + 32 * mb + j) * PJ_PITCH + 16 * (2 * s + hf));
  };
  auto mfmas = [&](int buf) {
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) acc[nb][mb] = mfma_bf16(wf[buf][nb], af[buf][mb], acc[nb][mb]);
  };
  read(smem, 0, 0);
  // The step's barrier sits before its last sub-step: by then every fragment of
  // the step is read (the last sub-step's during the one before), so the barrier
  // frees the stage and publishes the next step's loads; the next step's first
  // fragments are then read, and step kk + 2's loads issued into the freed stage,
  // while the last sub-step's MFMAs run (a barrier after the last sub-step leaves
  // the matrix cores idle while all waves read their first fragments at once).
  for (int kk = 0; kk < nk; ++kk) {
    const unsigned char* sa = smem + (kk & 1) * PJ_STAGE;
#pragma unroll
    for (int s = 0; s < NS - 1; ++s) {
      __builtin_amdgcn_s_waitcnt(0xC07F);              // lgkmcnt(0): sub-step s's fragments
      read(sa, s + 1, (s + 1) & 1);
      // the rest of step kk + 1's loads (the first LH went out after the last barrier)
      if (s == 0 && kk >= 1 && kk + 1 < nk) issue((kk + 1) & 1, kk + 1, LH, PJ_LX);
      __builtin_amdgcn_sched_barrier(0);
      mfmas(s & 1);
      __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_s_waitcnt(0);   // this wave's last fragments read, its loads of step kk + 1 landed
    __syncthreads();                 // ... and every wave's
    if (kk + 2 < nk) issue(kk & 1, kk + 2, 0, LH);
    if (kk + 1 < nk) read(smem + ((kk + 1) & 1) * PJ_STAGE, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
    mfmas((NS - 1) & 1);
    __builtin_amdgcn_sched_barrier(0);
  }

  // the output tile goes through LDS (free after the last step's barrier) so that
  // it leaves as whole rows: lane (j, hf), element 4 g + e of block (nb, mb) is
  // tile row 128 wm + 32 mb + j, column 64 wn + 32 nb + 8 g + 4 hf + e
  constexpr int YP = 2 * PJ_TN + 16;                    // LDS pitch of an output row (bytes)
  static_assert(PJ_TM * YP <= PJ_LDS, "the output tile fits in LDS");
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const floatx16& c = acc[nb][mb];
        *reinterpret_cast<uint2*>(smem + (128 * wm + 32 * mb + j) * YP + 2 * (64 * wn + 32 * nb + 8 * g + 4 * hf)) =
            make_uint2(pack_bf16x2(c[4 * g + 0], c[4 * g + 1]), pack_bf16x2(c[4 * g + 2], c[4 * g + 3]));
      }
  __syncthreads();
  // wave w writes tile rows 32 w .. 32 w + 31, two per instruction, 16 bytes a lane
  const int cl = lane & 31, rh = lane >> 5;
#pragma unroll
  for (int x = 0; x < 16; ++x) {
    const int row = 32 * w + 2 * x + rh;
    const int m = m0 + row, n = n0 + 8 * cl;
    if (m < M && n < N)
      *reinterpret_cast<uint4*>(Y + (size_t)m * N + n) = *reinterpret_cast<const uint4*>(smem + row * YP + 16 * cl);
  }
}

}  // namespace

hipError_t launch_proj(const uint16_t* A, const uint16_t* B, int M, int N, int K, uint16_t* Y, hipStream_t st,
                       int* qctr) {
  if (M <= 0 || N <= 0 || K <= 0 || K % PJ_TK != 0 || N % 8 != 0) return hipErrorInvalidValue;
  if ((long long)PJ_TM * 2 * K >= (1LL << 32)) return hipErrorInvalidValue;   // 32-bit buffer offsets
  // the stages, then one word that hands a queued tile to every wave
  constexpr int lds = PJ_LDS + 16;
  static std::atomic<unsigned long long> attr_done{0};
  hipError_t e = set_max_lds_once(reinterpret_cast<const void*>(&proj_kernel), lds, &attr_done);
  if (e != hipSuccess) return e;
  const long long tiles = (long long)((M + PJ_TM - 1) / PJ_TM) * ((N + PJ_TN - 1) / PJ_TN);
  if (tiles > 0x7fffffff - (0x7fffffff >> 3) - 128) return hipErrorInvalidValue;
  long long grid = tiles;
  if (qctr != nullptr) {
    // an eighth more workgroups than tiles: an XCD that runs ahead can take tiles
    // from the others' queues; the spare workgroups find every queue empty
    e = launch_fill_u32(reinterpret_cast<uint32_t*>(qctr), 8, 0u, st);
    if (e != hipSuccess) return e;
    grid = tiles + (tiles / 8 + 64 + 7) / 8 * 8;
  }
  hipLaunchKernelGGL(proj_kernel, dim3((unsigned)grid), dim3(64 * PJ_NW), lds, st, A, B, M, N, K, Y, qctr);
  return hipGetLastError();
}

}  // namespace vdn
