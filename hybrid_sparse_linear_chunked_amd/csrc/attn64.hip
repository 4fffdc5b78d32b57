// Softmax branch of the VDN hybrid layer at d = 128 (gfx950), with 64 queries per
// wave: the windowed + anchored softmax attention of the sd114.wiki article
// "VDN-Minimax-H3 ...", section 双向滑动窗口Softmax分支 (a query frame of chunk c
// attends to every token of chunks c-1, c, c+1 and of the first and last frame; the
// first and last frame attend to every frame), with the linear branch's readout
// and the gated merge in the epilogue (besthub article "VDN-H3 Generates
// 14-Second 768p Video ...", section Hybrid Attention Architecture).
//
// The tile loop's MFMAs are placed by hand (asm statements) so that each operand
// lives in the register file it needs: see the notes above Mma below.
#include "attn_common.h"

namespace vdn {

// ---------------------------------------------------------------- hand-placed MFMAs
// Every MFMA of the tile loop is an asm statement, so that the register classes
// are fixed: the scores (MFMA results the softmax reads) in VGPRs, the P.V
// accumulators in accumulation registers (AGPRs), which no VALU instruction
// touches inside the loop.  This matters for overlap: measured on gfx950, a wave's
// VALU instructions run in the shadow of its own in-flight MFMA when that MFMA's
// accumulators are AGPRs, and wait for it when they are VGPRs; so the softmax
// work is placed beside the P.V MFMAs only.  The compiler sees these as opaque
// instructions, so the wait states an MFMA result needs before a VALU access are
// inserted by hand (score_fence, acc_fence: 32 / 64 cycles, more than the 8-pass
// bf16 and 16-pass fp8 MFMAs need); operands written by the VALU or by LDS reads
// are produced well before their MFMA, behind explicit waits.
// Score MFMAs S = K Q^T (+ c) (fp8: each product scaled by the E8M0 bytes sk, sq):
// the Q fragment qi (query block x, reduction step
// st: qi = steps * x + st) is pinned to accumulation registers from a128 on, read
// there as the B operand (an in-out operand of the asm, so that the value stays
// in those registers between uses); the scores land in VGPRs.  FIRST starts from
// c (the -m start), otherwise the MFMA accumulates.
#define VDN_QK(T, QI, LO, HI)                                                                       \
  case QI:                                                                                           \
    if (FIRST)                                                                                       \
      asm volatile(VDN_QK_OP(T) " %0, %2, %1, %3" VDN_QK_SCALES(T)                                   \
                   : "=&v"(acc), "+{a[" #LO ":" #HI "]}"(q)                                          \
                   : "v"(k), "v"(c), "v"(sk), "v"(sq));                                              \
    else                                                                                             \
      asm volatile(VDN_QK_OP(T) " %0, %2, %1, %0" VDN_QK_SCALES(T)                                   \
                   : "+v"(acc), "+{a[" #LO ":" #HI "]}"(q)                                           \
                   : "v"(k), "v"(c), "v"(sk), "v"(sq));                                              \
    break;
#define VDN_QK_OP(T) VDN_QK_OP_##T
#define VDN_QK_OP_bf16 "v_mfma_f32_32x32x16_bf16"
#define VDN_QK_OP_f8f6f4 "v_mfma_scale_f32_32x32x64_f8f6f4"
// fp8: E8M0 scale bytes of K (operand A) and Q (operand B), low byte of each register
#define VDN_QK_SCALES(T) VDN_QK_SCALES_##T
#define VDN_QK_SCALES_bf16 ""
#define VDN_QK_SCALES_f8f6f4 ", %4, %5 op_sel_hi:[0,0,0]"
template <bool FP8>
struct Mma;
template <>
struct Mma<false> {
  using KFrag = bf16x8;
  using QFrag = bf16x8;
  template <bool FIRST>
  __device__ __forceinline__ static void qk(int qi, floatx16& acc, const KFrag& k, QFrag& q,
                                            const floatx16& c, int sk, int sq) {
    switch (qi) {
      VDN_QK(bf16, 0, 128, 131)
      VDN_QK(bf16, 1, 132, 135)
      VDN_QK(bf16, 2, 136, 139)
      VDN_QK(bf16, 3, 140, 143)
      VDN_QK(bf16, 4, 144, 147)
      VDN_QK(bf16, 5, 148, 151)
      VDN_QK(bf16, 6, 152, 155)
      VDN_QK(bf16, 7, 156, 159)
      VDN_QK(bf16, 8, 160, 163)
      VDN_QK(bf16, 9, 164, 167)
      VDN_QK(bf16, 10, 168, 171)
      VDN_QK(bf16, 11, 172, 175)
      VDN_QK(bf16, 12, 176, 179)
      VDN_QK(bf16, 13, 180, 183)
      VDN_QK(bf16, 14, 184, 187)
      VDN_QK(bf16, 15, 188, 191)
    }
  }
};
template <>
struct Mma<true> {
  using KFrag = intx8;
  using QFrag = intx8;
  template <bool FIRST>
  __device__ __forceinline__ static void qk(int qi, floatx16& acc, const KFrag& k, QFrag& q,
                                            const floatx16& c, int sk, int sq) {
    switch (qi) {
      VDN_QK(f8f6f4, 0, 128, 135)
      VDN_QK(f8f6f4, 1, 136, 143)
      VDN_QK(f8f6f4, 2, 144, 151)
      VDN_QK(f8f6f4, 3, 152, 159)
    }
  }
};
#undef VDN_QK
#undef VDN_QK_OP
#undef VDN_QK_OP_bf16
#undef VDN_QK_OP_f8f6f4
#undef VDN_QK_SCALES
#undef VDN_QK_SCALES_bf16
#undef VDN_QK_SCALES_f8f6f4
// Places the Q fragments in their pinned registers with the wait states an MFMA
// needs after they are written there (the copies happen before this statement)
__device__ __forceinline__ void q_fence(bf16x8 (&q)[2][8]) {
  asm volatile("s_nop 7"
               : "+{a[128:131]}"(q[0][0]), "+{a[132:135]}"(q[0][1]),
                 "+{a[136:139]}"(q[0][2]), "+{a[140:143]}"(q[0][3]),
                 "+{a[144:147]}"(q[0][4]), "+{a[148:151]}"(q[0][5]),
                 "+{a[152:155]}"(q[0][6]), "+{a[156:159]}"(q[0][7]),
                 "+{a[160:163]}"(q[1][0]), "+{a[164:167]}"(q[1][1]),
                 "+{a[168:171]}"(q[1][2]), "+{a[172:175]}"(q[1][3]),
                 "+{a[176:179]}"(q[1][4]), "+{a[180:183]}"(q[1][5]),
                 "+{a[184:187]}"(q[1][6]), "+{a[188:191]}"(q[1][7]));
}
__device__ __forceinline__ void q_fence(intx8 (&q)[2][2]) {
  asm volatile("s_nop 7" : "+{a[128:135]}"(q[0][0]), "+{a[136:143]}"(q[0][1]), "+{a[144:151]}"(q[1][0]), "+{a[152:159]}"(q[1][1]));
}

// O^T += V^T P^T for output block b (0..7), its accumulators pinned to
// a[16 b .. 16 b + 15]: every access to the output accumulators inside the tile
// loop names these registers, so they never move (see rescale_o_pinned)
#define VDN_PV(B, LO, HI)                                                                  \
  case B:                                                                                  \
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+{a[" #LO ":" #HI "]}"(acc) \
                 : "v"(v), "v"(p));                                                        \
    break;
__device__ __forceinline__ void mma_pv(int b, floatx16& acc, const bf16x8& v, const bf16x8& p) {
  switch (b) {
    VDN_PV(0, 0, 15)
    VDN_PV(1, 16, 31)
    VDN_PV(2, 32, 47)
    VDN_PV(3, 48, 63)
    VDN_PV(4, 64, 79)
    VDN_PV(5, 80, 95)
    VDN_PV(6, 96, 111)
    VDN_PV(7, 112, 127)
  }
}
#undef VDN_PV
// s_waitcnt vmcnt(N) alone: all but this wave's N most recent vector memory
// loads have completed (expcnt, lgkmcnt at their maxima)
template <int N>
__device__ inline void vm_wait_all_but() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// wait states between the last score MFMA and VALU reads of the scores
__device__ inline void score_fence2(floatx16 (&s)[2]) {
  asm volatile("s_nop 15\n\ts_nop 15" : "+v"(s[0]), "+v"(s[1]));
}
// wait states between the last P.V MFMA and VALU access to the accumulators
__device__ inline void acc_fence(floatx16 (&o)[2][4]) {
  asm volatile("s_nop 15\n\ts_nop 15\n\ts_nop 15\n\ts_nop 15"
               : "+a"(o[0][0]), "+a"(o[0][1]), "+a"(o[0][2]), "+a"(o[0][3]), "+a"(o[1][0]), "+a"(o[1][1]),
                 "+a"(o[1][2]), "+a"(o[1][3]));
}

// O *= alpha (blocks 0-3: alpha0, 4-7: alpha1) where `doit` (wave-uniform) is set,
// in place in the pinned accumulators a0..a127.  The branch is inside the asm
// statement: a conditional update written in C++ makes the register allocator
// split the accumulators' live ranges across the two register files.  The taken
// path starts with the wait states between the P.V MFMAs and reads of their
// accumulators, and ends with those before an MFMA reads them again.
#define VDN_RS1(al, i) "v_accvgpr_read_b32 %[t], a" #i "\n\tv_mul_f32 %[t], %[t], %[" #al "]\n\tv_accvgpr_write_b32 a" #i ", %[t]\n\t"
#define VDN_RS16(al, i0, i1, i2, i3, i4, i5, i6, i7, i8, i9, i10, i11, i12, i13, i14, i15)                   \
  VDN_RS1(al, i0) VDN_RS1(al, i1) VDN_RS1(al, i2) VDN_RS1(al, i3) VDN_RS1(al, i4) VDN_RS1(al, i5)               \
  VDN_RS1(al, i6) VDN_RS1(al, i7) VDN_RS1(al, i8) VDN_RS1(al, i9) VDN_RS1(al, i10) VDN_RS1(al, i11)             \
  VDN_RS1(al, i12) VDN_RS1(al, i13) VDN_RS1(al, i14) VDN_RS1(al, i15)
__device__ __forceinline__ void rescale_o_pinned(floatx16 (&o)[2][4], float alpha0, float alpha1, int doit) {
  float t;
  asm volatile("s_cmp_eq_u32 %[c], 0\n\ts_cbranch_scc1 1f\n\t"
               "s_nop 15\n\ts_nop 15\n\ts_nop 15\n\ts_nop 15\n\t"
               VDN_RS16(al0, 0,1,2,3,4,5,6,7,8,9,10,11,12,13,14,15)
               VDN_RS16(al0, 16,17,18,19,20,21,22,23,24,25,26,27,28,29,30,31)
               VDN_RS16(al0, 32,33,34,35,36,37,38,39,40,41,42,43,44,45,46,47)
               VDN_RS16(al0, 48,49,50,51,52,53,54,55,56,57,58,59,60,61,62,63)
               VDN_RS16(al1, 64,65,66,67,68,69,70,71,72,73,74,75,76,77,78,79)
               VDN_RS16(al1, 80,81,82,83,84,85,86,87,88,89,90,91,92,93,94,95)
               VDN_RS16(al1, 96,97,98,99,100,101,102,103,104,105,106,107,108,109,110,111)
               VDN_RS16(al1, 112,113,114,115,116,117,118,119,120,121,122,123,124,125,126,127)
               "s_nop 4\n1:"
               : "+{a[0:15]}"(o[0][0]), "+{a[16:31]}"(o[0][1]), "+{a[32:47]}"(o[0][2]), "+{a[48:63]}"(o[0][3]),
                 "+{a[64:79]}"(o[1][0]), "+{a[80:95]}"(o[1][1]), "+{a[96:111]}"(o[1][2]),
                 "+{a[112:127]}"(o[1][3]), [t] "=&v"(t)
               : [al0] "v"(alpha0), [al1] "v"(alpha1), [c] "s"(doit)
               : "scc");
}
#undef VDN_RS16
#undef VDN_RS1

// ============================================================ attention, 64 queries per wave
// The bf16 / fp8 video path at d = 128 with twice the queries per wave: each K and
// V^T operand fragment read from LDS feeds two MFMAs (one per 32-query block), so
// a tile costs half the LDS reads per MFMA of attn_lds_kernel.  Four waves of 64
// queries (the same 256-query work items), one wave per SIMD with up to 512
// registers: the output accumulators (128) and the Q fragments (64 at bf16) sit
// pinned in AGPRs, the scores, probabilities and operand stream in VGPRs.  With
// one wave per SIMD the matrix core is kept busy from within the wave: the loop
// runs over half-tiles of 32 keys, and one step (see `step`) issues the Q.K^T
// MFMAs of half-tile hh + 1 (phase A) and then the P.V MFMAs of half-tile hh with
// the softmax of hh + 1 beside them (phase B), over four LDS stages (tile t + 3
// loads while t and t + 1 are read and t + 2 lands), one barrier per tile.
// Arithmetic per element is that of attn_lds_kernel (scores start at -m, lazy max
// in log2 units, P rounded to bf16 once for P.V and the row sum).
//
// Measured on MI355X (768p workload, bf16): the LDS reads per MFMA halve (0.50
// LDS instructions per MFMA) and the clock holds higher (2.2 vs 1.9 GHz), but
// with one wave per SIMD the waits on LDS reads, tile loads and the barrier are
// no longer covered by a second wave: the matrix core is busy 46 % of the time
// against 66 % for attn_lds_kernel, and the kernel takes 296 ms against 261 ms.
// It is therefore opt-in (attn_w64_requested).
template <int D, int PREC>
__global__ __launch_bounds__(256, 1) void attn_w64_kernel(AttnArgs a) {
  static_assert(D == 128, "fences and fragment counts assume d = 128");
  using Cfg = LdsCfg<D, PREC>;
  constexpr bool FP8 = Cfg::FP8;
  using M = Mma<FP8>;
  constexpr int NW = 4;                 // waves per workgroup
  constexpr int NX = 2;                 // 32-query blocks per wave
  constexpr int NDB = D / 32;
  constexpr int NSTG = 4;               // LDS stages: tiles t .. t + 3
  constexpr int AHEAD = 3;              // tiles loaded ahead of the one in use
  constexpr int QS = Cfg::QSTEPS;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];

  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int j = lane & 31, hf = lane >> 5;
  const int F = a.F, N = a.N, H = a.H;
  const size_t rs = (size_t)H * D;
  const int nb = (N + BK - 1) / BK;
  const Item it = uniform_item(decode_item(a));
  const int h = it.h;
  const int ntiles = it.nslots * nb;

  // ---- Q operand fragments of the two query blocks (rows 64 w + 32 x + j)
  bool qvalid[NX];
  typename M::QFrag qf[NX][QS];
#pragma unroll
  for (int x = 0; x < NX; ++x) {
    const int qi = 64 * w + 32 * x + j;
    qvalid[x] = qi < it.q_rows;
    const size_t qoff = (size_t)(it.q_tok0 + qi) * rs + (size_t)h * D;
    if constexpr (FP8) {
#pragma unroll
      for (int s = 0; s < QS; ++s) {
        if (qvalid[x]) {
          const uint4* p = reinterpret_cast<const uint4*>(a.q8 + qoff + 64 * s + 32 * hf);
          const uint4 x0 = p[0], x1 = p[1];
          qf[x][s] = intx8{(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w, (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
        } else {
          qf[x][s] = intx8{};
        }
      }
    } else {
      const uint16_t* q = static_cast<const uint16_t*>(a.q);
      // the Q operand carries log2(e)/sqrt(d) (rounded once to bf16)
#pragma unroll
      for (int s = 0; s < QS; ++s) {
        bf16x8 v = qvalid[x] ? *reinterpret_cast<const bf16x8*>(q + qoff + 16 * s + 8 * hf) : bf16x8{};
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = (__bf16)((float)v[e] * a.scale_log2);
        qf[x][s] = v;
      }
    }
  }
  q_fence(qf);
  // fp8: the q codes carry log2(e)/sqrt(d); the power-of-two scales of the q and
  // k codes are the score MFMAs' E8M0 operand scales, so every score arrives in
  // log2 units, as at bf16
  const int sq = FP8 ? a.fexp[h] + 127 : 0, sk = FP8 ? a.fexp[H + h] + 127 : 0;

  // ---- global -> LDS tile loads (the padded layout of attn_lds_kernel, four
  // waves).  Every wave issues the same number of loads per tile, with no branch:
  // a wave's surplus loads (a tile is 17 K + 18 V^T wave-wide loads at bf16) and
  // every load of a tile past the item's end read out of range (zeros, no memory
  // access) into a 1 KiB pad after the stages.
  const unsigned char* kbase = FP8 ? reinterpret_cast<const unsigned char*>(a.k8)
                                   : static_cast<const unsigned char*>(a.k);
  auto frame_of = [&](int slot) {
    return it.mode == 0 ? it.k_f0 + slot : chunk_key_frame_sel(slot, it.wf, it.we, F);
  };
  constexpr int KX = (Cfg::K_INSTR + NW - 1) / NW, VX = (Cfg::V_INSTR + NW - 1) / NW;
  constexpr int PAD = NSTG * Cfg::STAGE;             // byte offset of the pad
  constexpr uint32_t OOB = 0x80000000u;               // past any buffer's end
  const size_t krs = rs * (FP8 ? 1 : 2);
  LaneOffsets<KX, VX> lo;
  uint32_t* koff = lo.koff;
  uint32_t* voff = lo.voff;
  int kdst[KX], vdst[VX];                             // LDS offsets in a stage (-1: surplus)
#pragma unroll
  for (int x = 0; x < KX; ++x) {
    const int ii = x * NW + w;
    const int q = 64 * ii + lane;
    const int row = q / (Cfg::KCH + 1), c = min(q % (Cfg::KCH + 1), Cfg::KCH - 1);
    const bool real = ii < Cfg::K_INSTR;
    koff[x] = real ? (uint32_t)(row * krs) + 16u * c : OOB;
    kdst[x] = real ? 1024 * ii : -1;
  }
#pragma unroll
  for (int x = 0; x < VX; ++x) {
    const int ii = x * NW + w;
    const int q = 64 * ii + lane;
    const int row = min(q / 9, D - 1), c = min(q % 9, 7);
    const bool real = ii < Cfg::V_INSTR;
    voff[x] = real ? (uint32_t)(row * 128 + 16 * c) : OOB;
    vdst[x] = real ? Cfg::K_BYTES + 1024 * ii : -1;
  }
  constexpr int LPT = KX + VX;
  // loads [x0, x1) of this wave's share of a tile (valid: the tile exists)
  auto issue_range = [&](int stage, int f, int b, bool valid, int x0, int x1) {
    const int nvalid = valid ? min(BK, N - BK * b) : 0;
    const unsigned char* kt = kbase + (((size_t)f * N + BK * b) * rs + (size_t)h * D) * (FP8 ? 1 : 2);
    const __amdgpu_buffer_rsrc_t krsrc = make_rsrc(kt, (uint32_t)(nvalid * krs));
#pragma unroll
    for (int x = 0; x < KX; ++x) {
      if (x < x0 || x >= x1) continue;
      const int dst = kdst[x] >= 0 ? stage * Cfg::STAGE + kdst[x] : PAD;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(krsrc, (lds_void_ptr)(smem + dst), 16, koff[x], 0, 0, 0);
    }
    const unsigned char* vsrc =
        reinterpret_cast<const unsigned char*>(a.vt + (((size_t)h * F + f) * nb + b) * (size_t)(D * BK));
    const __amdgpu_buffer_rsrc_t vrsrc = make_rsrc(vsrc, valid ? (uint32_t)(D * BK * 2) : 0u);
#pragma unroll
    for (int x = 0; x < VX; ++x) {
      if (KX + x < x0 || KX + x >= x1) continue;
      const int dst = vdst[x] >= 0 ? stage * Cfg::STAGE + vdst[x] : PAD;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(vrsrc, (lds_void_ptr)(smem + dst), 16, voff[x], 0, 0, 0);
    }
  };
  // load cursor (frame, 64-key block) of the next tile to load; past the item's
  // end it stays on the last frame (those loads read nothing)
  // (selects, no branch: a branch would split the tile loop's straight-line code)
  int ld_slot = 0, ld_b = 0, ld_f = frame_of(0);
  auto next_load = [&]() {
    const bool wrap = ld_b + 1 == nb;
    const int f_next = frame_of(min(ld_slot + 1, it.nslots - 1));
    ld_b = wrap ? 0 : ld_b + 1;
    ld_slot = wrap ? ld_slot + 1 : ld_slot;
    ld_f = wrap ? f_next : ld_f;
  };

  // ---- running state per query block (lane: query j of block x; m agrees
  // across the lane pair, l is a per-lane partial sum)
  floatx16 o[NX][NDB];
#pragma unroll
  for (int x = 0; x < NX; ++x)
#pragma unroll
    for (int db = 0; db < NDB; ++db) o[x][db] = floatx16{};
  float m_run[NX], l_run[NX];         // running max (log2 units), per-lane row-sum part
  // The score accumulators start at -m, so
  // the MFMAs deliver scores already shifted by the running max
  floatx16 nm[NX];
#pragma unroll
  for (int x = 0; x < NX; ++x) {
    m_run[x] = 0.f;
    l_run[x] = 0.f;
    nm[x] = floatx16{};
  }
  // a shifted score in log2 units (the MFMAs deliver log2 units at both precisions)
  auto lg = [&](float s) { return s; };
  auto set_nm = [&](int x) {
    const float v = -m_run[x];
#pragma unroll
    for (int r = 0; r < 16; ++r) nm[x][r] = v;
  };
  using KFrag = typename M::KFrag;

  // scores of keys past the frame's end to -inf (nvalid: valid keys of this
  // half-tile, may be <= 0), and the lane's maxima again
  auto mask_tail = [&](floatx16 (&s)[NX], int nvalid, float (&mx)[NX]) {
    asm volatile("");    // keeps this rare path a branch (not selects in every tile)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = 8 * (r >> 2) + 4 * hf + (r & 3);
      if (key >= nvalid) {
#pragma unroll
        for (int x = 0; x < NX; ++x) s[x][r] = -INFINITY;
      }
    }
#pragma unroll
    for (int x = 0; x < NX; ++x) {
      float v = s[x][0];
#pragma unroll
      for (int e = 1; e < 16; ++e) v = __builtin_fmaxf(v, s[x][e]);
      mx[x] = v;
    }
  };
  // Lazy raise of the running max by a half-tile's maxima mx (shifted scores,
  // MFMA units; see attn_lds_kernel): only where a shifted maximum passes kLazy
  // (log2 units) is m raised, l rescaled and the scores shifted down; the output
  // accumulators are rescaled later by alpha (returned; 1 if not raised), after the
  // P.V MFMAs in flight.  `first`: nothing accumulated yet, m is set to the
  // half-tile's maximum.
  auto raise = [&](floatx16 (&s)[NX], float (&mx)[NX], bool live, bool first, float (&alpha)[NX], int& resc) {
#pragma unroll
    for (int x = 0; x < NX; ++x) {
      alpha[x] = 1.f;
      if (live && (first || __any(lg(mx[x]) > kLazy))) {
        const float mp = lg(pair_max(mx[x]));
        const float dm = first ? mp : __builtin_fmaxf(mp, 0.f);
        if (!first) {
          alpha[x] = __builtin_amdgcn_exp2f(-dm);
          l_run[x] *= alpha[x];
          resc = 1;
        }
        m_run[x] += dm;
        const float ds = dm;
#pragma unroll
        for (int r = 0; r < 16; ++r) s[x][r] -= ds;
        set_nm(x);
      }
    }
  };
  // rescale the output accumulators by alpha where resc is set (after the P.V
  // MFMAs in flight)
  auto rescale_o = [&](const float (&alpha)[NX], int resc) { rescale_o_pinned(o, alpha[0], alpha[1], resc); };

  // ---- prologue: tiles 0, 1 and 2 in flight (0 and 1 landed); the scores,
  // maxima and probabilities of the first half-tile (keys 0..31)
#pragma unroll
  for (int x = 0; x < AHEAD; ++x) {
    issue_range(x, ld_f, ld_b, x < ntiles, 0, LPT);
    next_load();
  }
  vm_wait_all_but<LPT>();
  __syncthreads();
  // The loop runs over half-tiles of 32 keys (key block kb of a 64-key tile): one
  // 32 x 32 score accumulator per query block.
  const bf16x2 ones = {(__bf16)1.f, (__bf16)1.f};
  floatx16 sn[NX];                    // scores of the next half-tile
  bf16x8 pa[NX][2], pz[NX][2];        // probabilities (ping-pong): query block x, 16-key group g
  // exponentials of the scores s into probabilities p, with their row sums
  auto probs_all = [&](floatx16 (&sc)[NX], bf16x8 (&p)[NX][2], float (&psum)[NX]) {
#pragma unroll
    for (int x = 0; x < NX; ++x) {
      psum[x] = 0.f;
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        p[x][r / 8][r % 8] = (__bf16)__builtin_amdgcn_exp2f(lg(sc[x][r]));
        p[x][r / 8][r % 8 + 1] = (__bf16)__builtin_amdgcn_exp2f(lg(sc[x][r + 1]));
        psum[x] = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{p[x][r / 8][r % 8], p[x][r / 8][r % 8 + 1]}, ones,
                                                  psum[x], false);
      }
    }
  };
  {
#pragma unroll
    for (int st = 0; st < QS; ++st) {
      const KFrag kf = Cfg::kfrag(smem, 2 * st, j, hf);
#pragma unroll
      for (int x = 0; x < NX; ++x) {
        if (st == 0) M::template qk<true>(QS * x + st, sn[x], kf, qf[x][st], nm[x], sk, sq);
        else M::template qk<false>(QS * x + st, sn[x], kf, qf[x][st], nm[x], sk, sq);
      }
    }
    score_fence2(sn);
    float mx[NX], alpha[NX];
    mask_tail(sn, min(BK, N), mx);
    int resc0 = 0;
    raise(sn, mx, true, true, alpha, resc0);
    float psum[NX];
    probs_all(sn, pa, psum);
#pragma unroll
    for (int x = 0; x < NX; ++x) l_run[x] += psum[x];
  }

  const int nhalf = 2 * ntiles;
  int bcur = 0;                       // 64-key block (within its frame) of tile t

  // ---- LDS operand stream.  A half-tile step reads its operands as one stream
  // of 16-byte lane pieces: the K pieces of half-tile hh + 1 (bf16: one per MFMA
  // reduction step; fp8: two), then the V^T pieces of half-tile hh (16-key group
  // g, 32-channel block db).  Each piece is read PF pieces (several MFMAs) ahead,
  // across the two phases and into the next step, with one lgkmcnt wait per piece:
  // with one wave per SIMD nothing else hides the LDS latency.
  constexpr int KPC = FP8 ? 2 : 1;               // pieces per K fragment
  constexpr int NKP = QS * KPC;                  // K pieces of a half-tile
  constexpr int NVP = 2 * NDB;                   // V^T pieces of a half-tile
  constexpr int NP = NKP + NVP;                  // pieces of one step
  constexpr int PF = 4;                          // pieces read ahead
  static_assert(PF <= NKP && PF < 16, "the pieces read ahead into the next step are K pieces");
  // LDS address of piece n of step hh (n may run into the next step's stream)
  auto piece_addr = [&](int hh, int n) -> const unsigned char* {
    if (n >= NP) {
      hh += 1;
      n -= NP;
    }
    if (n < NKP) {
      const int tn = (hh + 1) >> 1, kbn = (hh + 1) & 1;       // half-tile hh + 1
      const unsigned char* row = smem + (tn % NSTG) * Cfg::STAGE + (32 * kbn + j) * Cfg::KP;
      const int chunk = FP8 ? 4 * (n / 2) + 2 * hf + (n % 2) : 2 * n + hf;
      return row + 16 * chunk;
    }
    const int m = n - NKP, g = m / NDB, db = m % NDB;
    const int t = hh >> 1, u = 2 * (hh & 1) + g;
    return smem + (t % NSTG) * Cfg::STAGE + Cfg::K_BYTES + (32 * db + j) * Cfg::VP + 16 * (2 * u + hf);
  };
  auto read_piece = [&](int hh, int n) { return *reinterpret_cast<const bf16x8*>(piece_addr(hh, n)); };
  // lgkmcnt(PF - 1): every piece but the PF - 1 most recent has arrived
  auto piece_wait = [&]() { __builtin_amdgcn_s_waitcnt(0xC07F | ((PF - 1) << 8)); };
  bf16x8 carry[PF];                   // the first PF pieces of the next step, in flight
#pragma unroll
  for (int n = 0; n < PF; ++n) carry[n] = read_piece(0, n);

  // One half-tile step hh (tile t = hh / 2, key block kb = hh % 2); pc holds the
  // probabilities of half-tile hh, pn receives those of half-tile hh + 1:
  //   phase A: Q.K^T of half-tile hh + 1 into sn (VGPR accumulators): MFMAs with
  //            only the LDS stream and the tile loads beside them;
  //   phase B: P.V of half-tile hh (AGPR accumulators), and beside its MFMAs the
  //            maxima of sn (slots 0-3), the lazy max check, then the
  //            exponentials, bf16 conversions and row sums of sn into pn
  //            (slots 4-15, skewed so that no VALU op waits on the one before).
  constexpr int NMS = 4;                         // phase B slots for the maxima
  static_assert(NVP * NX == 16, "16 P.V MFMAs per half-tile");
  auto step = [&](auto kbc, int hh, bf16x8 (&pc)[NX][2], bf16x8 (&pn)[NX][2]) {
    constexpr int kb = decltype(kbc)::value, kbn = 1 - kb;
    const int t = hh >> 1;
    const bool has_next = hh + 1 < nhalf;
    // 64-key block of half-tile hh + 1's tile, and that tile's valid keys
    const int bnext = kb == 0 ? bcur : (bcur + 1 == nb ? 0 : bcur + 1);
    const int nvalid_next = min(BK, N - BK * bnext);
    const bool ld = t + AHEAD < ntiles;                        // tile t + 3 exists
    const int ldf = ld_f, ldb = ld_b;
    // this half-tile's share of the loads of tile t + 3 (half of the wave's),
    // spread over the pieces
    constexpr int LX0 = kb * LPT / 2, NLD = (kb + 1) * LPT / 2 - LX0;

    bf16x8 pcs[NP];                   // this step's pieces
#pragma unroll
    for (int n = 0; n < PF; ++n) pcs[n] = carry[n];
    auto advance = [&](int n) {
      piece_wait();
      if (n + PF < NP) pcs[n + PF] = read_piece(hh, n + PF);
      else carry[n + PF - NP] = read_piece(hh, n + PF);
      issue_range((t + AHEAD) % NSTG, ldf, ldb, ld, LX0 + n * NLD / NP, LX0 + (n + 1) * NLD / NP);
    };

    // ---- phase A: Q.K^T of half-tile hh + 1 (past the last: of a stale stage,
    // the result unused)
#pragma unroll
    for (int n = 0; n < NKP; ++n) {
      advance(n);
      if (n % KPC == KPC - 1) {
        const int st = n / KPC;
        KFrag kf;
        if constexpr (FP8) {
          kf = __builtin_shufflevector(__builtin_bit_cast(intx4, pcs[n - 1]), __builtin_bit_cast(intx4, pcs[n]), 0,
                                       1, 2, 3, 4, 5, 6, 7);
        } else {
          kf = pcs[n];
        }
#pragma unroll
        for (int x = 0; x < NX; ++x) {
          if (st == 0) M::template qk<true>(QS * x + st, sn[x], kf, qf[x][st], nm[x], sk, sq);
          else M::template qk<false>(QS * x + st, sn[x], kf, qf[x][st], nm[x], sk, sq);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }

    // ---- phase B: P.V of half-tile hh, the softmax of half-tile hh + 1 beside it
    float mx[NX][2];                  // maxima: two chains per query block
    float alpha[NX] = {1.f, 1.f};
    int resc = 0;                     // the running max was raised: O is rescaled
    float psum[NX] = {0.f, 0.f};
    // exponential pairs (x, r) = (c / 8, 2 (c % 8)) of slot k >= NMS
    auto pair_lo = [](int k) { return (k - NMS) * 16 / (16 - NMS); };
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const int n = NKP + k / NX, m = k / NX, g = m / NDB, db = m % NDB, x = k % NX;
      if (x == 0) advance(n);
      mma_pv(NDB * x + db, o[x][db], pcs[n], pc[x][g]);
      if (k == 0) score_fence2(sn);
      if (k < NMS) {
        // one step of each of the four max chains (x, half h): elements 8h + 2k, + 1
#pragma unroll
        for (int xx = 0; xx < NX; ++xx)
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const int r = 8 * h + 2 * k;
            mx[xx][h] = k == 0 ? __builtin_fmaxf(sn[xx][r], sn[xx][r + 1])
                               : __builtin_fmaxf(__builtin_fmaxf(mx[xx][h], sn[xx][r]), sn[xx][r + 1]);
          }
        if (k == NMS - 1) {
          // the maxima are complete: masking of a partial block, lazy raise
          float mm[NX];
#pragma unroll
          for (int xx = 0; xx < NX; ++xx) mm[xx] = __builtin_fmaxf(mx[xx][0], mx[xx][1]);
          asm volatile("" ::"v"(mm[0]), "v"(mm[1]));   // formed here, beside the MFMAs
          if (has_next && 32 * kbn + 32 > nvalid_next) mask_tail(sn, nvalid_next - 32 * kbn, mm);
          raise(sn, mm, has_next, false, alpha, resc);
        }
      } else {
        // skewed: exponentials of this slot's pairs, conversions of the previous
        // slot's, row sums of the slot before that
#pragma unroll
        for (int c = pair_lo(k); c < pair_lo(k + 1); ++c) {
          const int xx = c / 8, r = 2 * (c % 8);
          // (in place: the scores are not needed after their exponential)
          sn[xx][r] = __builtin_amdgcn_exp2f(lg(sn[xx][r]));
          sn[xx][r + 1] = __builtin_amdgcn_exp2f(lg(sn[xx][r + 1]));
        }
        if (k > NMS) {
#pragma unroll
          for (int c = pair_lo(k - 1); c < pair_lo(k); ++c) {
            const int xx = c / 8, r = 2 * (c % 8);
            pn[xx][r / 8][r % 8] = (__bf16)sn[xx][r];
            pn[xx][r / 8][r % 8 + 1] = (__bf16)sn[xx][r + 1];
          }
        }
        if (k > NMS + 1) {
#pragma unroll
          for (int c = pair_lo(k - 2); c < pair_lo(k - 1); ++c) {
            const int xx = c / 8, r = 2 * (c % 8);
            psum[xx] = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{pn[xx][r / 8][r % 8], pn[xx][r / 8][r % 8 + 1]},
                                                       ones, psum[xx], false);
          }
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    // the skew's tail: conversions of the last slot's pairs, row sums of the last two
#pragma unroll
    for (int c = pair_lo(15); c < 16; ++c) {
      const int xx = c / 8, r = 2 * (c % 8);
      pn[xx][r / 8][r % 8] = (__bf16)sn[xx][r];
      pn[xx][r / 8][r % 8 + 1] = (__bf16)sn[xx][r + 1];
    }
#pragma unroll
    for (int c = pair_lo(14); c < 16; ++c) {
      const int xx = c / 8, r = 2 * (c % 8);
      psum[xx] = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{pn[xx][r / 8][r % 8], pn[xx][r / 8][r % 8 + 1]}, ones,
                                                 psum[xx], false);
    }
    // the probabilities are formed here, beside this step's MFMAs (not where the
    // next step reads them)
    asm volatile("" ::"v"(pn[0][0]), "v"(pn[0][1]), "v"(pn[1][0]), "v"(pn[1][1]), "v"(psum[0]), "v"(psum[1]));
#pragma unroll
    for (int x = 0; x < NX; ++x) l_run[x] += has_next ? psum[x] : 0.f;
    rescale_o(alpha, resc);
    if (kb == 1) {
      vm_wait_all_but<LPT>();          // this wave's loads of tile t + 2 landed (t + 3's may fly)
      __syncthreads();                 // ... and every wave's; the stage of tile t is free
      next_load();                     // (after the straight-line part of the step)
      bcur = bnext;
    }
  };
  for (int hh = 0; hh < nhalf; hh += 2) {
    step(std::integral_constant<int, 0>{}, hh, pa, pz);
    step(std::integral_constant<int, 1>{}, hh + 1, pz, pa);
  }

  // ---- epilogue (as attn_lds_kernel: fused readout + gated merge for chunk items)
  __builtin_amdgcn_s_waitcnt(0);     // the last (empty) tile loads and stream reads are done
                                     // before LDS is reused
  __syncthreads();
  acc_fence(o);
  float l_tot[NX];
#pragma unroll
  for (int x = 0; x < NX; ++x) l_tot[x] = pair_sum(l_run[x]);
  constexpr int WCH = D / 8;
  constexpr int WP = 16 * (WCH + 1);
  constexpr int W_INSTR = (D * (WCH + 1) + 63) / 64;
  static_assert(1024 * W_INSTR <= NSTG * Cfg::STAGE, "W fits in the LDS stages");
  using KArgs = const __attribute__((address_space(4))) AttnArgs*;
  KArgs kargs = (KArgs)__builtin_amdgcn_kernarg_segment_ptr();
  asm volatile("" : "+s"(kargs));
  const uint16_t* Wp = kargs->W;
  const bool lin = it.split < 0 && Wp != nullptr;
  constexpr int QSB = D / 16;
  bf16x8 qr[NX][QSB];
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
#pragma unroll
    for (int x = 0; x < NX; ++x) {
      const uint16_t* qrow =
          static_cast<const uint16_t*>(kargs->q) + (size_t)(it.q_tok0 + 64 * w + 32 * x + j) * rs + (size_t)h * D;
#pragma unroll
      for (int s = 0; s < QSB; ++s)
        qr[x][s] = qvalid[x] ? *reinterpret_cast<const bf16x8*>(qrow + 16 * s + 8 * hf) : bf16x8{};
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }
  float inv[NX];
#pragma unroll
  for (int x = 0; x < NX; ++x) inv[x] = 1.f / l_tot[x];
  if (lin) {
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      floatx16 acc[NX] = {};
#pragma unroll
      for (int s = 0; s < QSB; ++s) {
        const bf16x8 wf = *reinterpret_cast<const bf16x8*>(smem + (32 * db + j) * WP + 16 * (2 * s + hf));
#pragma unroll
        for (int x = 0; x < NX; ++x) acc[x] = mfma_bf16(wf, qr[x][s], acc[x]);
      }
#pragma unroll
      for (int x = 0; x < NX; ++x)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[x][db][r] = fmaf(o[x][db][r], inv[x], acc[x][r]);
    }
#pragma unroll
    for (int x = 0; x < NX; ++x) inv[x] = 1.f;
  }
#pragma unroll
  for (int x = 0; x < NX; ++x) {
    if (!qvalid[x]) continue;
    const int qi = 64 * w + 32 * x + j;
    if (it.split < 0) {
      const size_t ooff = (size_t)(it.q_tok0 + qi) * rs + (size_t)h * D;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int dd = 32 * db + 8 * g + 4 * hf;
          const uint2 pk = make_uint2(pack_bf16x2(o[x][db][4 * g + 0] * inv[x], o[x][db][4 * g + 1] * inv[x]),
                                      pack_bf16x2(o[x][db][4 * g + 2] * inv[x], o[x][db][4 * g + 3] * inv[x]));
          *reinterpret_cast<uint2*>(static_cast<uint16_t*>(kargs->O) + ooff + dd) = pk;
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
              make_float4(o[x][db][4 * g + 0], o[x][db][4 * g + 1], o[x][db][4 * g + 2], o[x][db][4 * g + 3]);
        }
      if (hf == 0) {
        kargs->part_ml[2 * row + 0] = m_run[x];
        kargs->part_ml[2 * row + 1] = l_tot[x];
      }
    }
  }
}


// the video path at d = 128 (bf16 or fp8 q.k, no extra tokens, O or anchor
// partials): 64 queries per wave
hipError_t launch_attn_w64(int prec, const AttnArgs& a0, hipStream_t st) {
  AttnArgs a = a0;
  a.bq = 256;
  if (prec == 1) {
    static std::atomic<unsigned long long> done{0};
    return attn_launch_items(&attn_w64_kernel<128, 1>, 4 * LdsCfg<128, 1>::STAGE + 1024, &done, a, st, 256);
  }
  if (prec == 2) {
    static std::atomic<unsigned long long> done{0};
    return attn_launch_items(&attn_w64_kernel<128, 2>, 4 * LdsCfg<128, 2>::STAGE + 1024, &done, a, st, 256);
  }
  return hipErrorInvalidValue;
}

}  // namespace vdn
