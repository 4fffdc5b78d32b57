// Definitions shared by the attention kernels (attn.hip, attn64.hip): the kernel
// argument block, the work items (256 query rows of one query frame's chunk and
// one head, or one key slice of an anchor frame's rows) and the LDS tile layout
// of the direct-load kernels.
#pragma once

#include <algorithm>
#include <atomic>
#include <cstdlib>
#include <type_traits>
#include <vector>

#include "common.h"
#include "kernels.h"

namespace vdn {

// ============================================================ attention
// Work items, one per 128-query tile:
//   anchor items (first and last frame, all key frames split into `nsplit`
//   slices of `fs` frames; partial results go to part_O / part_ml), then
//   chunk items (head-major, chunk-major: the non-anchor query frames of each
//   chunk, as one contiguous token range, against the chunk's key frames).
struct AttnArgs {
  const void* q;
  const void* k;
  const void* v;          // fp32 path: raw v
  const uint16_t* vt;     // bf16 / fp8 paths: transposed v
  const uint8_t* q8;      // fp8 path: E4M3 codes
  const uint8_t* k8;
  const int* fexp;        // fp8 paths: [3][H] power-of-two scale exponents (q, k, v)
  void* O;
  float* part_O;          // [nsplit][H][na][N][D]
  float* part_ml;         // [nsplit][H][na][N][2]
  const uint16_t* W;      // bf16 / fp8 paths: readout weights g (.) (S_fwd + S_bwd), bf16
                          // [C][H][D][D] (row = value dim); when set, chunk items write
                          // O_soft + W q, else O_soft
  int F, N, H;
  int nsplit, fs, na, qt_anchor;
  int n_anchor_items;
  int tiles_per_head;     // sum over chunks of the chunk items' tile counts
  int bq;                 // query rows per work item (32 per wave)
  float scale_log2;       // log2(e) / sqrt(D)
  // extra (text / audio) tokens: T tokens after the F*N video tokens of q, k, v, O;
  // every interaction involving one of them is plain softmax.  bf16 / fp8 paths.
  int T;                  // 0: none
  int nbx;                // 64-key blocks of the extra tokens
  int qt_x;               // query tiles of the extra tokens' rows
  const uint16_t* vtx;    // their V^T blocks [H][nbx][D][64], laid out as vt
  // with extra tokens: the online-softmax state of every video query row after the
  // extra tokens' keys, [H][F*N][D + 4] (o unnormalised, m, l, 2 pad), written by the
  // extra-token instantiation and the start of the video pass
  float* px;
  // Item queues (attn_lds_kernel without extra tokens; null: the static map of
  // decode_item).  Queue x holds, head after head, the items [run[x], run[x+1]) of
  // every head (contiguous runs of about equal cost); qctr[x] is its cursor, zero
  // at launch.  A workgroup takes the next item of its own XCD's queue, or, once
  // that is empty, of the next non-empty queue.
  int* qctr;
  int run[9];
};

constexpr int BQ = 128;   // queries per work item of attn_kernel (4 waves x 32)
#ifndef VDN_LDS_WAVES
#define VDN_LDS_WAVES 8
#endif
constexpr int kLdsWaves = VDN_LDS_WAVES;   // waves per workgroup of attn_lds_kernel
#ifndef VDN_LDS_STAGES
#define VDN_LDS_STAGES 2
#endif
constexpr int kLdsStages = VDN_LDS_STAGES;  // LDS tile stages of attn_lds_kernel (2 or 4)
#ifndef VDN_QK_BATCH
#define VDN_QK_BATCH 4       // Q.K^T MFMAs per operand batch of attn_lds_kernel
#endif
constexpr int kQkBatch = VDN_QK_BATCH;
#ifndef VDN_LDS_WAITALL
#define VDN_LDS_WAITALL 1    // wait for all LDS reads before issuing each operand batch (measured ~0.7 % faster)
#endif
constexpr int BK = 64;    // keys per tile
constexpr float kLazy = 8.f;   // log2 headroom before the running max is raised

// Frame of slot `s` in the key-frame list of a chunk item: the first frame (if not
// in the window), the window frames, the last frame (if not in the window).
__device__ inline int chunk_key_frame(int s, int wf, int we, int F) {
  if (wf > 0) {
    if (s == 0) return 0;
    --s;
  }
  if (s < we - wf) return wf + s;
  return F - 1;
}
// The same, written with selects only (for tile loops that call it in
// straight-line code)
__device__ inline int chunk_key_frame_sel(int s, int wf, int we, int F) {
  const int sw = wf > 0 ? s - 1 : s;                  // slot among the window frames
  const int f = sw < we - wf ? wf + sw : F - 1;
  return (wf > 0 && s == 0) ? 0 : f;
}

// ============================================================ attention, bf16 / fp8
// Same work items and arithmetic as attn_kernel, with K and V^T tiles moved
// global -> LDS by the 16-byte direct loads of gfx950 (buffer_load_dwordx4 ...
// lds): no staging registers, no LDS store instructions.  A direct load writes
// the 64 lanes' 16-byte pieces to 1 KiB of consecutive LDS; every LDS row holds
// one 16-byte padding chunk after its data (the lane that lands there re-reads a
// chunk of the row), so 16 consecutive rows read at one chunk hit 16 distinct
// bank groups, and the address of every operand fragment is one lane register
// plus an immediate offset.
template <int D, int PREC>
struct LdsCfg {
  static constexpr bool FP8 = PREC >= 2;           // q.k on E4M3 codes
  static constexpr bool FP8V = PREC == 3;          // P.V on E4M3 codes too
  static constexpr int KROW = FP8 ? D : 2 * D;     // bytes per K row in global memory
  static constexpr int KCH = KROW / 16;            // 16-byte chunks per K row
  static constexpr int KP = 16 * (KCH + 1);        // LDS pitch of a K row
  static constexpr int VCH = FP8V ? 4 : 8;         // 16-byte chunks of a V^T row (64 keys)
  static constexpr int VP = 16 * (VCH + 1);        // LDS pitch of a V^T row (+ pad)
  static constexpr int K_INSTR = KCH + 1;          // wave-wide direct loads per K tile (64 rows)
  static constexpr int V_INSTR = ((VCH + 1) * D + 63) / 64;
  static constexpr int K_BYTES = 1024 * K_INSTR;
  static constexpr int V_BYTES = 1024 * V_INSTR;
  static constexpr int STAGE = K_BYTES + V_BYTES;
  static constexpr int QSTEPS = FP8 ? D / 64 : D / 16;
  static_assert(BK * (KCH + 1) == 64 * K_INSTR, "a K tile is whole wave-wide loads");
  // LDS operand of one Q.K^T MFMA: K rows 32*kb + (lane & 31), reduction step
  // st, for item i = 2*st + kb (bf16: 16 dims; fp8: 64 dims)
  using KFrag = typename std::conditional<FP8, intx8, bf16x8>::type;
  __device__ static KFrag kfrag(const unsigned char* sbase, int i, int j, int hf) {
    const int st = i >> 1, kb = i & 1;
    const unsigned char* krow = sbase + (32 * kb + j) * KP;
    if constexpr (FP8) {
      const int c0 = 4 * st + 2 * hf;
      const uint4 x0 = *reinterpret_cast<const uint4*>(krow + 16 * c0);
      const uint4 x1 = *reinterpret_cast<const uint4*>(krow + 16 * (c0 + 1));
      return KFrag{(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w, (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
    } else {
      return *reinterpret_cast<const bf16x8*>(krow + 16 * (2 * st + hf));
    }
  }
  // LDS operand of one P.V MFMA: V^T rows 32*db + (lane & 31), keys 16u..16u+15
  __device__ static bf16x8 vfrag(const unsigned char* vbase, int u, int db, int j, int hf) {
    return *reinterpret_cast<const bf16x8*>(vbase + (32 * db + j) * VP + 16 * (2 * u + hf));
  }
  // fp8 P.V: V^T rows 32*db + (lane & 31), the 32 codes of lane half hf (all 64 keys
  // of the tile in one 64-deep MFMA; see the vt8 layout)
  __device__ static intx8 vfrag8(const unsigned char* vbase, int db, int j, int hf) {
    const unsigned char* row = vbase + (32 * db + j) * VP + 32 * hf;
    const uint4 x0 = *reinterpret_cast<const uint4*>(row);
    const uint4 x1 = *reinterpret_cast<const uint4*>(row + 16);
    return intx8{(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w, (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
  }
};

// s_waitcnt lgkmcnt(0) alone (vmcnt and expcnt at their maxima)
__device__ inline void lds_wait_all() { __builtin_amdgcn_s_waitcnt(0xC07F); }

template <int KX, int VX>
struct LaneOffsets {
  uint32_t koff[KX], voff[VX];
};

struct Item {
  int h, q_tok0, q_rows, split, anchor_idx;
  int mode;          // 0: frames [k_f0, k_f0 + nslots); 1: chunk key list
  int k_f0, wf, we, nslots;
};

// Item li of head hh (items per head: the anchor items, then the chunk items).
__device__ inline Item decode_item_at(const AttnArgs& a, int hh, int li) {
  Item it;
  const int F = a.F, N = a.N;
  const int na_h = a.na * a.qt_anchor * a.nsplit;        // anchor items per head
  it.wf = it.we = it.k_f0 = 0;
  if (li < na_h) {
    int rr = li;
    const int qt = rr % a.qt_anchor;
    rr /= a.qt_anchor;
    it.anchor_idx = rr % a.na;
    it.split = rr / a.na;
    it.h = hh;
    const int qf = it.anchor_idx == 0 ? 0 : F - 1;
    it.q_tok0 = qf * N + qt * a.bq;
    it.q_rows = min(a.bq, N - qt * a.bq);
    it.mode = 0;
    it.k_f0 = it.split * a.fs;
    it.nslots = min(F, it.k_f0 + a.fs) - it.k_f0;
  } else {
    int rr = li - na_h;
    it.split = -1;
    it.anchor_idx = 0;
    it.h = hh;
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
    it.nslots = (it.wf > 0 ? 1 : 0) + (it.we - it.wf) + (it.we < F ? 1 : 0);
  }
  return it;
}

// Work item of this workgroup from its block index (same numbering as attn_kernel).
// Blocks go out head by head (all XCDs stream one head's K / V^T at a time, which
// the last-level cache holds); inside a head, the blocks one XCD receives (every
// 8th, as the dispatcher deals them round-robin) take a contiguous run of the
// head's items, so the items that share key frames share that XCD's L2.
__device__ inline Item decode_item(const AttnArgs& a) {
  const int M = a.na * a.qt_anchor * a.nsplit + a.tiles_per_head;   // items per head
  const int b = blockIdx.x;
  const int hh = b / M, p = b - hh * M;
  const int q8 = M >> 3, m8 = M & 7, r = p & 7;
  return decode_item_at(a, hh, r * q8 + min(r, m8) + (p >> 3));
}

// Next item from the queues (one thread per workgroup): hh * M + li, or -1 when
// every queue is empty.  The XCD a workgroup runs on only picks the queue it tries
// first, so every item is taken exactly once whatever the dispatcher does, as long
// as the grid has at least as many workgroups as items.
__device__ inline int acquire_item(const AttnArgs& a) {
  const int M = a.na * a.qt_anchor * a.nsplit + a.tiles_per_head;
  const int x = __builtin_amdgcn_s_getreg((15 << 11) | 20) & 7;   // HW_REG_XCC_ID
  for (int k = 0; k < 8; ++k) {
    const int y = (x + k) & 7;
    const int rl = a.run[y + 1] - a.run[y];
    const int n = rl * a.H;
    if (n == 0 || __hip_atomic_load(a.qctr + y, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= n) continue;
    const int i = __hip_atomic_fetch_add(a.qctr + y, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (i < n) {
      const int hh = i / rl;
      return hh * M + a.run[y] + (i - hh * rl);
    }
  }
  return -1;
}


// An item with every field read from the first lane: it is the same in every
// lane, and this lets the compiler keep it and what derives from it in SGPRs.
__device__ inline Item uniform_item(Item it) {
  it.h = __builtin_amdgcn_readfirstlane(it.h);
  it.q_tok0 = __builtin_amdgcn_readfirstlane(it.q_tok0);
  it.q_rows = __builtin_amdgcn_readfirstlane(it.q_rows);
  it.split = __builtin_amdgcn_readfirstlane(it.split);
  it.anchor_idx = __builtin_amdgcn_readfirstlane(it.anchor_idx);
  it.mode = __builtin_amdgcn_readfirstlane(it.mode);
  it.k_f0 = __builtin_amdgcn_readfirstlane(it.k_f0);
  it.wf = __builtin_amdgcn_readfirstlane(it.wf);
  it.we = __builtin_amdgcn_readfirstlane(it.we);
  it.nslots = __builtin_amdgcn_readfirstlane(it.nslots);
  return it;
}

// ---------------------------------------------------------------- launches
// Work-item counts for query tiles of a.bq rows.
inline void attn_items(AttnArgs& a) {
  a.qt_anchor = (a.N + a.bq - 1) / a.bq;
  a.qt_x = (a.T + a.bq - 1) / a.bq;
  a.n_anchor_items = a.H * (a.na * a.qt_anchor + a.qt_x) * a.nsplit;
  int tph = 0;
  for (int c = 0; c < num_chunks(a.F); ++c) {
    const int nf = nq_end(c, a.F) - nq_first(c);
    if (nf > 0) tph += (int)(((long long)nf * a.N + a.bq - 1) / a.bq);
  }
  a.tiles_per_head = tph;
}

// Item queues: the 8 runs of every head's items, cut where the running cost (key
// tiles, plus about 7 tiles' worth for an item's prologue and epilogue) crosses
// k/8 of the head's total.
inline void attn_queue_plan(AttnArgs& a) {
  const int nb = (a.N + BK - 1) / BK;
  const int na_h = a.na * a.qt_anchor * a.nsplit;
  std::vector<long long> cost;
  for (int li = 0; li < na_h; ++li) {
    const int split = li / a.qt_anchor / a.na;
    const int k0 = split * a.fs;
    cost.push_back((long long)(std::min(a.F, k0 + a.fs) - k0) * nb + 7);
  }
  for (int c = 0; c < num_chunks(a.F); ++c) {
    const int nf = nq_end(c, a.F) - nq_first(c);
    if (nf <= 0) continue;
    const int t = (int)(((long long)nf * a.N + a.bq - 1) / a.bq);
    const int wf = win_first(c), we = win_end(c, a.F);
    const int nsl = (wf > 0 ? 1 : 0) + (we - wf) + (we < a.F ? 1 : 0);
    for (int r = 0; r < t; ++r) cost.push_back((long long)nsl * nb + 7);
  }
  long long total = 0;
  for (long long c : cost) total += c;
  const int M = (int)cost.size();
  a.run[0] = 0;
  long long acc = 0;
  int li = 0;
  for (int k = 1; k < 8; ++k) {
    while (li < M && 8 * (acc + cost[li] / 2) < k * total) acc += cost[li++];
    a.run[k] = li;
  }
  a.run[8] = M;
}

// One workgroup per work item of a.bq query rows (a.bq set by the caller); with
// queue, items come from the queues of a.qctr (cleared here), and the grid has
// an eighth more workgroups than items so that an XCD that runs ahead can take
// items from the others' queues (the extra workgroups find every queue empty and
// return).
template <typename KernelFn>
inline hipError_t attn_launch_items(KernelFn fn, int lds, std::atomic<unsigned long long>* attr_done, AttnArgs a,
                                    hipStream_t st, int threads, bool queue = false) {
  attn_items(a);
  hipError_t e = set_max_lds_once(reinterpret_cast<const void*>(fn), lds, attr_done);
  if (e != hipSuccess) return e;
  const int nitems = a.n_anchor_items + a.H * a.tiles_per_head;
  if (nitems == 0) return hipSuccess;
  int grid = nitems;
  if (queue && a.qctr != nullptr) {
    attn_queue_plan(a);
    e = launch_fill_u32(reinterpret_cast<uint32_t*>(a.qctr), 8, 0u, st);
    if (e != hipSuccess) return e;
    grid = nitems + (nitems / 8 + 64 + 7) / 8 * 8;
  } else {
    a.qctr = nullptr;
  }
  hipLaunchKernelGGL(fn, dim3(grid), dim3(threads), lds, st, a);
  return hipGetLastError();
}

// attn64.hip: the video path at d = 128 with 64 queries per wave (prec 1: bf16,
// 2: fp8 q.k); no extra tokens
hipError_t launch_attn_w64(int prec, const AttnArgs& a, hipStream_t st);
// VDN_ATTN_W64=1 in the environment (read at every launch) routes the video pass
// of the bf16 / fp8 paths at d = 128 without extra tokens to attn_w64_kernel
inline bool attn_w64_requested() {
  const char* e = std::getenv("VDN_ATTN_W64");
  return e != nullptr && e[0] == '1';
}

}  // namespace vdn
