// C ABI of the VDN hybrid video-to-video attention layer: argument checks, the
// frame-partition table, workspace carving and the launch sequence.  Every step
// of the computation runs in the kernels of attn.hip and vda.hip.
#include "vdn_hybrid_attn.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdint>
#include <vector>

#include "common.h"
#include "kernels.h"

namespace {

thread_local int g_last_hip_error = 0;
thread_local hipEvent_t g_stage_ev[VDN_NUM_STAGES][2] = {};

int fail_hip(hipError_t e) {
  g_last_hip_error = static_cast<int>(e);
  return VDN_ERR_HIP;
}

#define VDN_TRY(expr)                        \
  do {                                       \
    hipError_t e_ = (expr);                  \
    if (e_ != hipSuccess) return fail_hip(e_); \
  } while (0)

hipError_t mark(int stage, int which, hipStream_t st) {
  hipEvent_t e = g_stage_ev[stage][which];
  return e ? hipEventRecord(e, st) : hipSuccess;
}

// Enqueue one stage, bracketed by the caller's measurement events if set.
#define VDN_STAGE(stage, st, expr)          \
  do {                                      \
    VDN_TRY(mark((stage), 0, (st)));        \
    VDN_TRY(expr);                          \
    VDN_TRY(mark((stage), 1, (st)));        \
  } while (0)

int check_shape(int F, int N, int H, int d, int prec) {
  if (F < 1 || N < 1 || H < 1) return VDN_ERR_INVALID_ARG;
  if (prec < VDN_PREC_FP32 || prec > VDN_PREC_FP8) return VDN_ERR_INVALID_ARG;
  if (d != 32 && d != 64 && d != 128) return VDN_ERR_UNSUPPORTED;
  if (prec >= VDN_PREC_BF16_FP8QK && d == 32) return VDN_ERR_UNSUPPORTED;
  // token indices are 32-bit inside the kernels; grid y/z dimensions carry H
  if (static_cast<long long>(F) * N > (1LL << 30) || H > 65535) return VDN_ERR_UNSUPPORTED;
  return VDN_OK;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

size_t al256(size_t x) { return (x + 255) / 256 * 256; }

// Extra (text / audio) tokens: bf16 / fp8 only; every token index stays 32-bit.
int check_extra(int F, int N, int T, int prec) {
  if (T < 0) return VDN_ERR_INVALID_ARG;
  if (T > 0 && (prec == VDN_PREC_FP32 || prec == VDN_PREC_FP8)) return VDN_ERR_UNSUPPORTED;
  if (static_cast<long long>(F) * N + T > (1LL << 30)) return VDN_ERR_UNSUPPORTED;
  return VDN_OK;
}

// Workspace carving (byte offsets).
struct Layout {
  size_t vt = 0, vtx = 0, px = 0, G = 0, B = 0, Sf = 0, Sb = 0, W = 0, pO = 0, pml = 0, q8 = 0, k8 = 0, fexp = 0,
         qctr = 0;
  size_t total = 0;
};

// T: extra tokens after the F*N video tokens (0: none)
Layout layout(int F, int N, int H, int d, int prec, int T = 0) {
  Layout L;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += al256(bytes);
    return o;
  };
  const size_t nb = (static_cast<size_t>(N) + 63) / 64;
  const size_t C = static_cast<size_t>(vdn::num_chunks(F));
  const size_t dd = static_cast<size_t>(d) * d;
  int nsplit = 1, fs = 1;
  vdn::attn_split_plan(F, &nsplit, &fs);
  const size_t na = F >= 2 ? 2 : 1;
  L.vt = take(prec == VDN_PREC_FP32 ? 0 : static_cast<size_t>(H) * F * nb * d * 64 * 2);
  L.vtx = take(static_cast<size_t>(H) * ((static_cast<size_t>(T) + 63) / 64) * d * 64 * 2);
  // with extra tokens: softmax state of every video query row, [H][F*N][d + 4] fp32 (16-byte rows)
  L.px = take(T > 0 ? static_cast<size_t>(H) * F * N * (d + 4) * 4 : 0);
  L.G = take(static_cast<size_t>(F) * H * dd * 4);
  L.B = take(static_cast<size_t>(F) * H * dd * 4);
  L.Sf = take(C * H * dd * 4);
  L.Sb = take(C * H * dd * 4);
  L.W = take(C * H * dd * 4);              // bf16 (first half), or fp32
  const size_t rows = na * N + static_cast<size_t>(T);      // split rows per head: anchors, extras
  L.pO = take(static_cast<size_t>(nsplit) * H * rows * d * 4);
  L.pml = take(static_cast<size_t>(nsplit) * H * rows * 2 * 4);
  L.qctr = take(prec == VDN_PREC_FP32 ? 0 : 8 * 4);        // attention item-queue cursors
  if (prec >= VDN_PREC_BF16_FP8QK) {
    const size_t ntok = static_cast<size_t>(F) * N + T;
    L.q8 = take(ntok * H * d);
    L.k8 = take(ntok * H * d);
    L.fexp = take(3 * static_cast<size_t>(H) * 4);        // q, k, v scale exponents
  }
  L.total = off;
  return L;
}

struct WsPtr {
  unsigned char* base;
  template <typename T>
  T* at(size_t off) const { return reinterpret_cast<T*>(base + off); }
};

int check_ws(int F, int N, int H, int d, int prec, void* ws, size_t ws_bytes, Layout* L, int T = 0) {
  *L = layout(F, N, H, d, prec, T);
  if (ws == nullptr && L->total > 0) return VDN_ERR_INVALID_ARG;
  if (!aligned(ws, 256)) return VDN_ERR_INVALID_ARG;
  if (ws_bytes < L->total) return VDN_ERR_WORKSPACE;
  return VDN_OK;
}

hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

// ---- pieces of the launch sequence
// v laid out for the softmax branch (bf16 vt; with fp8 P.V, E4M3 codes in the vt8
// layout after v's per-head scale exponents), and with grams the frame Grams
int launch_vt(const void* k, const void* v, int F, int N, int H, int d, int prec, float* G, float* B, int grams,
              const Layout& L, WsPtr ws, hipStream_t st) {
  const uint16_t* k16 = static_cast<const uint16_t*>(k);
  const uint16_t* v16 = static_cast<const uint16_t*>(v);
  if (prec == VDN_PREC_FP8) {
    int* vexp = ws.at<int>(L.fexp) + 2 * H;
    VDN_TRY(vdn::launch_fp8_scale(v16, F, N, H, d, 1.f, vexp, st));
    VDN_TRY(vdn::launch_prep(k16, v16, F, N, H, d, nullptr, G, B, grams, st, ws.at<uint8_t>(L.vt), vexp));
  } else {
    VDN_TRY(vdn::launch_prep(k16, v16, F, N, H, d, ws.at<uint16_t>(L.vt), G, B, grams, st));
  }
  return VDN_OK;
}

// W: bf16 readout weights to fold into the attention epilogue (O = O_soft + W q on
// the non-anchor frames), or null for O = O_soft.  T: extra tokens after the video
// tokens of q, k, v, O (0: none).  split: O is [F*N][2][H][d], O_soft then W q
// (zero on the anchor frames), the output projection's input.
int run_softmax(const void* q, const void* k, const void* v, int F, int N, int H, int d, int prec,
                void* O, const Layout& L, WsPtr ws, bool vt_ready, const uint16_t* W, hipStream_t st,
                int T = 0, int split = 0) {
  const uint8_t* q8 = nullptr;
  const uint8_t* k8 = nullptr;
  const int* fexp = nullptr;
  if (prec >= VDN_PREC_BF16_FP8QK) {
    // per-head power-of-two scales over every token of the layer (the quantiser
    // sees F*N+T tokens as one frame); q is quantised after its multiplication by
    // the base-2 softmax temperature, so the Q.K^T MFMAs deliver log2 units
    const int qF = T > 0 ? 1 : F, qN = T > 0 ? F * N + T : N;
    VDN_TRY(mark(VDN_STAGE_QUANT, 0, st));
    VDN_TRY(vdn::launch_fp8_quant(static_cast<const uint16_t*>(q), qF, qN, H, d, vdn::softmax_temperature_log2(d),
                                  ws.at<uint8_t>(L.q8), ws.at<int>(L.fexp), st));
    VDN_TRY(vdn::launch_fp8_quant(static_cast<const uint16_t*>(k), qF, qN, H, d, 1.f, ws.at<uint8_t>(L.k8),
                                  ws.at<int>(L.fexp) + H, st));
    VDN_TRY(mark(VDN_STAGE_QUANT, 1, st));
    q8 = ws.at<uint8_t>(L.q8);
    k8 = ws.at<uint8_t>(L.k8);
    fexp = ws.at<int>(L.fexp);
  }
  if (prec != VDN_PREC_FP32 && !vt_ready) {
    VDN_TRY(mark(VDN_STAGE_PREP, 0, st));
    const int s = launch_vt(k, v, F, N, H, d, prec, nullptr, nullptr, 0, L, ws, st);
    if (s != VDN_OK) return s;
    VDN_TRY(mark(VDN_STAGE_PREP, 1, st));
  }
  if (T > 0) {
    // the extra tokens' V^T blocks, laid out as one more frame of T tokens (no
    // Grams; a few microseconds, outside the stage brackets)
    const size_t voff = static_cast<size_t>(F) * N * H * d;
    VDN_TRY(vdn::launch_prep(static_cast<const uint16_t*>(k) + voff, static_cast<const uint16_t*>(v) + voff, 1, T,
                             H, d, ws.at<uint16_t>(L.vtx), nullptr, nullptr, 0, st));
  }
  const int kprec = prec;      // 0 fp32, 1 bf16, 2 fp8 q.k, 3 fp8 q.k and P.V
  VDN_STAGE(VDN_STAGE_ATTN, st,
            vdn::launch_attn(kprec, q, k, v, ws.at<uint16_t>(L.vt), q8, k8, fexp, F, N, H, d, O,
                             ws.at<float>(L.pO), ws.at<float>(L.pml), W, T, ws.at<uint16_t>(L.vtx), split,
                             ws.at<float>(L.px), prec == VDN_PREC_FP32 ? nullptr : ws.at<int>(L.qctr), st));
  VDN_STAGE(VDN_STAGE_COMBINE, st,
            vdn::launch_combine(prec == VDN_PREC_FP32 ? 0 : 1, ws.at<float>(L.pO), ws.at<float>(L.pml),
                                F, N, T, H, d, O, split, st));
  return VDN_OK;
}

// Grams (and, on the bf16 paths, v transposed for the softmax branch), then the
// per-frame maps and the scan into Sf / Sb.
int run_states(const void* k, const void* v, const float* beta, int F, int N, int H, int d, int prec,
               float* Sf, float* Sb, const Layout& L, WsPtr ws, hipStream_t st) {
  float* G = ws.at<float>(L.G);
  float* B = ws.at<float>(L.B);
  if (prec == VDN_PREC_FP32)
    VDN_STAGE(VDN_STAGE_PREP, st,
              vdn::launch_gram_f32(static_cast<const float*>(k), static_cast<const float*>(v), F, N, H, d,
                                   G, B, st));
  else {
    VDN_TRY(mark(VDN_STAGE_PREP, 0, st));
    const int s = launch_vt(k, v, F, N, H, d, prec, G, B, 1, L, ws, st);
    if (s != VDN_OK) return s;
    VDN_TRY(mark(VDN_STAGE_PREP, 1, st));
  }
  VDN_STAGE(VDN_STAGE_FACTOR, st, vdn::launch_factor(G, B, beta, F, H, d, st));
  VDN_STAGE(VDN_STAGE_SCAN, st, vdn::launch_scan(G, B, F, H, d, Sf, Sb, st));
  return VDN_OK;
}

}  // namespace

extern "C" {

const char* vdn_status_string(int status) {
  switch (status) {
    case VDN_OK: return "ok";
    case VDN_ERR_INVALID_ARG: return "invalid argument";
    case VDN_ERR_UNSUPPORTED: return "unsupported shape or precision";
    case VDN_ERR_WORKSPACE: return "workspace too small";
    case VDN_ERR_HIP: return "HIP error";
    case VDN_ERR_TOO_LARGE: return "shape needs more scratch than vdn_hybrid_attn_noalloc holds";
  }
  return "unknown status";
}

int vdn_last_hip_error(void) { return g_last_hip_error; }

int vdn_set_stage_events(int stage, void* before, void* after) {
  if (stage < 0 || stage >= VDN_NUM_STAGES) return VDN_ERR_INVALID_ARG;
  g_stage_ev[stage][0] = static_cast<hipEvent_t>(before);
  g_stage_ev[stage][1] = static_cast<hipEvent_t>(after);
  return VDN_OK;
}

size_t vdn_workspace_bytes(int F, int N, int H, int d, int precision) {
  if (check_shape(F, N, H, d, precision) != VDN_OK) return 0;
  return layout(F, N, H, d, precision).total;
}

int vdn_schedule(int F, int* table, int cap) {
  if (F < 1 || cap < 0 || (cap > 0 && table == nullptr)) return VDN_ERR_INVALID_ARG;
  std::vector<int> rows;
  auto row = [&](int q0, int q1, const std::vector<int>& frames, int f0, int f1, int b0, int b1) {
    // compress the sorted frame list into at most three inclusive ranges
    int r[6] = {-1, -1, -1, -1, -1, -1};
    int n = 0;
    for (size_t x = 0; x < frames.size(); ++x) {
      if (n > 0 && frames[x] == r[2 * (n - 1) + 1] + 1) {
        r[2 * (n - 1) + 1] = frames[x];
      } else {
        r[2 * n] = r[2 * n + 1] = frames[x];
        ++n;
      }
    }
    const int v[VDN_SCHED_COLS] = {q0, q1, n, r[0], r[1], r[2], r[3], r[4], r[5], f0, f1, b0, b1};
    rows.insert(rows.end(), v, v + VDN_SCHED_COLS);
  };
  std::vector<int> all(F);
  for (int i = 0; i < F; ++i) all[i] = i;
  row(0, 0, all, -1, -1, -1, -1);
  for (int c = 0; c < vdn::num_chunks(F); ++c) {
    const int q0 = vdn::nq_first(c), q1 = vdn::nq_end(c, F) - 1;
    if (q1 < q0) continue;
    const int wf = vdn::win_first(c), we = vdn::win_end(c, F);
    std::vector<int> fr;
    if (wf > 0) fr.push_back(0);
    for (int x = wf; x < we; ++x) fr.push_back(x);
    if (we < F) fr.push_back(F - 1);
    const bool has_f = wf - 1 >= 1;
    const bool has_b = we <= F - 2;
    row(q0, q1, fr, has_f ? 1 : -1, has_f ? wf - 1 : -1, has_b ? we : -1, has_b ? F - 2 : -1);
  }
  if (F >= 2) row(F - 1, F - 1, all, -1, -1, -1, -1);
  const int nrows = static_cast<int>(rows.size() / VDN_SCHED_COLS);
  std::copy(rows.begin(), rows.begin() + std::min(nrows, cap) * VDN_SCHED_COLS, table);
  return nrows;
}

int vdn_hybrid_attn(const void* q, const void* k, const void* v, const float* beta, const float* gate,
                    int F, int N, int H, int d, int precision, void* O, void* workspace,
                    size_t workspace_bytes, void* stream) {
  int s = check_shape(F, N, H, d, precision);
  if (s != VDN_OK) return s;
  if (!q || !k || !v || !beta || !gate || !O) return VDN_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(O, 16)) return VDN_ERR_INVALID_ARG;
  Layout L;
  if ((s = check_ws(F, N, H, d, precision, workspace, workspace_bytes, &L)) != VDN_OK) return s;
  const hipStream_t st = as_stream(stream);
  WsPtr ws{static_cast<unsigned char*>(workspace)};
  float* Sf = ws.at<float>(L.Sf);
  float* Sb = ws.at<float>(L.Sb);
  // linear branch first: its pass over k and v also lays out v for the softmax branch,
  // and its readout weights are ready when the attention kernel ends its items
  if ((s = run_states(k, v, beta, F, N, H, d, precision, Sf, Sb, L, ws, st)) != VDN_OK) return s;
  const bool bf16 = precision != VDN_PREC_FP32;
  VDN_STAGE(VDN_STAGE_WPREP, st,
            vdn::launch_wprep(Sf, Sb, gate, vdn::num_chunks(F), H, d, bf16 ? 1 : 0, ws.at<void>(L.W), st));
  // bf16 / fp8: the readout and merge run in the attention kernel's epilogue;
  // fp32: O_soft first, then the readout adds g (.) O_lin
  const uint16_t* Wfused = bf16 ? ws.at<uint16_t>(L.W) : nullptr;
  if ((s = run_softmax(q, k, v, F, N, H, d, precision, O, L, ws, true, Wfused, st)) != VDN_OK) return s;
  if (!bf16)
    VDN_STAGE(VDN_STAGE_READOUT, st, vdn::launch_readout(0, q, ws.at<void>(L.W), F, N, H, d, O, 1, st));
  return VDN_OK;
}

// ---- the layer without any allocation: workspace in a static device array
}  // extern "C"

namespace {

// Workspace of vdn_hybrid_attn_noalloc.  In host code `scratch` names a host-side
// stand-in, not device memory: its device address on each GPU comes from
// hipGetSymbolAddress (each device holds its own copy), kept per device below and
// used for every kernel argument.
__device__ __align__(256) unsigned char scratch[VDN_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_addr[kMaxDevices];

// Device address of `scratch` on the current device (looked up once per device).
hipError_t scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* p = g_scratch_addr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_addr[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return hipSuccess;
}

}  // namespace

extern "C" {

int vdn_hybrid_attn_noalloc(const void* q, const void* k, const void* v, const float* beta, const float* gate,
                            int F, int N, int H, int d, int precision, void* O, void* stream) {
  int s = check_shape(F, N, H, d, precision);
  if (s != VDN_OK) return s;
  if (!q || !k || !v || !beta || !gate || !O) return VDN_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(O, 16)) return VDN_ERR_INVALID_ARG;
  const size_t need = layout(F, N, H, d, precision).total;
  if (need > VDN_NOALLOC_SCRATCH_BYTES) return VDN_ERR_TOO_LARGE;
  void* ws = nullptr;
  VDN_TRY(scratch_address(&ws));
  // every piece of the workspace is written before it is read within one call
  // (the fp8 maxima are cleared by a fill kernel), so nothing is cleared here
  return vdn_hybrid_attn(q, k, v, beta, gate, F, N, H, d, precision, O, ws, VDN_NOALLOC_SCRATCH_BYTES, stream);
}

// ---- the layer followed by the two branches' output projections
size_t layer_ws_proj(const Layout& L, int F, int N, int H, int d) {
  return L.total + al256(static_cast<size_t>(F) * N * 2 * H * d * 2);   // [F*N][2][H][d] bf16
}

size_t vdn_workspace_bytes_proj(int F, int N, int H, int d, int D, int precision) {
  if (check_shape(F, N, H, d, precision) != VDN_OK) return 0;
  if (precision == VDN_PREC_FP32 || precision == VDN_PREC_FP8 || D < 8 || D % 8 != 0) return 0;
  return layer_ws_proj(layout(F, N, H, d, precision), F, N, H, d);
}

int vdn_hybrid_attn_proj(const void* q, const void* k, const void* v, const float* beta, const float* gate,
                         const void* Wp, int F, int N, int H, int d, int D, int precision, void* Y,
                         void* workspace, size_t workspace_bytes, void* stream) {
  int s = check_shape(F, N, H, d, precision);
  if (s != VDN_OK) return s;
  if (precision == VDN_PREC_FP32 || precision == VDN_PREC_FP8) return VDN_ERR_UNSUPPORTED;
  if (D < 8 || D % 8 != 0) return VDN_ERR_UNSUPPORTED;
  if (static_cast<long long>(256) * 2 * (2LL * H * d) >= (1LL << 32)) return VDN_ERR_UNSUPPORTED;
  if (!q || !k || !v || !beta || !gate || !Wp || !Y) return VDN_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(Wp, 16) || !aligned(Y, 16))
    return VDN_ERR_INVALID_ARG;
  Layout L = layout(F, N, H, d, precision);
  if (workspace == nullptr || !aligned(workspace, 256)) return VDN_ERR_INVALID_ARG;
  if (workspace_bytes < layer_ws_proj(L, F, N, H, d)) return VDN_ERR_WORKSPACE;
  const hipStream_t st = as_stream(stream);
  WsPtr ws{static_cast<unsigned char*>(workspace)};
  uint16_t* Acat = ws.at<uint16_t>(L.total);           // [F*N][2][H][d]: O_soft, g (.) O_lin
  if ((s = run_states(k, v, beta, F, N, H, d, precision, ws.at<float>(L.Sf), ws.at<float>(L.Sb), L, ws, st)) !=
      VDN_OK)
    return s;
  VDN_STAGE(VDN_STAGE_WPREP, st,
            vdn::launch_wprep(ws.at<float>(L.Sf), ws.at<float>(L.Sb), gate, vdn::num_chunks(F), H, d, 1,
                              ws.at<void>(L.W), st));
  if ((s = run_softmax(q, k, v, F, N, H, d, precision, Acat, L, ws, true, ws.at<uint16_t>(L.W), st, 0, 1)) !=
      VDN_OK)
    return s;
  VDN_STAGE(VDN_STAGE_PROJ, st,
            vdn::launch_proj(Acat, static_cast<const uint16_t*>(Wp), F * N, D, 2 * H * d, static_cast<uint16_t*>(Y),
                             st, ws.at<int>(L.qctr)));
  return VDN_OK;
}

int vdn_out_proj(const void* A, const void* B, int M, int K, int N, void* Y, void* stream) {
  if (!A || !B || !Y) return VDN_ERR_INVALID_ARG;
  if (M < 1 || K < 1 || N < 1) return VDN_ERR_INVALID_ARG;
  if (K % 64 != 0 || N % 8 != 0 || static_cast<long long>(256) * 2 * K >= (1LL << 32)) return VDN_ERR_UNSUPPORTED;
  if (!aligned(A, 16) || !aligned(B, 16) || !aligned(Y, 16)) return VDN_ERR_INVALID_ARG;
  const hipStream_t st = as_stream(stream);
  VDN_STAGE(VDN_STAGE_PROJ, st,
            vdn::launch_proj(static_cast<const uint16_t*>(A), static_cast<const uint16_t*>(B), M, N, K,
                             static_cast<uint16_t*>(Y), st));
  return VDN_OK;
}

size_t vdn_workspace_bytes_mixed(int F, int N, int T, int H, int d, int precision) {
  if (check_shape(F, N, H, d, precision) != VDN_OK || check_extra(F, N, T, precision) != VDN_OK) return 0;
  return layout(F, N, H, d, precision, T).total;
}

int vdn_hybrid_attn_mixed(const void* q, const void* k, const void* v, const float* beta, const float* gate,
                          int F, int N, int T, int H, int d, int precision, void* O, void* workspace,
                          size_t workspace_bytes, void* stream) {
  int s = check_shape(F, N, H, d, precision);
  if (s != VDN_OK) return s;
  if ((s = check_extra(F, N, T, precision)) != VDN_OK) return s;
  if (T == 0)
    return vdn_hybrid_attn(q, k, v, beta, gate, F, N, H, d, precision, O, workspace, workspace_bytes, stream);
  if (!q || !k || !v || !beta || !gate || !O) return VDN_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(O, 16)) return VDN_ERR_INVALID_ARG;
  Layout L;
  if ((s = check_ws(F, N, H, d, precision, workspace, workspace_bytes, &L, T)) != VDN_OK) return s;
  const hipStream_t st = as_stream(stream);
  WsPtr ws{static_cast<unsigned char*>(workspace)};
  float* Sf = ws.at<float>(L.Sf);
  float* Sb = ws.at<float>(L.Sb);
  // the linear branch sees the video tokens only (the first F*N of every tensor)
  if ((s = run_states(k, v, beta, F, N, H, d, precision, Sf, Sb, L, ws, st)) != VDN_OK) return s;
  VDN_STAGE(VDN_STAGE_WPREP, st,
            vdn::launch_wprep(Sf, Sb, gate, vdn::num_chunks(F), H, d, 1, ws.at<void>(L.W), st));
  return run_softmax(q, k, v, F, N, H, d, precision, O, L, ws, true, ws.at<uint16_t>(L.W), st, T);
}

int vdn_softmax_branch(const void* q, const void* k, const void* v, int F, int N, int H, int d,
                       int precision, void* O_soft, void* workspace, size_t workspace_bytes,
                       void* stream) {
  int s = check_shape(F, N, H, d, precision);
  if (s != VDN_OK) return s;
  if (!q || !k || !v || !O_soft) return VDN_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(O_soft, 16)) return VDN_ERR_INVALID_ARG;
  Layout L;
  if ((s = check_ws(F, N, H, d, precision, workspace, workspace_bytes, &L)) != VDN_OK) return s;
  WsPtr ws{static_cast<unsigned char*>(workspace)};
  return run_softmax(q, k, v, F, N, H, d, precision, O_soft, L, ws, false, nullptr, as_stream(stream));
}

int vdn_vda_states(const void* k, const void* v, const float* beta, int F, int N, int H, int d,
                   int precision, float* S_fwd, float* S_bwd, void* workspace, size_t workspace_bytes,
                   void* stream) {
  int s = check_shape(F, N, H, d, precision);
  if (s != VDN_OK) return s;
  if (!k || !v || !beta || !S_fwd || !S_bwd) return VDN_ERR_INVALID_ARG;
  if (!aligned(k, 16) || !aligned(v, 16) || !aligned(S_fwd, 16) || !aligned(S_bwd, 16)) return VDN_ERR_INVALID_ARG;
  Layout L;
  if ((s = check_ws(F, N, H, d, precision, workspace, workspace_bytes, &L)) != VDN_OK) return s;
  WsPtr ws{static_cast<unsigned char*>(workspace)};
  return run_states(k, v, beta, F, N, H, d, precision, S_fwd, S_bwd, L, ws, as_stream(stream));
}

int vdn_vda_linear(const void* q, const float* S_fwd, const float* S_bwd, int F, int N, int H, int d,
                   int precision, void* O_lin, void* workspace, size_t workspace_bytes, void* stream) {
  int s = check_shape(F, N, H, d, precision);
  if (s != VDN_OK) return s;
  if (!q || !S_fwd || !S_bwd || !O_lin) return VDN_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(O_lin, 16)) return VDN_ERR_INVALID_ARG;
  Layout L;
  if ((s = check_ws(F, N, H, d, precision, workspace, workspace_bytes, &L)) != VDN_OK) return s;
  WsPtr ws{static_cast<unsigned char*>(workspace)};
  const hipStream_t st = as_stream(stream);
  const bool bf16 = precision != VDN_PREC_FP32;
  VDN_STAGE(VDN_STAGE_WPREP, st,
            vdn::launch_wprep(S_fwd, S_bwd, nullptr, vdn::num_chunks(F), H, d, bf16 ? 1 : 0,
                              ws.at<void>(L.W), st));
  const size_t frame_bytes = static_cast<size_t>(N) * H * d * (bf16 ? 2 : 4);
  VDN_TRY(vdn::launch_zero(O_lin, frame_bytes, st));
  if (F >= 2)
    VDN_TRY(vdn::launch_zero(static_cast<unsigned char*>(O_lin) + (F - 1) * frame_bytes, frame_bytes, st));
  VDN_STAGE(VDN_STAGE_READOUT, st,
            vdn::launch_readout(bf16 ? 1 : 0, q, ws.at<void>(L.W), F, N, H, d, O_lin, 0, st));
  return VDN_OK;
}

int vdn_fp8_quantize(const void* x, int F, int N, int H, int d, float prescale, unsigned char* codes,
                     int* scale_exp, void* stream) {
  int s = check_shape(F, N, H, d, VDN_PREC_BF16_FP8QK);
  if (s != VDN_OK) return s;
  if (!x || !codes || !scale_exp) return VDN_ERR_INVALID_ARG;
  if (!(prescale > 0.f) || !std::isfinite(prescale)) return VDN_ERR_INVALID_ARG;
  if (!aligned(x, 16) || !aligned(codes, 8) || !aligned(scale_exp, 4)) return VDN_ERR_INVALID_ARG;
  VDN_TRY(vdn::launch_fp8_quant(static_cast<const uint16_t*>(x), F, N, H, d, prescale, codes, scale_exp,
                                as_stream(stream)));
  return VDN_OK;
}

}  // extern "C"
