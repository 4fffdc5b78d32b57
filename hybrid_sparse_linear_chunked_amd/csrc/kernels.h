// Launchers of the device kernels (attn.hip, vda.hip), called by api.cpp.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <atomic>
#include <cmath>

namespace vdn {

// One-time opt-in of kernel `fn` to `lds` bytes of dynamic LDS on the current
// device.  `done` holds one bit per device id (ids from 64 up set the attribute on
// every call); the atomic makes first calls from several threads well defined,
// and setting the same value twice is harmless.
inline hipError_t set_max_lds_once(const void* fn, int lds, std::atomic<unsigned long long>* done) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const unsigned long long bit = dev >= 0 && dev < 64 ? (1ull << dev) : 0ull;
  if (bit != 0 && (done->load(std::memory_order_acquire) & bit) != 0) return hipSuccess;
  e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (e != hipSuccess) return e;
  if (bit != 0) done->fetch_or(bit, std::memory_order_release);
  return hipSuccess;
}

// proj.hip: Y[M, N] = A[M, K] B[N, K]^T (bf16, fp32 accumulation); K % 64 == 0, N % 8 == 0
// qctr: 8 ints of scratch for the tile queues (cleared by the launch), or null for
// the static block -> tile map
hipError_t launch_proj(const uint16_t* A, const uint16_t* B, int M, int N, int K, uint16_t* Y, hipStream_t st,
                       int* qctr = nullptr);
// p[0, n) = value (a kernel, so that it can sit in a captured graph)
hipError_t launch_fill_u32(uint32_t* p, int n, uint32_t value, hipStream_t st);

// attn.hip
// vt8 (optional): V^T as E4M3 codes in the vt8 layout, with scale exponents vexp [H],
// instead of bf16 vt
hipError_t launch_prep(const uint16_t* k, const uint16_t* v, int F, int N, int H, int D,
                       uint16_t* vt, float* G, float* B, int grams, hipStream_t st, uint8_t* vt8 = nullptr,
                       const int* vexp = nullptr);
// qctr: 8 ints of scratch for the bf16 / fp8 kernel's item queues (cleared by the
// launch), or null for the static block -> item map
hipError_t launch_attn(int prec, const void* q, const void* k, const void* v, const uint16_t* vt,
                       const uint8_t* q8, const uint8_t* k8, const int* fexp, int F, int N, int H,
                       int D, void* O, float* part_O, float* part_ml, const uint16_t* W,
                       int T, const uint16_t* vtx, int split, float* px, int* qctr, hipStream_t st);
hipError_t launch_combine(int prec, const float* part_O, const float* part_ml, int F, int N, int T,
                          int H, int D, void* O, int split, hipStream_t st);
// The softmax temperature in base-2 units, log2(e) / sqrt(d), in fp32 (the bf16
// Q operand and the fp8 q codes carry it)
inline float softmax_temperature_log2(int d) { return 1.4426950408889634f / sqrtf(static_cast<float>(d)); }
// per-head power-of-two scale exponents of fp32(x * prescale) into fexp [H]
hipError_t launch_fp8_scale(const uint16_t* x, int F, int N, int H, int D, float prescale, int* fexp,
                            hipStream_t st);
hipError_t launch_fp8_quant(const uint16_t* x, int F, int N, int H, int D, float prescale, uint8_t* codes,
                            int* fexp, hipStream_t st);
void attn_split_plan(int F, int* nsplit, int* fs);

// vda.hip
hipError_t launch_gram_f32(const float* k, const float* v, int F, int N, int H, int D, float* G,
                           float* B, hipStream_t st);
hipError_t launch_factor(float* G, float* B, const float* beta, int F, int H, int D, hipStream_t st);
hipError_t launch_scan(const float* M, const float* Cm, int F, int H, int D, float* Sf, float* Sb,
                       hipStream_t st);
hipError_t launch_wprep(const float* Sf, const float* Sb, const float* gate, int C, int H, int D,
                        int bf16, void* W, hipStream_t st);
hipError_t launch_readout(int prec, const void* q, const void* W, int F, int N, int H, int D,
                          void* O, int accumulate, hipStream_t st);
hipError_t launch_zero(void* p, size_t bytes, hipStream_t st);

}  // namespace vdn
