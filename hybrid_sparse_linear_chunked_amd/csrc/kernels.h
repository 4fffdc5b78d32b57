// Launchers of the device kernels (attn.hip, vda.hip), called by api.cpp.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace vdn {

// proj.hip: Y[M, N] = A[M, K] B[N, K]^T (bf16, fp32 accumulation); K % 64 == 0, N % 8 == 0
hipError_t launch_proj(const uint16_t* A, const uint16_t* B, int M, int N, int K, uint16_t* Y, hipStream_t st);

// attn.hip
hipError_t launch_prep(const uint16_t* k, const uint16_t* v, int F, int N, int H, int D,
                       uint16_t* vt, float* G, float* B, int grams, hipStream_t st);
hipError_t launch_attn(int prec, const void* q, const void* k, const void* v, const uint16_t* vt,
                       const uint8_t* q8, const uint8_t* k8, const float* amax, int F, int N, int H,
                       int D, void* O, float* part_O, float* part_ml, const uint16_t* W,
                       int T, const uint16_t* vtx, int split, float* px, hipStream_t st);
hipError_t launch_combine(int prec, const float* part_O, const float* part_ml, int F, int N, int T,
                          int H, int D, void* O, int split, hipStream_t st);
hipError_t launch_fp8_quant(const uint16_t* x, int F, int N, int H, int D, uint8_t* codes,
                            float* amax, hipStream_t st);
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
