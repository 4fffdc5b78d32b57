// Shared device-side helpers for the gfx950 kernels: element types, MFMA
// wrappers and the frame arithmetic of the layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace vdn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef int intx8 __attribute__((ext_vector_type(8)));
typedef int intx4 __attribute__((ext_vector_type(4)));
typedef int intx2 __attribute__((ext_vector_type(2)));

// LDS (address space 3) pointer, as the direct global->LDS load builtin takes it;
// convert from a generic pointer into __shared__ memory with an explicit cast
typedef __attribute__((address_space(3))) void* lds_void_ptr;

// Buffer resource for raw byte-offset loads of `bytes` bytes from `base` (gfx9
// word 3: 32-bit data format, no swizzle); offsets past `bytes` read zeros.
__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// 16-byte chunk swizzle for rows of `bytes` bytes in LDS (64 banks x 4 B = 256 B
// per cycle, i.e. 16 lanes of a ds_read_b128): rows that start on the same
// 16-byte bank group get their chunk index XOR-ed with different values, so 16
// consecutive rows read at one logical chunk hit 16 distinct bank groups.
__device__ inline int swz_rows(int r, int bytes) {
  const int rpb = bytes >= 256 ? 1 : 256 / bytes;    // rows per 256-byte bank cycle
  const int nch = bytes / 16 < 16 ? bytes / 16 : 16;
  return (r / rpb) & (nch - 1);
}

constexpr int kChunk = 5;        // latent frames per chunk
constexpr int kWave = 64;

// ---------------------------------------------------------------- frames
// Chunk c covers frames [5c, 5c+5).  The softmax window of a non-anchor query
// frame of chunk c is chunks c-1..c+1 (clipped), i.e. frames
// [max(0, 5(c-1)), min(F, 5(c+2))), plus the two anchor frames 0 and F-1.
__host__ __device__ inline int num_chunks(int F) { return (F + kChunk - 1) / kChunk; }
__host__ __device__ inline int win_first(int c) { return c >= 1 ? kChunk * (c - 1) : 0; }
__host__ __device__ inline int win_end(int c, int F) {
  int e = kChunk * (c + 2);
  return e < F ? e : F;
}
// Non-anchor query frames of chunk c: [nq_first, nq_end).
__host__ __device__ inline int nq_first(int c) { return c == 0 ? 1 : kChunk * c; }
__host__ __device__ inline int nq_end(int c, int F) {
  int e = kChunk * (c + 1);
  return e < F - 1 ? e : F - 1;
}

// ---------------------------------------------------------------- bf16
__device__ inline float bf16_bits_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}
__device__ inline uint32_t pack_bf16x2(float a, float b) {
  bf16x2 v = {(__bf16)a, (__bf16)b};   // v_cvt_pk_bf16_f32, round to nearest even
  return __builtin_bit_cast(uint32_t, v);
}
__device__ inline uint16_t f32_to_bf16_bits(float a) {
  return static_cast<uint16_t>(pack_bf16x2(a, 0.f) & 0xffffu);
}

// ---------------------------------------------------------------- MFMA
// 32x32 output tiles.  Output layout (all 32x32 variants): lane l, element r
// holds C[row = 8*(r/4) + 4*(l/32) + r%4][col = l%32].
// Input layouts: A lane l holds A[row = l%32][k-slots of half l/32],
// B lane l holds B[k-slots of half l/32][col = l%32]; only the pairing of A's and
// B's k-slots matters for the product, so callers may assign any reduction
// index to a slot as long as A and B agree.
__device__ inline floatx16 mfma_bf16(const bf16x8& a, const bf16x8& b, const floatx16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ inline floatx16 mfma_f32(float a, float b, const floatx16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}
// OCP E4M3 x E4M3, 64-deep reduction (32 codes per lane per operand), every
// product scaled by 2^(sa - 127) 2^(sb - 127): sa, sb are E8M0 scale bytes (the
// low byte of each register is used), applied exactly by the matrix core.
__device__ inline floatx16 mfma_fp8_scaled(const intx8& a, const intx8& b, const floatx16& c, int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, sa, 0, sb);
}

// max / sum of x over the lane pair (j, j + 32), in both lanes: v_permlane32_swap
// exchanges the two halves of the wave on the VALU, without an LDS round trip
__device__ inline float pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __builtin_fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float pair_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ inline float wave_max(float x) {
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}
__device__ inline float wave_sum(float x) {
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

}  // namespace vdn
