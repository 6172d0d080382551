// device.hpp -- gfx950 building blocks shared by the GEMM kernels:
// vector types, buffer resources, MFMA wrappers, the swizzled LDS layout,
// fp32 -> fp16/bf16 packing and the fused epilogue functions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tg {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Element-type tags.
struct F16 {};
struct BF16 {};

// Epilogue codes (same values as tg_epilogue in include/tg.h).
enum : int { EPI_NONE = 0, EPI_BIAS = 1, EPI_RELU = 2, EPI_GELU = 3, EPI_SOFTMAX = 4 };

// ---------------------------------------------------------------------------
// Buffer resources.  A raw (stride 0) descriptor whose range is 2^31 - 1 bytes:
// any offset with bit 31 set lies outside it, and the hardware returns zeros
// for such a load.  Edge tiles use that to zero-fill rows / columns / k beyond
// the matrix without branches.
// ---------------------------------------------------------------------------
constexpr int kOOB = int(0x80000000u);

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base) {
  // word 3 = 0x00020000: 32-bit data format, the usual raw-buffer setting on gfx9.
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, 0x7fffffff, 0x00020000);
}

__device__ __forceinline__ u32x4 buffer_load16(__amdgpu_buffer_rsrc_t r, int byte_off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 0);
}

// ---------------------------------------------------------------------------
// MFMA: D(16x16, fp32) += A(16x32) . B(32x16), one wavefront.
// Operand lane layout (both inputs): lane l holds row (resp. column) l % 16 and
// 8 consecutive k values of k-group l / 16.  The same k order is used for both
// inputs, so any hardware permutation of k inside an instruction cancels.
// Output: lane l holds column l % 16, rows 4 * (l / 16) + i, i = 0..3.
// ---------------------------------------------------------------------------
__device__ __forceinline__ f32x4 mfma16x16x32(F16, const u32x4& a, const u32x4& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0,
                                                 0, 0);
}
__device__ __forceinline__ f32x4 mfma16x16x32(BF16, const u32x4& a, const u32x4& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                  0, 0, 0);
}

// ---------------------------------------------------------------------------
// LDS tile layout for 64-element (128-byte) K rows.
//
// A tile of R rows x 64 k (fp16/bf16) is stored as R/2 lines of 256 bytes,
// two rows per line, in 16-byte slots.  Row r, 16-byte chunk c (k = 8c..8c+7)
// lives in line r/2 at slot
//     ((r & 1) ^ (line >> 2 & 1)) * 8 + (c ^ (line & 7)),   line = r / 2.
// Fragment reads (16 consecutive rows, one chunk) hit 16 distinct slots, i.e.
// all 64 banks once; row writes of 16-byte chunks are conflict-free too, and
// the transposed 8-byte writes of row-major B spread over both halves.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int lds_off64(int row, int chunk) {
  const int line = row >> 1;
  const int slot = ((((row & 1) ^ ((line >> 2) & 1))) << 3) | (chunk ^ (line & 7));
  return (line << 8) | (slot << 4);
}

__device__ __forceinline__ u32x4 lds_read16(const unsigned char* base, int off) {
  return *reinterpret_cast<const u32x4*>(base + off);
}
__device__ __forceinline__ void lds_write16(unsigned char* base, int off, const u32x4& v) {
  *reinterpret_cast<u32x4*>(base + off) = v;
}
__device__ __forceinline__ void lds_write8(unsigned char* base, int off, const u32x2& v) {
  *reinterpret_cast<u32x2*>(base + off) = v;
}

// ---------------------------------------------------------------------------
// Conversions.  Inputs widen exactly; outputs round once, to nearest even
// (v_cvt_f16_f32 and gfx950's v_cvt_pk_bf16_f32 both round to nearest even).
// ---------------------------------------------------------------------------
__device__ __forceinline__ float lo_to_f32(F16, uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu));
}
__device__ __forceinline__ float hi_to_f32(F16, uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
}
__device__ __forceinline__ float lo_to_f32(BF16, uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float hi_to_f32(BF16, uint32_t w) { return __builtin_bit_cast(float, w & 0xffff0000u); }

__device__ __forceinline__ uint32_t pack2(F16, float a, float b) {
  const uint32_t lo = __builtin_bit_cast(uint16_t, (_Float16)a);
  const uint32_t hi = __builtin_bit_cast(uint16_t, (_Float16)b);
  return lo | (hi << 16);
}
__device__ __forceinline__ uint32_t pack2(BF16, float a, float b) {
  const uint32_t lo = __builtin_bit_cast(uint16_t, (__bf16)a);
  const uint32_t hi = __builtin_bit_cast(uint16_t, (__bf16)b);
  return lo | (hi << 16);
}

// ---------------------------------------------------------------------------
// Epilogue activations (fp32).
//
// GELU(x) = x * Phi(x) = 0.5 * x * erfc(-x / sqrt 2).  erfc is evaluated with
// the Chebyshev-fitted approximation "erfcc" of Press, Teukolsky, Vetterling &
// Flannery, Numerical Recipes (2nd ed., section 6.2):
//     erfc(z) ~= t * exp(-z^2 + P(t)),  t = 1 / (1 + z/2),  z >= 0,
// with fractional error below 1.2e-7 for every z >= 0 (relative, so the tail
// for negative x keeps full precision, unlike 1 + erf(x)).  For x < 0,
// Phi(x) = erfc(|x|/sqrt2) / 2; for x >= 0, Phi(x) = 1 - erfc(|x|/sqrt2) / 2.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float gelu_erf(float x) {
  const float z = __builtin_fabsf(x) * 0.70710678118654752f;
  const float t = __builtin_amdgcn_rcpf(__builtin_fmaf(0.5f, z, 1.0f));
  float p = 0.17087277f;
  p = __builtin_fmaf(p, t, -0.82215223f);
  p = __builtin_fmaf(p, t, 1.48851587f);
  p = __builtin_fmaf(p, t, -1.13520398f);
  p = __builtin_fmaf(p, t, 0.27886807f);
  p = __builtin_fmaf(p, t, -0.18628806f);
  p = __builtin_fmaf(p, t, 0.09678418f);
  p = __builtin_fmaf(p, t, 0.37409196f);
  p = __builtin_fmaf(p, t, 1.00002368f);
  p = __builtin_fmaf(p, t, -1.26551223f);
  const float u = __builtin_fmaf(-z, z, p);                          // -z^2 + P(t)
  const float e = __builtin_amdgcn_exp2f(u * 1.4426950408889634f);  // exp(u)
  const float h = (0.5f * x) * (t * e);                              // x * erfc(z) / 2
  return x < 0.0f ? h : x - h;
}

__device__ __forceinline__ float apply_act(int epi, float x) {
  if (epi == EPI_RELU) return __builtin_fmaxf(x, 0.0f);
  if (epi == EPI_GELU) return gelu_erf(x);
  return x;
}

}  // namespace tg
