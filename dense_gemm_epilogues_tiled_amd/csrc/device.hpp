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
// LDS tile layouts.  LDS has 64 four-byte banks: one 256-byte window.
//
// K-contiguous tiles (A, and B stored N x K): R rows x BK k of 16-bit values,
// row r at r * 2BK bytes, 16-byte chunk c (k = 8c .. 8c+7) stored in slot
//     c ^ ((r / (16 / KCH)) % KCH),      KCH = BK / 8 chunks per row.
// A fragment read touches 16 consecutive rows at one chunk; the XOR spreads
// them over 16 distinct 16-byte slots of the 256-byte bank window.
//
// N-contiguous tiles (B stored K x N, BN >= 128): row k at k * 2BN bytes,
// 16-byte chunk c (n = 8c .. 8c+7) stored in slot
//     ((c / 2) ^ s(k)) * 2 + (c % 2),    s(k) = (k % 4) + 4 * ((k / 8) % 2).
// ds_read_b64_tr_b16 fragment reads touch 8 rows x 32 bytes per half-wave;
// the XOR puts those 8 pairs of chunks in distinct slots.
// ---------------------------------------------------------------------------
template <int BK>
__device__ __forceinline__ int kc_off(int row, int chunk) {
  constexpr int KCH = BK / 8;
  constexpr int R = 16 / KCH;
  return row * (BK * 2) + 16 * (chunk ^ ((row / R) % KCH));
}

__device__ __forceinline__ int nc_swz(int k) { return (k & 3) | (((k >> 3) & 1) << 2); }

template <int BN>
__device__ __forceinline__ int nc_off(int k, int chunk) {
  return k * (BN * 2) + 16 * ((((chunk >> 1) ^ nc_swz(k)) << 1) | (chunk & 1));
}

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

__device__ __forceinline__ u32x4 lds_read16(const unsigned char* base, int off) {
  return *reinterpret_cast<const u32x4*>(base + off);
}

// Transposing LDS read (gfx950): within each 16-lane group, lane j supplies
// the address of 4 consecutive 16-bit values; lane i receives element i % 4 of
// lanes i/4, 4 + i/4, 8 + i/4, 12 + i/4.  When lanes 4q .. 4q+3 point at the
// four 8-byte pieces of a 16-wide row q, lane i ends with column i of rows 0..3.
__device__ __forceinline__ u32x2 lds_read_tr8(const unsigned char* base, int off) {
  typedef __attribute__((address_space(3))) unsigned char lds_u8;
  lds_u8* q = (lds_u8*)(unsigned char*)(base + off);  // generic -> LDS address space
  const v4i16 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)q);
  return __builtin_bit_cast(u32x2, v);
}

// Byte address of a shared-memory object as seen by LDS instructions / M0.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  typedef __attribute__((address_space(3))) unsigned char lds_u8;
  return (uint32_t)(uintptr_t)(lds_u8*)(unsigned char*)p;
}

// Direct global -> LDS copy of 16 bytes per lane (gfx950 buffer_load_dwordx4
// ... lds): lane i's bytes land at LDS address m0 + 16 i.  Out-of-range
// offsets (kOOB) write zeros.  Issued as inline asm so the compiler does not
// model these LDS writes: completion is tracked explicitly with vmcnt waits
// before the barrier that publishes a stage.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, uint32_t lds_base_uniform, int voff) {
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"(lds_base_uniform), "v"(voff), "s"(r)
               : "memory", "m0");
#pragma clang diagnostic pop
}

// Wait until at most N vector-memory operations of this wave are in flight
// and all its LDS operations are done, then join the workgroup barrier.
template <int N>
__device__ __forceinline__ void wait_vm_barrier() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" : : "n"(N) : "memory");
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
