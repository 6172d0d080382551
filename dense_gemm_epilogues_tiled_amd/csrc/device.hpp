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
// before the barrier that publishes a stage.  gfx950 needs one wait state
// between a scalar write of M0 and an LDS DMA that reads it; the compiler's
// hazard pass cannot see into the asm string, so the s_nop is written here
// (it is what the compiler itself emits around its own LDS-DMA builtin).
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, uint32_t lds_base_uniform, int voff) {
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"(lds_base_uniform), "v"(voff), "s"(r)
               : "memory", "m0");
#pragma clang diagnostic pop
}

// 16-byte store of an output the kernel never reads back, marked
// non-temporal: written once, it streams towards memory instead of waiting in
// L2 for the write-back at the end of the kernel.  Measured against plain
// stores on the same GPU: 2048^3 + bias + GELU (K-split kernel) 0.5 us less
// per launch, the 4096 x 1024 x 128 softmax GEMM 0.64 us less.
template <class T>
__device__ __forceinline__ void store_nt(T* p, const T& v) {
  __builtin_nontemporal_store(v, p);
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

// Two values converted as one two-element vector: one v_cvt_pk_f16_f32 /
// v_cvt_pk_bf16_f32 (round to nearest even) instead of two conversions and a
// shift-or.
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack2(F16, float a, float b) {
  return __builtin_bit_cast(uint32_t, f16x2{(_Float16)a, (_Float16)b});
}
__device__ __forceinline__ uint32_t pack2(BF16, float a, float b) {
  return __builtin_bit_cast(uint32_t, bf16x2{(__bf16)a, (__bf16)b});
}

// ---------------------------------------------------------------------------
// Epilogue activations (fp32).
//
// GELU(x) = x * Phi(x) with Phi(x) = erfc(-x / sqrt 2) / 2 (erf form).  With
// q = erfc(|x| / sqrt 2) / 2, Phi = 1 - q for x >= 0 and q for x < 0, so
//     GELU(x) = max(x, 0) - |x| * q
// for both signs (one max and one fma instead of a select chain).
// erfc(z) is evaluated as t * exp(-z^2 + P(t)), t = 1 / (1 + z/2), the form of
// the Chebyshev-fitted "erfcc" of Numerical Recipes (Press et al., 2nd ed.,
// section 6.2), with our own cubic P, sized to the outputs the epilogue
// rounds to: a weighted minimax fit (linear programming on a grid) of
// ln(erfc(z) e^{z^2} / t) whose relative error in erfc is below 1.2e-4 for
// z <= 4.3 (|x| <= 6.1: every GELU value an fp16 output resolves) and below
// 9.4e-4 up to z = 9 (|x| <= 12.7, the bf16 tail), against half an output
// ulp of at least 2.4e-4 (fp16) and 2.0e-3 (bf16); tests/test_device_math.py
// checks both bounds against scipy.special.erfc and the fp32 evaluation
// against x Phi(x).  A rounded result is therefore never more than one ulp
// from the correctly rounded GELU.  Relative accuracy holds in the negative
// tail, where 1 + erf(x) would cancel.
// The constants below fold log2(e) and the factor 1/2 into P so that
// exp2(fma(-zz, zz, P2(t))) = exp(-z^2 + P(t)) / 2, zz = |x| sqrt(log2(e) / 2).
// ---------------------------------------------------------------------------
// Natural-log coefficients of P (t^0 .. t^3), as fitted:
//   -1.25433464, 0.894261401, 0.7242145, -0.364253358
__device__ __forceinline__ float gelu_erf(float x) {
  const float ax = __builtin_fabsf(x);
  const float t = __builtin_amdgcn_rcpf(__builtin_fmaf(ax, 0.353553391f, 1.0f));  // 1 / (1 + z/2), z = |x|/sqrt2
  float p = -0.525506513f;                                                         // log2(e) * P(t) - 1
  p = __builtin_fmaf(p, t, 1.04482067f);
  p = __builtin_fmaf(p, t, 1.29014649f);
  p = __builtin_fmaf(p, t, -2.80962236f);
  const float zz = ax * 0.849321800f;                              // |x| * sqrt(log2(e) / 2)
  const float q = t * __builtin_amdgcn_exp2f(__builtin_fmaf(-zz, zz, p));  // erfc(|x|/sqrt2) / 2
  return __builtin_fmaf(-ax, q, __builtin_fmaxf(x, 0.0f));
}

__device__ __forceinline__ float apply_act(int epi, float x) {
  if (epi == EPI_RELU) return __builtin_fmaxf(x, 0.0f);
  if (epi == EPI_GELU) return gelu_erf(x);
  return x;
}

}  // namespace tg
