// stream.hip -- the tutorial's two bandwidth-bound kernels for gfx950:
//
//   * vector addition C[i] = A[i] + B[i] (noticiai.com.br, section "Adicao de
//     vetores: o 'Hello World' dos kernels": one element per thread behind a
//     bounds check; the edgex.exchange page's opening paragraph);
//   * the standalone row softmax Y = softmax(alpha X) per row (noticiai.com.br,
//     section "Softmax por linha e FlashAttention": row max, subtract,
//     exponentiate, normalise).
//
// Both are bound by HBM bandwidth, so the design is about moving bytes:
// consecutive lanes touch consecutive bytes, every wave issues all its loads
// before it needs any of them, every element is read and written exactly
// once, and the outputs are written with non-temporal stores.  Arithmetic is
// fp32; fp16 / bf16 results are rounded once, to nearest even.

#include "device.hpp"
#include "kernels.hpp"

namespace tg {

struct F32 {};

// Bit casts between a 32-bit word and an fp32 value.  The word is taken by
// value on purpose: hipcc's __builtin_bit_cast applied directly to an element
// of an ext_vector_type (v[e]) reads element 0 whatever e is, so vector
// elements always pass through these.
__device__ __forceinline__ float as_f32(uint32_t w) { return __builtin_bit_cast(float, w); }
__device__ __forceinline__ uint32_t as_u32(float f) { return __builtin_bit_cast(uint32_t, f); }

// ---------------------------------------------------------------------------
// Vector addition.
// ---------------------------------------------------------------------------
__device__ __forceinline__ u32x4 add16(F32, const u32x4& a, const u32x4& b) {
  u32x4 r;
#pragma unroll
  for (int e = 0; e < 4; ++e)
    r[e] = as_u32(as_f32(a[e]) + as_f32(b[e]));
  return r;
}
// Two 16-bit values per word: widen exactly, add in fp32, round once.  The fp32
// sum of two fp16 (bf16) values rounded to fp16 (bf16) is the correctly rounded
// sum: fp32 has 24 >= 2 * 11 + 2 (2 * 8 + 2) significand bits, so its own
// rounding cannot move the final one.
template <class DT>
__device__ __forceinline__ u32x4 add16(DT, const u32x4& a, const u32x4& b) {
  u32x4 r;
#pragma unroll
  for (int e = 0; e < 4; ++e)
    r[e] = pack2(DT{}, lo_to_f32(DT{}, a[e]) + lo_to_f32(DT{}, b[e]), hi_to_f32(DT{}, a[e]) + hi_to_f32(DT{}, b[e]));
  return r;
}

__device__ __forceinline__ uint32_t add_scalar(F32, uint32_t a, uint32_t b) {
  return as_u32(as_f32(a) + as_f32(b));
}
template <class DT>
__device__ __forceinline__ uint32_t add_scalar(DT, uint32_t a, uint32_t b) {  // low 16 bits only
  return pack2(DT{}, lo_to_f32(DT{}, a) + lo_to_f32(DT{}, b), 0.f) & 0xffffu;
}

// One 16-byte vector per thread over a grid that covers the whole vector (no
// loop: every wave issues its loads at once, and consecutive blocks stream
// consecutive 4 KiB pieces, spread evenly over the HBM channels); the last
// n % (elements per vector) elements go one per thread to the threads just
// past the last vector.  Stores are non-temporal.  Loads are non-temporal too
// when the three arrays far exceed the last-level cache (NT_LOAD): there,
// measured on MI355X, it lifts the stream from ~6.3 to ~6.8 TB/s, while for
// cache-sized vectors plain loads are faster.
template <class DT, int ESIZE, int BS, bool NT_LOAD>
__global__ __launch_bounds__(BS) void vector_add_kernel(VectorAddParams p) {
  constexpr int EPV = 16 / ESIZE;  // elements per vector
  const int64_t nvec = p.n / EPV;
  const int64_t j = (int64_t)blockIdx.x * BS + threadIdx.x;
  if (j < nvec) {
    // no __restrict__: C may be A or B (in place; each element is read and
    // then written by the same lane)
    const u32x4* A = static_cast<const u32x4*>(p.A);
    const u32x4* B = static_cast<const u32x4*>(p.B);
    u32x4 a, b;
    if constexpr (NT_LOAD) {
      a = __builtin_nontemporal_load(A + j);
      b = __builtin_nontemporal_load(B + j);
    } else {
      a = A[j];
      b = B[j];
    }
    __builtin_nontemporal_store(add16(DT{}, a, b), static_cast<u32x4*>(p.C) + j);
    return;
  }
  const int64_t t = nvec * EPV + (j - nvec);  // tail element
  if (t < p.n) {
    if constexpr (ESIZE == 4) {
      const uint32_t* a = static_cast<const uint32_t*>(p.A);
      const uint32_t* b = static_cast<const uint32_t*>(p.B);
      static_cast<uint32_t*>(p.C)[t] = add_scalar(DT{}, a[t], b[t]);
    } else {
      const uint16_t* a = static_cast<const uint16_t*>(p.A);
      const uint16_t* b = static_cast<const uint16_t*>(p.B);
      static_cast<uint16_t*>(p.C)[t] = (uint16_t)add_scalar(DT{}, a[t], b[t]);
    }
  }
}

// Bytes moved (A, B read, C written) up to which the cache-sized form is used.
constexpr int64_t kVectorAddCachedBytes = int64_t(512) << 20;

template <class DT, int ESIZE>
static hipError_t launch_vector_add(const VectorAddParams& p, hipStream_t stream) {
  constexpr int EPV = 16 / ESIZE;
  const int64_t nvec = p.n / EPV;
  const int64_t items = nvec + (p.n - nvec * EPV);
  void* args[] = {const_cast<VectorAddParams*>(&p)};
  if (3 * p.n * ESIZE <= kVectorAddCachedBytes)
    return hipLaunchKernel(reinterpret_cast<const void*>(&vector_add_kernel<DT, ESIZE, 256, false>),
                           dim3((unsigned)((items + 255) / 256)), dim3(256), args, 0, stream);
  return hipLaunchKernel(reinterpret_cast<const void*>(&vector_add_kernel<DT, ESIZE, 64, true>),
                         dim3((unsigned)((items + 63) / 64)), dim3(64), args, 0, stream);
}

__host__ VectorAddFn vector_add_launcher(int dtype) {
  switch (dtype) {
    case TG_DTYPE_F16: return &launch_vector_add<F16, 2>;
    case TG_DTYPE_BF16: return &launch_vector_add<BF16, 2>;
    case TG_DTYPE_F32: return &launch_vector_add<F32, 4>;
    default: return nullptr;
  }
}

// ---------------------------------------------------------------------------
// Standalone row softmax.
// ---------------------------------------------------------------------------
// One wave per row, four rows per workgroup.  Chunk c of lane l holds the
// four elements [4 (64 c + l), +4) of its row: an 8-byte load for fp16 / bf16
// (16 bytes for fp32), so that its four fp32 results are one 16-byte store
// and every store instruction of the wave writes 1 KiB contiguously.  The
// whole row stays in registers (CH chunks per lane): X is read once, Y
// written once.  Loads and stores go through buffer resources whose range is
// exactly the row: chunks past the row's end read zeros and their stores are
// dropped by the hardware, so the kernel has no branches on the column index
// (guarded loads made the compiler copy the whole register array at every
// branch).  Y stores are non-temporal: measured on MI355X, the 16384 x 4096
// fp16 row softmax streams at ~6.9 TB/s this way against ~5.4 with plain
// stores.
template <int ESIZE>
struct Chunk;
template <>
struct Chunk<2> {  // four 16-bit elements
  u32x2 w;
  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t r, int off) {
    w = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
  }
  template <class DT>
  __device__ __forceinline__ float get(DT, int e) const {
    return (e & 1) ? hi_to_f32(DT{}, w[e >> 1]) : lo_to_f32(DT{}, w[e >> 1]);
  }
};
template <>
struct Chunk<4> {  // four fp32 elements
  u32x4 w;
  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t r, int off) {
    w = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
  }
  template <class DT>
  __device__ __forceinline__ float get(DT, int e) const { return as_f32(w[e]); }
};

// Cache-policy bits of a buffer instruction on gfx950: 2 = non-temporal.
constexpr int kCpolNT = 2;

// RECOMP: the output pass recomputes the conversions and exponentials
// instead of keeping the sum pass's values live (an empty asm statement that
// "modifies" the chunks and the max hides them from common-subexpression
// elimination): half the registers, twice the exp2 work.
template <class DT, int ESIZE, int CH, bool RECOMP>
__global__ __launch_bounds__(256) void row_softmax_kernel(RowSoftmaxParams p) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= p.rows) return;  // whole waves: no barrier below
  const int64_t cols = p.cols;
  const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<unsigned char*>(static_cast<const unsigned char*>(p.X) + row * cols * ESIZE), (short)0,
      (int)(cols * ESIZE), 0x00020000);
  const __amdgpu_buffer_rsrc_t yr =
      __builtin_amdgcn_make_buffer_rsrc(p.Y + row * cols, (short)0, (int)(cols * 4), 0x00020000);
  // t = alpha x rounded once; the max is taken over t and exp(t - m) is
  // formed as exp2((t - m) log2 e): t - m is exact near the max (Sterbenz),
  // so the largest entry gets exp2(0) = 1 at any magnitude of t.
  const float alpha = p.alpha;
  constexpr float kLog2e = 1.4426950408889634f;

  Chunk<ESIZE> v[CH];
#pragma unroll
  for (int c = 0; c < CH; ++c) v[c].load(xr, (64 * c + lane) * 4 * ESIZE);
  // cols is a multiple of 4: a chunk is wholly inside the row or wholly past it
  // row max of t (alpha may be negative: scale before the max)
  float m = -__builtin_inff();
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    float t = v[c].get(DT{}, 0) * alpha;
#pragma unroll
    for (int e = 1; e < 4; ++e) t = __builtin_fmaxf(t, v[c].get(DT{}, e) * alpha);
    m = __builtin_fmaxf(m, (64 * c + lane) * 4 < cols ? t : -__builtin_inff());
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) m = __builtin_fmaxf(m, __shfl_xor(m, o));
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    float sc = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) sc += __builtin_amdgcn_exp2f((v[c].get(DT{}, e) * alpha - m) * kLog2e);
    s += (64 * c + lane) * 4 < cols ? sc : 0.f;
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) s += __shfl_xor(s, o);
  const float inv = __builtin_amdgcn_rcpf(s);
  if constexpr (RECOMP) {
    asm volatile("" : "+v"(m));
#pragma unroll
    for (int c = 0; c < CH; ++c) asm volatile("" : "+v"(v[c].w));
  }
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    f32x4 y;
#pragma unroll
    for (int e = 0; e < 4; ++e) y[e] = __builtin_amdgcn_exp2f((v[c].get(DT{}, e) * alpha - m) * kLog2e) * inv;
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, y), yr, (64 * c + lane) * 16, 0, kCpolNT);
  }
}

template <class DT, int ESIZE, int CH>
static hipError_t launch_row_softmax(const RowSoftmaxParams& p, hipStream_t stream) {
  void* args[] = {const_cast<RowSoftmaxParams*>(&p)};
  return hipLaunchKernel(reinterpret_cast<const void*>(&row_softmax_kernel<DT, ESIZE, CH, (CH >= 32)>),
                         dim3((unsigned)((p.rows + 3) / 4)), dim3(256), args, 0, stream);
}

// The fewest chunks (of 256 elements per wave) that cover the row.
template <class DT, int ESIZE>
static RowSoftmaxFn pick_row_softmax(int64_t cols) {
  if (cols <= 256 * 1) return &launch_row_softmax<DT, ESIZE, 1>;
  if (cols <= 256 * 2) return &launch_row_softmax<DT, ESIZE, 2>;
  if (cols <= 256 * 4) return &launch_row_softmax<DT, ESIZE, 4>;
  if (cols <= 256 * 8) return &launch_row_softmax<DT, ESIZE, 8>;
  if (cols <= 256 * 16) return &launch_row_softmax<DT, ESIZE, 16>;
  if constexpr (ESIZE == 2)
    if (cols <= 256 * 32) return &launch_row_softmax<DT, ESIZE, 32>;
  return nullptr;
}

__host__ RowSoftmaxFn row_softmax_launcher(int dtype, int64_t cols) {
  switch (dtype) {
    case TG_DTYPE_F16: return pick_row_softmax<F16, 2>(cols);
    case TG_DTYPE_BF16: return pick_row_softmax<BF16, 2>(cols);
    case TG_DTYPE_F32: return pick_row_softmax<F32, 4>(cols);
    default: return nullptr;
  }
}

}  // namespace tg
