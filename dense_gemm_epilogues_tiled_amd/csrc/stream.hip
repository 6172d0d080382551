// stream.hip -- the tutorial's two bandwidth-bound kernels for gfx950:
//
//   * vector addition C[i] = A[i] + B[i] (noticiai.com.br, section "Adicao de
//     vetores: o 'Hello World' dos kernels": one element per thread behind a
//     bounds check; the edgex.exchange page's opening paragraph);
//   * the standalone row softmax Y = softmax(alpha X) per row (noticiai.com.br,
//     section "Softmax por linha e FlashAttention": row max, subtract,
//     exponentiate, normalise).
//
// Both are bound by HBM bandwidth, so the design is about moving bytes: every
// lane moves 16-byte vectors, consecutive lanes touch consecutive vectors,
// several loads are in flight per lane before any result is needed, and every
// element is read and written exactly once.  Arithmetic is fp32; fp16 / bf16
// results are rounded once, to nearest even.

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

// Grid-stride loop over 16-byte vectors, UNROLL vectors per thread per trip
// (all loads issued before the first add); the last n % per-vector elements
// are added one by one by the first threads of the grid.
template <class DT, int ESIZE>
__global__ __launch_bounds__(256) void vector_add_kernel(VectorAddParams p) {
  constexpr int UNROLL = 4;
  constexpr int EPV = 16 / ESIZE;  // elements per vector
  // no __restrict__: C may be A or B (in place; each element is read and
  // then written by the same lane)
  const u32x4* A = static_cast<const u32x4*>(p.A);
  const u32x4* B = static_cast<const u32x4*>(p.B);
  u32x4* C = static_cast<u32x4*>(p.C);
  const int64_t nvec = p.n / EPV;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (; i + (UNROLL - 1) * stride < nvec; i += UNROLL * stride) {
    u32x4 a[UNROLL], b[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      a[u] = A[i + u * stride];
      b[u] = B[i + u * stride];
    }
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) C[i + u * stride] = add16(DT{}, a[u], b[u]);
  }
  for (; i < nvec; i += stride) C[i] = add16(DT{}, A[i], B[i]);
  // tail: elements nvec * EPV .. n - 1
  const int64_t t = nvec * EPV + (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
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

template <class DT, int ESIZE>
static hipError_t launch_vector_add(const VectorAddParams& p, hipStream_t stream) {
  constexpr int EPV = 16 / ESIZE;
  const int64_t nvec = p.n / EPV;
  // enough workgroups to keep every CU's memory pipeline full (8 per CU),
  // fewer when the vector is short; at least one, for the tail
  int64_t blocks = (nvec + 255) / 256;
  if (blocks > 256 * 8) blocks = 256 * 8;
  if (blocks < 1) blocks = 1;
  void* args[] = {const_cast<VectorAddParams*>(&p)};
  return hipLaunchKernel(reinterpret_cast<const void*>(&vector_add_kernel<DT, ESIZE>), dim3((unsigned)blocks),
                         dim3(256), args, 0, stream);
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
// Chunk c of lane l holds elements [(64 c + l) E, +E) of its row (E = 16 /
// element size): one 16-byte load per chunk, consecutive lanes reading
// consecutive 16 bytes.  The whole row stays in registers (CH chunks per
// lane), so X is read once and Y written once.
__device__ __forceinline__ void chunk_to_f32(F32, const u32x4& v, float (&x)[8]) {
#pragma unroll
  for (int e = 0; e < 4; ++e) x[e] = as_f32(v[e]);
}
template <class DT>
__device__ __forceinline__ void chunk_to_f32(DT, const u32x4& v, float (&x)[8]) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    x[2 * e] = lo_to_f32(DT{}, v[e]);
    x[2 * e + 1] = hi_to_f32(DT{}, v[e]);
  }
}

template <class DT, int ESIZE, int CH>
__global__ __launch_bounds__(256) void row_softmax_kernel(RowSoftmaxParams p) {
  constexpr int E = 16 / ESIZE;  // elements per chunk
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= p.rows) return;  // whole waves: no barrier below
  const int64_t cols = p.cols;
  const u32x4* __restrict__ X = reinterpret_cast<const u32x4*>(static_cast<const unsigned char*>(p.X) +
                                                                row * cols * ESIZE);
  float* __restrict__ Y = p.Y + row * cols;
  // t = alpha x rounded once; the max is taken over t and exp(t - m) is
  // formed as exp2((t - m) log2 e): t - m is exact near the max (Sterbenz),
  // so the largest entry gets exp2(0) = 1 at any magnitude of t.
  const float alpha = p.alpha;
  constexpr float kLog2e = 1.4426950408889634f;

  u32x4 v[CH];
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int64_t first = (int64_t)(64 * c + lane) * E;
    v[c] = first < cols ? X[64 * c + lane] : u32x4{0u, 0u, 0u, 0u};
  }
  // row max of t (alpha may be negative: scale before the max)
  float m = -__builtin_inff();
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    float x[8];
    chunk_to_f32(DT{}, v[c], x);
    const int64_t first = (int64_t)(64 * c + lane) * E;
#pragma unroll
    for (int e = 0; e < E; ++e)
      if (first + e < cols) m = __builtin_fmaxf(m, x[e] * alpha);
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) m = __builtin_fmaxf(m, __shfl_xor(m, o));
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    float x[8];
    chunk_to_f32(DT{}, v[c], x);
    const int64_t first = (int64_t)(64 * c + lane) * E;
#pragma unroll
    for (int e = 0; e < E; ++e)
      if (first + e < cols) s += __builtin_amdgcn_exp2f((x[e] * alpha - m) * kLog2e);
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) s += __shfl_xor(s, o);
  const float inv = __builtin_amdgcn_rcpf(s);
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    float x[8];
    chunk_to_f32(DT{}, v[c], x);
    const int64_t first = (int64_t)(64 * c + lane) * E;
    if (first < cols) {  // cols is a multiple of E: a chunk is wholly in or out
#pragma unroll
      for (int h = 0; h < E / 4; ++h) {
        f32x4 y;
#pragma unroll
        for (int e = 0; e < 4; ++e) y[e] = __builtin_amdgcn_exp2f((x[4 * h + e] * alpha - m) * kLog2e) * inv;
        *reinterpret_cast<f32x4*>(Y + first + 4 * h) = y;
      }
    }
  }
}

template <class DT, int ESIZE, int CH>
static hipError_t launch_row_softmax(const RowSoftmaxParams& p, hipStream_t stream) {
  void* args[] = {const_cast<RowSoftmaxParams*>(&p)};
  return hipLaunchKernel(reinterpret_cast<const void*>(&row_softmax_kernel<DT, ESIZE, CH>),
                         dim3((unsigned)((p.rows + 3) / 4)), dim3(256), args, 0, stream);
}

template <class DT, int ESIZE>
static RowSoftmaxFn pick_row_softmax(int64_t cols) {
  constexpr int E = 16 / ESIZE;
  if (cols <= 64 * E * 1) return &launch_row_softmax<DT, ESIZE, 1>;
  if (cols <= 64 * E * 2) return &launch_row_softmax<DT, ESIZE, 2>;
  if (cols <= 64 * E * 4) return &launch_row_softmax<DT, ESIZE, 4>;
  if (cols <= 64 * E * 8) return &launch_row_softmax<DT, ESIZE, 8>;
  if (cols <= 64 * E * 16) return &launch_row_softmax<DT, ESIZE, 16>;
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
