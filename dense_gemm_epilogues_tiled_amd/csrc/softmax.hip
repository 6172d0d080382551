// softmax.hip -- GEMM with a fused row softmax epilogue for gfx950 (MI355X).
//
//   C[m, n] = exp(x[m, n] - max_j x[m, j]) / sum_j exp(x[m, j] - max_j x[m, j]),
//   x = alpha * A.B
//
// The row softmax is the one of the TileLang tutorial ("TileLang: Criando
// Kernels de GPU de Alto Desempenho ...", noticiai.com.br, section "Softmax
// por linha e FlashAttention": per-row max, subtract, exponentiate,
// normalise), applied in the GEMM epilogue so the product never reaches
// global memory ("Designing High-Performance GPU Kernels with TileLang ...",
// spaxe.top, fused-softmax paragraph), with the reductions kept in registers
// (edgex.exchange page, fused-epilogue paragraph).
//
// gfx950 realisation: a workgroup owns 16 whole rows.  Its WAVES wave64s
// split the row into contiguous column ranges of n_sub 16-wide MFMA tiles
// each; a wave keeps all of its n_sub 16x16 fp32 accumulator tiles in
// registers.  Operand fragments come straight from HBM/L2 into registers with
// 128-bit buffer loads (no LDS: no two waves share a B column), one K step
// ahead of the MFMAs.  The row max and row sum are reduced first inside each
// lane, then across the 4 lanes sharing a row (lane xor 16, xor 32), then
// across waves through a few bytes of LDS.  exp uses v_exp_f32 (2^x) on
// (x - max) * log2(e).  Each lane writes 4 consecutive fp32 per tile.

#include "device.hpp"
#include "kernels.hpp"

namespace tg {

template <int WAVES, int MAX_SUB, bool B_COL, class DT>
__global__ __launch_bounds__(WAVES * 64, 1) void gemm_softmax_kernel(SoftmaxParams p) {
  __shared__ float red_max[WAVES][16];
  __shared__ float red_sum[WAVES][16];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int fr = lane & 15, fk = lane >> 4;
  const int M = p.M, N = p.N, K = p.K;
  const int n_sub = p.n_sub;
  const int m0 = blockIdx.x * 16;
  const int col0 = wave * n_sub * 16;  // first column of this wave

  const uint16_t* __restrict__ gA = static_cast<const uint16_t*>(p.A);
  const uint16_t* __restrict__ gB = static_cast<const uint16_t*>(p.B);
  const __amdgpu_buffer_rsrc_t rA = make_rsrc(gA + (size_t)m0 * K);
  const bool a_row_ok = (m0 + fr) < M;

  f32x4 acc[MAX_SUB];
#pragma unroll
  for (int s = 0; s < MAX_SUB; ++s) acc[s] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int KB = (K + 31) / 32;  // 32-deep MFMA steps

  // fragment loads of one K step
  auto load_a = [&](int kb) -> u32x4 {
    const int k = kb * 32 + fk * 8;
    const bool ok = a_row_ok && k < K;
    return buffer_load16(rA, ok ? (fr * K + k) * 2 : kOOB);
  };
  // B offsets stay 32-bit: the descriptor is rebased at this wave's first
  // column (column-major B) or at the K step's first row (row-major B).
  const __amdgpu_buffer_rsrc_t rBc = make_rsrc(gB + (size_t)col0 * K);
  auto load_b = [&](int kb, int s) -> u32x4 {
    const int nl = s * 16 + fr;  // column inside this wave's range
    const int k = kb * 32 + fk * 8;
    const bool ok = (s < n_sub) && (col0 + nl) < N && k < K;
    if constexpr (B_COL) {
      // B stored N x K: the 8 k values of column n are contiguous
      return buffer_load16(rBc, ok ? (nl * K + k) * 2 : kOOB);
    } else {
      // B stored K x N: gather the 8 k values of column n (stride N)
      const __amdgpu_buffer_rsrc_t rBr = make_rsrc(gB + (size_t)kb * 32 * N);
      const int n = col0 + nl, kl = fk * 8;
      u32x4 v;
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        const bool ok0 = ok && (k + 2 * h) < K, ok1 = ok && (k + 2 * h + 1) < K;
        const int o0 = ok0 ? ((kl + 2 * h) * N + n) * 2 : kOOB;
        const int o1 = ok1 ? ((kl + 2 * h + 1) * N + n) * 2 : kOOB;
        const uint32_t lo = __builtin_bit_cast(uint16_t, __builtin_amdgcn_raw_buffer_load_b16(rBr, o0, 0, 0));
        const uint32_t hi = __builtin_bit_cast(uint16_t, __builtin_amdgcn_raw_buffer_load_b16(rBr, o1, 0, 0));
        v[h] = lo | (hi << 16);
      }
      return v;
    }
  };

  if (KB > 0) {
    u32x4 a_cur = load_a(0);
    u32x4 b_cur[MAX_SUB];
#pragma unroll
    for (int s = 0; s < MAX_SUB; ++s) b_cur[s] = load_b(0, s);
    for (int kb = 0; kb < KB; ++kb) {
      const bool more = (kb + 1) < KB;
      u32x4 a_nxt = a_cur;
      u32x4 b_nxt[MAX_SUB];
      if (more) {
        a_nxt = load_a(kb + 1);
#pragma unroll
        for (int s = 0; s < MAX_SUB; ++s) b_nxt[s] = load_b(kb + 1, s);
      }
#pragma unroll
      for (int s = 0; s < MAX_SUB; ++s) acc[s] = mfma16x16x32(DT{}, b_cur[s], a_cur, acc[s]);
      if (more) {
        a_cur = a_nxt;
#pragma unroll
        for (int s = 0; s < MAX_SUB; ++s) b_cur[s] = b_nxt[s];
      }
    }
  }

  // ---- row softmax on the accumulators ----
  // lane holds row m0 + fr, columns col0 + 16 s + 4 fk + i
  const float alpha = p.alpha;
  const float NEG_INF = -__builtin_inff();
  float mx = NEG_INF;
#pragma unroll
  for (int s = 0; s < MAX_SUB; ++s) {
    const int nb = col0 + s * 16 + 4 * fk;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bool ok = (s < n_sub) && (nb + i) < N;
      const float x = ok ? alpha * acc[s][i] : NEG_INF;
      acc[s][i] = x;
      mx = __builtin_fmaxf(mx, x);
    }
  }
  mx = __builtin_fmaxf(mx, __shfl_xor(mx, 16));
  mx = __builtin_fmaxf(mx, __shfl_xor(mx, 32));
  if (fk == 0) red_max[wave][fr] = mx;
  __syncthreads();
  mx = red_max[0][fr];
#pragma unroll
  for (int w = 1; w < WAVES; ++w) mx = __builtin_fmaxf(mx, red_max[w][fr]);

  const float L2E = 1.4426950408889634f;
  float sum = 0.f;
#pragma unroll
  for (int s = 0; s < MAX_SUB; ++s) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float e = __builtin_amdgcn_exp2f((acc[s][i] - mx) * L2E);  // exp2(-inf) = 0 for padding
      acc[s][i] = e;
      sum += e;
    }
  }
  sum += __shfl_xor(sum, 16);
  sum += __shfl_xor(sum, 32);
  if (fk == 0) red_sum[wave][fr] = sum;
  __syncthreads();
  sum = red_sum[0][fr];
#pragma unroll
  for (int w = 1; w < WAVES; ++w) sum += red_sum[w][fr];
  const float inv = __builtin_amdgcn_rcpf(sum);

  const int m = m0 + fr;
  if (m < M) {
    float* __restrict__ crow = p.C + (size_t)m * N;
#pragma unroll
    for (int s = 0; s < MAX_SUB; ++s) {
      const int nb = col0 + s * 16 + 4 * fk;
      if (s < n_sub && nb < N) {
        f32x4 y = acc[s] * inv;
        *reinterpret_cast<f32x4*>(crow + nb) = y;
      }
    }
  }
}

template <int WAVES, int MAX_SUB, bool B_COL, class DT>
static hipError_t launch_softmax(const SoftmaxParams& p, hipStream_t stream) {
  void* args[] = {const_cast<SoftmaxParams*>(&p)};
  const dim3 grid((unsigned)((p.M + 15) / 16)), block(WAVES * 64);
  return hipLaunchKernel(reinterpret_cast<const void*>(&gemm_softmax_kernel<WAVES, MAX_SUB, B_COL, DT>), grid, block,
                         args, 0, stream);
}

template <int W, int S>
static SoftmaxVariant make_softmax_variant() {
  SoftmaxVariant v;
  // bm = 16 rows per workgroup, bn = longest row, bk = one 32-deep MFMA step
  v.cfg = tg_tile_config{0, TG_KERNEL_GEMM_SOFTMAX, 16, W * S * 16, 32, 2, W, 16, 16, 32, 1, W, 1, 0,
                         2 * W * 16 * 4, -1};
  v.fn[0][0] = &launch_softmax<W, S, false, F16>;
  v.fn[0][1] = &launch_softmax<W, S, true, F16>;
  v.fn[1][0] = &launch_softmax<W, S, false, BF16>;
  v.fn[1][1] = &launch_softmax<W, S, true, BF16>;
  return v;
}

// The compiled row-softmax configurations (ids follow the GEMM ones).
__host__ const SoftmaxVariant* softmax_variants(int* count) {
  static const SoftmaxVariant table[] = {
      make_softmax_variant<4, 16>(),  // rows up to 1024
      make_softmax_variant<8, 16>(),  // rows up to 2048
      make_softmax_variant<8, 8>(),   // rows up to 1024, two waves per SIMD
  };
  *count = (int)(sizeof(table) / sizeof(table[0]));
  return table;
}

}  // namespace tg
