// gemm.hip -- tiled MFMA GEMM with fused epilogues for gfx950 (MI355X).
//
//   C[m, n] = act(alpha * sum_k A[m, k] B[k, n] + bias[n])
//
// The method is the tiled tensor-core product of the TileLang tutorial
// ("TileLang: Criando Kernels de GPU de Alto Desempenho ...", noticiai.com.br,
// section "GEMM com Tensor Cores": operand tiles move global -> shared ->
// registers, the product runs on the matrix units; section "GEMM com epilogo
// fundido": bias / ReLU / GELU applied to the accumulator in the same kernel).
// The tile sizes, pipeline and L2 rasterisation are knobs the spaxe.top page
// ("Designing High-Performance GPU Kernels with TileLang ...", schedule
// paragraph) and the edgex.exchange page (GEMM paragraph: tile sizes,
// pipeline stages, thread counts, L2 swizzling) name.  The realisation here is
// gfx950's own:
//   * one workgroup per BM x BN output tile, WAVES_M x WAVES_N wave64s, each
//     wave owning a (BM/WAVES_M) x (BN/WAVES_N) block of 16x16 MFMA tiles;
//   * v_mfma_f32_16x16x32_{f16,bf16} with fp32 accumulators in registers;
//   * 128-bit buffer loads (zero-filled outside the matrix) staged through
//     registers into a double-buffered, XOR-swizzled LDS ring: the next K step
//     is fetched from HBM/L2 while the current one feeds the MFMAs;
//   * row-major B (N contiguous) is transposed in registers on its way into
//     LDS so both operands are read as k-contiguous 128-bit fragments;
//   * workgroup ids are regrouped so every XCD (own L2) works on a contiguous
//     block of tiles, rasterised in bands of GROUP_M tile rows;
//   * the epilogue runs on the accumulator registers, rounds once and writes
//     C exactly once.

#include "device.hpp"
#include "kernels.hpp"

namespace tg {

// Workgroup id -> output tile.  Hardware hands consecutive workgroup ids to
// the 8 XCDs in turn; regroup so XCD x owns logical tiles
// [x*q + min(x, r), ...) (q = G / 8, r = G % 8), then walk the logical order
// in bands of group_m tile rows, column by column inside a band, so the tiles
// an XCD runs at the same time share A rows and B columns in its L2.
__device__ __forceinline__ void map_tile(int bid, int tiles_m, int tiles_n, int group_m, int xcd_remap, int& tm,
                                         int& tn) {
  const int G = tiles_m * tiles_n;
  int w = bid;
  if (xcd_remap) {
    const int q = G >> 3, r = G & 7, x = bid & 7, j = bid >> 3;
    w = x * q + (x < r ? x : r) + j;
  }
  const int per_group = group_m * tiles_n;
  const int g = w / per_group;
  const int first = g * group_m;
  const int gm = (tiles_m - first) < group_m ? (tiles_m - first) : group_m;
  const int in = w - g * per_group;
  tm = first + in % gm;
  tn = in / gm;
}

template <int BM, int BN, int BK, int WAVES_M, int WAVES_N, bool B_COL, class DT>
__global__ __launch_bounds__(WAVES_M* WAVES_N * 64, 1) void gemm_tile_kernel(GemmParams p) {
  static_assert(BK == 64, "LDS layout is written for 64-element K rows");
  constexpr int NT = WAVES_M * WAVES_N * 64;
  constexpr int WTM = BM / WAVES_M, WTN = BN / WAVES_N;
  constexpr int FM = WTM / 16, FN = WTN / 16;
  constexpr int KCH = BK / 8;  // 16-byte chunks per K row
  constexpr int A_BYTES = BM * BK * 2, B_BYTES = BN * BK * 2;
  constexpr int STAGE = A_BYTES + B_BYTES;
  constexpr int A_LOADS = BM * KCH / NT;  // 16-byte A chunks per thread per K step
  static_assert(A_LOADS * NT == BM * KCH, "A tile must split evenly over the threads");
  // B, k-contiguous (column-major) source: same scheme as A.
  constexpr int BC_LOADS = BN * KCH / NT;
  // B, n-contiguous (row-major) source: units of 4 k-rows x 8 n-columns.
  constexpr int BR_UNITS = (BK / 4) * (BN / 8) / NT;
  static_assert(B_COL ? (BC_LOADS * NT == BN * KCH) : (BR_UNITS * NT == (BK / 4) * (BN / 8)),
                "B tile must split evenly over the threads");

  __shared__ __attribute__((aligned(16))) unsigned char smem[2 * STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;

  int tile_m, tile_n;
  map_tile(blockIdx.x, p.tiles_m, p.tiles_n, p.group_m, p.xcd_remap, tile_m, tile_n);
  const int m0 = tile_m * BM, n0 = tile_n * BN;
  const int M = p.M, N = p.N, K = p.K;
  const int KT = (K + BK - 1) / BK;

  const uint16_t* __restrict__ gA = static_cast<const uint16_t*>(p.A);
  const uint16_t* __restrict__ gB = static_cast<const uint16_t*>(p.B);

  // ---- per-thread load assignments (fixed over the K loop) ----
  int a_off[A_LOADS], a_lds[A_LOADS];
  bool a_row_ok[A_LOADS];
  int a_k8[A_LOADS];
#pragma unroll
  for (int i = 0; i < A_LOADS; ++i) {
    const int q = tid + i * NT, row = q / KCH, c = q % KCH;
    a_off[i] = row * K * 2 + c * 16;
    a_lds[i] = lds_off64(row, c);
    a_row_ok[i] = (m0 + row) < M;
    a_k8[i] = c * 8;
  }
  constexpr int B_REGS = B_COL ? BC_LOADS : BR_UNITS * 4;
  int b_off[B_REGS];
  bool b_ok[B_REGS];
  int b_k[B_REGS];  // k offset inside the K step of the chunk / row
  int b_lds[B_COL ? BC_LOADS : 1];
  if constexpr (B_COL) {
#pragma unroll
    for (int i = 0; i < BC_LOADS; ++i) {
      const int q = tid + i * NT, row = q / KCH, c = q % KCH;
      b_off[i] = row * K * 2 + c * 16;
      b_lds[i] = lds_off64(row, c);
      b_ok[i] = (n0 + row) < N;
      b_k[i] = c * 8;
    }
  } else {
#pragma unroll
    for (int u = 0; u < BR_UNITS; ++u) {
      const int q = tid + u * NT;
      const int kg = q % (BK / 4), nc = q / (BK / 4);
      // this thread's rows 4kg..4kg+3, columns 8nc..8nc+7 of the B step
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        b_off[u * 4 + r] = (4 * kg + r) * N * 2 + nc * 16;
        b_ok[u * 4 + r] = (n0 + 8 * nc) < N;
        b_k[u * 4 + r] = 4 * kg + r;
      }
    }
    b_lds[0] = 0;
  }

  u32x4 ra[A_LOADS];
  u32x4 rb[B_REGS];

  auto load_step = [&](int kt) {
    const int k0 = kt * BK;
    const __amdgpu_buffer_rsrc_t rA = make_rsrc(gA + (size_t)m0 * K + k0);
#pragma unroll
    for (int i = 0; i < A_LOADS; ++i) {
      const bool ok = a_row_ok[i] && (k0 + a_k8[i]) < K;
      ra[i] = buffer_load16(rA, ok ? a_off[i] : kOOB);
    }
    if constexpr (B_COL) {
      const __amdgpu_buffer_rsrc_t rB = make_rsrc(gB + (size_t)n0 * K + k0);
#pragma unroll
      for (int i = 0; i < BC_LOADS; ++i) {
        const bool ok = b_ok[i] && (k0 + b_k[i]) < K;
        rb[i] = buffer_load16(rB, ok ? b_off[i] : kOOB);
      }
    } else {
      const __amdgpu_buffer_rsrc_t rB = make_rsrc(gB + (size_t)k0 * N + n0);
#pragma unroll
      for (int i = 0; i < B_REGS; ++i) {
        const bool ok = b_ok[i] && (k0 + b_k[i]) < K;
        rb[i] = buffer_load16(rB, ok ? b_off[i] : kOOB);
      }
    }
  };

  auto store_step = [&](int stage) {
    unsigned char* sA = smem + stage * STAGE;
    unsigned char* sB = sA + A_BYTES;
#pragma unroll
    for (int i = 0; i < A_LOADS; ++i) lds_write16(sA, a_lds[i], ra[i]);
    if constexpr (B_COL) {
#pragma unroll
      for (int i = 0; i < BC_LOADS; ++i) lds_write16(sB, b_lds[i], rb[i]);
    } else {
#pragma unroll
      for (int u = 0; u < BR_UNITS; ++u) {
        const int q = tid + u * NT;
        const int kg = q % (BK / 4), nc = q / (BK / 4);
        const u32x4& r0 = rb[u * 4 + 0];
        const u32x4& r1 = rb[u * 4 + 1];
        const u32x4& r2 = rb[u * 4 + 2];
        const u32x4& r3 = rb[u * 4 + 3];
        // column 2d   of the unit: low halves of word d of rows 0..3
        // column 2d+1 of the unit: high halves of word d of rows 0..3
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          u32x2 ev, od;
          ev.x = (r0[d] & 0xffffu) | (r1[d] << 16);
          ev.y = (r2[d] & 0xffffu) | (r3[d] << 16);
          od.x = (r0[d] >> 16) | (r1[d] & 0xffff0000u);
          od.y = (r2[d] >> 16) | (r3[d] & 0xffff0000u);
          const int row_e = 8 * nc + 2 * d;
          lds_write8(sB, lds_off64(row_e, kg >> 1) + ((kg & 1) << 3), ev);
          lds_write8(sB, lds_off64(row_e + 1, kg >> 1) + ((kg & 1) << 3), od);
        }
      }
    }
  };

  f32x4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // fragment rows of this lane inside the A / B tiles
  const int fr = lane & 15, fk = lane >> 4;
  const int a_row0 = wm * WTM + fr;
  const int b_row0 = wn * WTN + fr;

  auto compute_step = [&](int stage) {
    const unsigned char* sA = smem + stage * STAGE;
    const unsigned char* sB = sA + A_BYTES;
#pragma unroll
    for (int kk = 0; kk < BK / 32; ++kk) {
      u32x4 af[FM], bf[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i) af[i] = lds_read16(sA, lds_off64(a_row0 + 16 * i, 4 * kk + fk));
#pragma unroll
      for (int j = 0; j < FN; ++j) bf[j] = lds_read16(sB, lds_off64(b_row0 + 16 * j, 4 * kk + fk));
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = mfma16x16x32(DT{}, bf[j], af[i], acc[i][j]);
    }
  };

  if (KT > 0) {
    load_step(0);
    store_step(0);
    __syncthreads();
    for (int kt = 0; kt < KT; ++kt) {
      const bool more = (kt + 1) < KT;
      if (more) load_step(kt + 1);
      compute_step(kt & 1);
      if (more) store_step((kt + 1) & 1);
      __syncthreads();
    }
  }

  // ---- epilogue on the accumulators; lane holds C[m][n .. n+3] per (i, j) ----
  const uint16_t* __restrict__ gbias = static_cast<const uint16_t*>(p.bias);
  uint16_t* __restrict__ gC = static_cast<uint16_t*>(p.C);
  const float alpha = p.alpha;
  auto run_epilogue = [&](auto epi_tag) {
    constexpr int EPI = decltype(epi_tag)::value;
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int n = n0 + wn * WTN + 16 * j + 4 * fk;
      if (n >= N) continue;
      float b0 = 0.f, b1 = 0.f, b2 = 0.f, b3 = 0.f;
      if constexpr (EPI != EPI_NONE) {
        const u32x2 bb = *reinterpret_cast<const u32x2*>(gbias + n);
        b0 = lo_to_f32(DT{}, bb.x);
        b1 = hi_to_f32(DT{}, bb.x);
        b2 = lo_to_f32(DT{}, bb.y);
        b3 = hi_to_f32(DT{}, bb.y);
      }
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const int m = m0 + wm * WTM + 16 * i + fr;
        if (m >= M) continue;
        const f32x4 a = acc[i][j];
        float x0 = __builtin_fmaf(alpha, a[0], b0);
        float x1 = __builtin_fmaf(alpha, a[1], b1);
        float x2 = __builtin_fmaf(alpha, a[2], b2);
        float x3 = __builtin_fmaf(alpha, a[3], b3);
        if constexpr (EPI == EPI_RELU) {
          x0 = __builtin_fmaxf(x0, 0.f);
          x1 = __builtin_fmaxf(x1, 0.f);
          x2 = __builtin_fmaxf(x2, 0.f);
          x3 = __builtin_fmaxf(x3, 0.f);
        } else if constexpr (EPI == EPI_GELU) {
          x0 = gelu_erf(x0);
          x1 = gelu_erf(x1);
          x2 = gelu_erf(x2);
          x3 = gelu_erf(x3);
        }
        u32x2 out;
        out.x = pack2(DT{}, x0, x1);
        out.y = pack2(DT{}, x2, x3);
        *reinterpret_cast<u32x2*>(gC + (size_t)m * N + n) = out;
      }
    }
  };
  switch (p.epilogue) {
    case EPI_RELU: run_epilogue(std::integral_constant<int, EPI_RELU>{}); break;
    case EPI_GELU: run_epilogue(std::integral_constant<int, EPI_GELU>{}); break;
    case EPI_BIAS: run_epilogue(std::integral_constant<int, EPI_BIAS>{}); break;
    default: run_epilogue(std::integral_constant<int, EPI_NONE>{}); break;
  }
}

// ---------------------------------------------------------------------------
// Launchers for the compiled variants.
// ---------------------------------------------------------------------------
template <int BM, int BN, int BK, int WAVES_M, int WAVES_N, bool B_COL, class DT>
static hipError_t launch_gemm(const GemmParams& p, hipStream_t stream) {
  void* args[] = {const_cast<GemmParams*>(&p)};
  const dim3 grid((unsigned)(p.tiles_m * p.tiles_n)), block(WAVES_M * WAVES_N * 64);
  return hipLaunchKernel(reinterpret_cast<const void*>(&gemm_tile_kernel<BM, BN, BK, WAVES_M, WAVES_N, B_COL, DT>),
                         grid, block, args, 0, stream);
}

#define TG_GEMM_LAUNCHERS(BM, BN, BK, WM, WN)                                                  \
  {{                                                                                            \
    {&launch_gemm<BM, BN, BK, WM, WN, false, F16>, &launch_gemm<BM, BN, BK, WM, WN, true, F16>}, \
    {&launch_gemm<BM, BN, BK, WM, WN, false, BF16>, &launch_gemm<BM, BN, BK, WM, WN, true, BF16>}   \
  }}

// Order and shapes must match kVariants in api.cpp.  (A host function holding
// the table keeps the host-only launcher addresses out of device compilation.)
__host__ const GemmLauncherSet* gemm_launchers(int* count) {
  static const GemmLauncherSet table[] = {
      TG_GEMM_LAUNCHERS(128, 128, 64, 2, 2),
      TG_GEMM_LAUNCHERS(256, 128, 64, 2, 2),
      TG_GEMM_LAUNCHERS(256, 256, 64, 2, 4),
      TG_GEMM_LAUNCHERS(128, 64, 64, 2, 1),
  };
  *count = (int)(sizeof(table) / sizeof(table[0]));
  return table;
}

}  // namespace tg
