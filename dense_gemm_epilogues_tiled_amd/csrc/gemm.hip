// gemm.hip -- tiled MFMA GEMM with fused epilogues for gfx950 (MI355X).
//
//   C[m, n] = act(alpha * sum_k A[m, k] B[k, n] + bias[n])
//
// The method is the tiled tensor-core product of the TileLang tutorial
// ("TileLang: Criando Kernels de GPU de Alto Desempenho ...", noticiai.com.br,
// section "GEMM com Tensor Cores": operand tiles move global -> shared ->
// registers, the product runs on the matrix units, the global -> shared copy
// is pipelined; section "GEMM com epilogo fundido": bias / ReLU / GELU applied
// to the accumulator in the same kernel, no second pass over C).  Tile sizes,
// pipeline depth and L2 rasterisation are the knobs the spaxe.top page
// ("Designing High-Performance GPU Kernels with TileLang ...", schedule
// paragraph) and the edgex.exchange page (tiled-GEMM paragraph) name.  The
// realisation is gfx950's own:
//   * one workgroup per BM x BN output tile, WAVES_M x WAVES_N wave64s, each
//     wave owning a (BM/WAVES_M) x (BN/WAVES_N) block of 16x16 MFMA tiles;
//   * v_mfma_f32_16x16x32_{f16,bf16}, fp32 accumulators in registers;
//   * operands go HBM/L2 -> LDS directly (buffer_load_dwordx4 ... lds, no
//     VGPR staging), STAGES K steps in flight in an LDS ring, one workgroup
//     barrier per K step; out-of-range rows / columns / k are zero-filled by
//     the buffer range check (no branches in the loop);
//   * A (and a k-contiguous B) are read as 128-bit fragments from an
//     XOR-swizzled layout; a row-major (n-contiguous) B is kept in that
//     orientation and read with gfx950's transposing ds_read_b64_tr_b16;
//   * workgroup ids are regrouped so every XCD (private L2) works on a
//     contiguous band of tiles;
//   * the epilogue runs on the accumulator registers, rounds once to the
//     output type and writes C once.

#include "device.hpp"
#include "kernels.hpp"

namespace tg {

// Compile-time loop: f(integral_constant<int, 0>) ... f(integral_constant<int, N-1>).
template <int N, class F, int I = 0>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<N, F, I + 1>(static_cast<F&&>(f));
  }
}

// Workgroup id -> output tile.  The hardware deals consecutive workgroup ids
// to the 8 XCDs in turn; regroup so XCD x owns logical tiles
// [x*q + min(x, r), ...) (q = G / 8, r = G % 8), then walk the logical order
// in bands of group_m tile rows, column by column inside a band, so tiles that
// run at the same time on one XCD share A rows and B columns in its L2.
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

template <int BM, int BN, int BK, int WAVES_M, int WAVES_N, int STAGES, bool B_COL>
struct GemmShape {
  static constexpr int NW = WAVES_M * WAVES_N;
  static constexpr int NT = NW * 64;
  static constexpr int WTM = BM / WAVES_M, WTN = BN / WAVES_N;
  static constexpr int FM = WTM / 16, FN = WTN / 16;
  static constexpr int A_BYTES = BM * BK * 2, B_BYTES = BN * BK * 2;
  static constexpr int STAGE = A_BYTES + B_BYTES;
  static constexpr int LDS = STAGES * STAGE;
  // 1 KB direct-to-LDS wave instructions per stage, per wave
  static constexpr int DA = A_BYTES / 1024 / NW;
  static constexpr int DB = B_BYTES / 1024 / NW;
  static constexpr int DMA = DA + DB;
  static_assert(DA * 1024 * NW == A_BYTES && DB * 1024 * NW == B_BYTES, "tiles must split into 1 KB per wave");
  static_assert(BK == 32 || BK == 64, "K step of 32 or 64");
  static_assert(B_COL || BN >= 128, "n-contiguous B tiles need 128+ columns");
  static_assert(WTM % 16 == 0 && WTN % 16 == 0, "wave tile of whole MFMA tiles");
  static_assert(LDS <= 160 * 1024, "LDS of one gfx950 CU");
  static_assert(STAGES >= 2 && STAGES <= 4, "2 to 4 stages");
  static_assert((STAGES - 1) * DMA < 64, "vmcnt range");
};

template <int BM, int BN, int BK, int WAVES_M, int WAVES_N, int STAGES, bool B_COL, class DT>
__global__ __launch_bounds__(WAVES_M* WAVES_N * 64, 1) void gemm_tile_kernel(GemmParams p) {
  using S = GemmShape<BM, BN, BK, WAVES_M, WAVES_N, STAGES, B_COL>;
  constexpr int NW = S::NW, FM = S::FM, FN = S::FN, DA = S::DA, DB = S::DB;
  constexpr int KCH = BK / 8;

  __shared__ __attribute__((aligned(1024))) unsigned char smem[S::LDS];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;

  int tile_m, tile_n;
  map_tile(blockIdx.x, p.tiles_m, p.tiles_n, p.group_m, p.xcd_remap, tile_m, tile_n);
  const int m0 = tile_m * BM, n0 = tile_n * BN;
  const int M = p.M, N = p.N, K = p.K;
  const int KT = (K + BK - 1) / BK;

  const uint16_t* __restrict__ gA = static_cast<const uint16_t*>(p.A);
  const uint16_t* __restrict__ gB = static_cast<const uint16_t*>(p.B);

  // ---- direct-to-LDS copy plan: which global 16 bytes each lane fetches ----
  // Wave `wave` issues the 1 KB blocks q = wave + NW * j of each region; lane
  // i of block q fills LDS bytes [1024 q + 16 i, +16) of the region, so the
  // lane fetches the (row, chunk) the layout stores there.
  int a_off[DA], a_kc[DA];  // offset (kOOB for rows past M), k of the chunk
#pragma unroll
  for (int j = 0; j < DA; ++j) {
    const int pos = 1024 * (wave + NW * j) + 16 * lane;
    const int row = pos / (BK * 2);
    const int slot = (pos % (BK * 2)) / 16;
    const int chunk = slot ^ ((row / (16 / KCH)) % KCH);
    a_off[j] = (m0 + row) < M ? row * K * 2 + chunk * 16 : kOOB;
    a_kc[j] = chunk * 8;
  }
  int b_off[DB], b_kc[DB];
#pragma unroll
  for (int j = 0; j < DB; ++j) {
    const int pos = 1024 * (wave + NW * j) + 16 * lane;
    if constexpr (B_COL) {
      const int row = pos / (BK * 2);  // n
      const int slot = (pos % (BK * 2)) / 16;
      const int chunk = slot ^ ((row / (16 / KCH)) % KCH);
      b_off[j] = (n0 + row) < N ? row * K * 2 + chunk * 16 : kOOB;
      b_kc[j] = chunk * 8;
    } else {
      const int k = pos / (BN * 2);
      const int slot = (pos % (BN * 2)) / 16;
      const int chunk = (((slot >> 1) ^ nc_swz(k)) << 1) | (slot & 1);
      b_off[j] = (n0 + chunk * 8) < N ? k * N * 2 + chunk * 16 : kOOB;
      b_kc[j] = k;
    }
  }
  const uint32_t smem_base = lds_addr(smem);

  // Copy K step kt into LDS slot `slot`: copies [from, from + count) of the
  // step's DA + DB wave-wide 1 KB copies (A chunks first, then B).  Steps at
  // or past the end of K have every chunk out of range: they only write zeros.
  auto issue_part = [&](int kt, int slot, auto from_c, auto count_c) {
    constexpr int FROM = decltype(from_c)::value, COUNT = decltype(count_c)::value;
    const int k0 = kt * BK;
    const int k_left = K - k0;  // chunks at k >= k_left are zero-filled
    const uint32_t sbase = smem_base + slot * S::STAGE;
    if constexpr (FROM < DA) {
      const __amdgpu_buffer_rsrc_t rA = make_rsrc(gA + (size_t)m0 * K + k0);
#pragma unroll
      for (int j = FROM; j < DA && j < FROM + COUNT; ++j)
        dma16(rA, sbase + 1024 * (wave + NW * j), a_kc[j] < k_left ? a_off[j] : kOOB);
    }
    if constexpr (FROM + COUNT > DA) {
      const __amdgpu_buffer_rsrc_t rB = make_rsrc(B_COL ? gB + (size_t)n0 * K + k0 : gB + (size_t)k0 * N + n0);
#pragma unroll
      for (int j = (FROM > DA ? FROM - DA : 0); j < DB && j + DA < FROM + COUNT; ++j)
        dma16(rB, sbase + S::A_BYTES + 1024 * (wave + NW * j), b_kc[j] < k_left ? b_off[j] : kOOB);
    }
  };
  auto issue_stage = [&](int kt, int slot) {
    issue_part(kt, slot, std::integral_constant<int, 0>{}, std::integral_constant<int, S::DMA>{});
  };

  f32x4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // fragment coordinates of this lane
  const int fr = lane & 15, fk = lane >> 4;
  const int a_row0 = wm * S::WTM + fr;

  // ---- fragments: one 32-deep slice (kk) of a stage ----
  struct Frags {
    u32x4 a[FM];
    u32x4 b[FN];
  };
  auto load_frags = [&](int slot, int kk, Frags& f) {
    const unsigned char* sA = smem + slot * S::STAGE;
    const unsigned char* sB = sA + S::A_BYTES;
#pragma unroll
    for (int i = 0; i < FM; ++i) f.a[i] = lds_read16(sA, kc_off<BK>(a_row0 + 16 * i, 4 * kk + fk));
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      if constexpr (B_COL) {
        f.b[j] = lds_read16(sB, kc_off<BK>(wn * S::WTN + 16 * j + fr, 4 * kk + fk));
      } else {
        // lanes 4q..4q+3 of each 16-lane group read row k = 32kk + 8fk + 4h + q
        const int nb = wn * S::WTN + 16 * j;  // first column of the MFMA tile
        const int chunk = nb / 8 + ((fr & 3) >> 1);
        const int k_lo = 32 * kk + 8 * fk + (fr >> 2);
        const u32x2 lo = lds_read_tr8(sB, nc_off<BN>(k_lo, chunk) + 8 * (fr & 1));
        const u32x2 hi = lds_read_tr8(sB, nc_off<BN>(k_lo + 4, chunk) + 8 * (fr & 1));
        f.b[j] = u32x4{lo.x, lo.y, hi.x, hi.y};
      }
    }
  };
  auto mfma_frags = [&](const Frags& f) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) acc[i][j] = mfma16x16x32(DT{}, f.b[j], f.a[i], acc[i][j]);
  };
  // One interleaved phase: the FM*FN MFMAs on `use`, the LDS reads of slice
  // `kk` of slot `rslot` into `fill`, and copies [FROM, FROM+COUNT) of step
  // `dkt` into slot `dslot`, spread evenly over the MFMA stream.
  auto run_phase = [&](const Frags& use, Frags& fill, int rslot, int kk, int dkt, int dslot, auto from_c,
                       auto count_c) {
    constexpr int FROM = decltype(from_c)::value, COUNT = decltype(count_c)::value;
    constexpr int NMF = FM * FN;
    constexpr int NRD = FM + FN;  // fragment loads (a B load is 1 or 2 instructions)
    const unsigned char* sA = smem + rslot * S::STAGE;
    const unsigned char* sB = sA + S::A_BYTES;
    const int k0 = dkt * BK;
    const int k_left = K - k0;
    const uint32_t dbase = smem_base + dslot * S::STAGE;
    __amdgpu_buffer_rsrc_t rA, rB;
    if constexpr (COUNT > 0) {
      rA = make_rsrc(gA + (size_t)m0 * K + k0);
      rB = make_rsrc(B_COL ? gB + (size_t)n0 * K + k0 : gB + (size_t)k0 * N + n0);
    }
    static_for<NMF>([&](auto t_c) {
      constexpr int t = decltype(t_c)::value;
      constexpr int i = t / FN, j = t % FN;
      acc[i][j] = mfma16x16x32(DT{}, use.b[j], use.a[i], acc[i][j]);
      // fragment loads r with r * NMF / NRD == t, in the order the next phase
      // first needs them: a0, b0 .. b(FN-1), a1 .. a(FM-1)
      static_for<NRD>([&](auto r_c) {
        constexpr int r = decltype(r_c)::value;
        constexpr bool is_a = (r == 0) || (r > FN);
        constexpr int ia = r == 0 ? 0 : r - FN;
        if constexpr ((r * NMF) / NRD == t) {
          if constexpr (is_a) {
            fill.a[ia] = lds_read16(sA, kc_off<BK>(a_row0 + 16 * ia, 4 * kk + fk));
          } else {
            constexpr int jj = r - 1;
            if constexpr (B_COL) {
              fill.b[jj] = lds_read16(sB, kc_off<BK>(wn * S::WTN + 16 * jj + fr, 4 * kk + fk));
            } else {
              const int nb = wn * S::WTN + 16 * jj;
              const int chunk = nb / 8 + ((fr & 3) >> 1);
              const int k_lo = 32 * kk + 8 * fk + (fr >> 2);
              const u32x2 lo = lds_read_tr8(sB, nc_off<BN>(k_lo, chunk) + 8 * (fr & 1));
              const u32x2 hi = lds_read_tr8(sB, nc_off<BN>(k_lo + 4, chunk) + 8 * (fr & 1));
              fill.b[jj] = u32x4{lo.x, lo.y, hi.x, hi.y};
            }
          }
        }
      });
      // copies c with c * NMF / COUNT == t
      if constexpr (COUNT > 0) {
        static_for<COUNT>([&](auto c_c) {
          constexpr int c = decltype(c_c)::value;
          if constexpr ((c * NMF) / COUNT == t) {
            constexpr int q = FROM + c;
            if constexpr (q < DA)
              dma16(rA, dbase + 1024 * (wave + NW * q), a_kc[q] < k_left ? a_off[q] : kOOB);
            else
              dma16(rB, dbase + S::A_BYTES + 1024 * (wave + NW * (q - DA)),
                    b_kc[q - DA] < k_left ? b_off[q - DA] : kOOB);
          }
        });
      }
      __builtin_amdgcn_sched_barrier(0);
    });
  };

  // Publish a stage: wait until at most LATER stages of this wave's copies
  // (those issued after it) are still in flight, then the workgroup barrier.
  // Every wave waited for its own LDS reads before the barrier, so passing it
  // also means no wave reads any earlier stage's slot any more.
  auto publish_first = [&]() { wait_vm_barrier<(STAGES - 1) * S::DMA>(); };
  auto publish_next = [&]() { wait_vm_barrier<(STAGES - 2) * S::DMA>(); };

  // ---- main loop ----
  // STAGES steps are in flight before the loop; at every step boundary the
  // slot just finished is refilled with the step STAGES ahead, so STAGES-1
  // steps are always in flight while one is computed.  Fragments of the next
  // 32-deep slice are read from LDS while the MFMAs of the current slice run
  // (two register buffers F0 / F1 with fixed roles).
  constexpr int KK = BK / 32;
  Frags F0, F1;
  if constexpr (KK == 2) {
#pragma unroll
    for (int s = 0; s < STAGES - 1; ++s) issue_stage(s, s);
    issue_part(STAGES - 1, STAGES - 1, std::integral_constant<int, 0>{}, std::integral_constant<int, S::DMA / 2>{});
  } else {
#pragma unroll
    for (int s = 0; s < STAGES; ++s) issue_stage(s, s);
  }
  if (KT > 0) {
    if constexpr (KK == 2)
      wait_vm_barrier<(STAGES - 2) * S::DMA + S::DMA / 2>();
    else
      publish_first();
    load_frags(0, 0, F0);
    if constexpr (KK == 2) {
      // Explicitly interleaved K step (two 32-deep slices):
      //   phase A: MFMAs on slice 0 of step kt, interleaved with the LDS reads
      //            of slice 1 and the second half of the copies of step
      //            kt+STAGES-1 (into the slot step kt-1 used);
      //   publish step kt+1 (vmcnt wait + barrier);
      //   phase B: MFMAs on slice 1, interleaved with the LDS reads of slice 0
      //            of step kt+1 and the first half of the copies of step
      //            kt+STAGES (into step kt's slot, free after the barrier).
      // Between two MFMAs the wave issues at most one LDS read and one copy,
      // so neither the LDS queue nor the copy queue stalls the MFMA stream;
      // scheduling fences keep the compiler from regrouping them.
      for (int kt = 0; kt < KT - 1; ++kt) {
        const int slot = kt % STAGES;
        const int prev = (kt + STAGES - 1) % STAGES;
        run_phase(F0, F1, slot, 1, kt + STAGES - 1, prev, std::integral_constant<int, S::DMA / 2>{},
                  std::integral_constant<int, S::DMA - S::DMA / 2>{});
        publish_next();
        run_phase(F1, F0, (kt + 1) % STAGES, 0, kt + STAGES, slot, std::integral_constant<int, 0>{},
                  std::integral_constant<int, S::DMA / 2>{});
      }
      run_phase(F0, F1, (KT - 1) % STAGES, 1, 0, 0, std::integral_constant<int, 0>{},
                std::integral_constant<int, 0>{});
      mfma_frags(F1);
    } else {
      int kt = 0;
      for (; kt + 1 < KT; kt += 2) {
        publish_next();
        issue_stage(kt + STAGES, kt % STAGES);
        load_frags((kt + 1) % STAGES, 0, F1);
        mfma_frags(F0);
        if (kt + 2 < KT) {
          publish_next();
          issue_stage(kt + 1 + STAGES, (kt + 1) % STAGES);
          load_frags((kt + 2) % STAGES, 0, F0);
        }
        mfma_frags(F1);
      }
      if (kt < KT) mfma_frags(F0);
    }
  }
  // copies issued past the end of K may still be writing LDS
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  // ---- epilogue on the accumulators; lane holds C[m][n .. n+3] per (i, j) ----
  const uint16_t* __restrict__ gbias = static_cast<const uint16_t*>(p.bias);
  uint16_t* __restrict__ gC = static_cast<uint16_t*>(p.C);
  const float alpha = p.alpha;
  auto run_epilogue = [&](auto epi_tag) {
    constexpr int EPI = decltype(epi_tag)::value;
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int n = n0 + wn * S::WTN + 16 * j + 4 * fk;
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
        const int m = m0 + wm * S::WTM + 16 * i + fr;
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
// Compiled variants.
// ---------------------------------------------------------------------------
template <int BM, int BN, int BK, int WM, int WN, int ST, bool B_COL, class DT>
static hipError_t launch_gemm(const GemmParams& p, hipStream_t stream) {
  void* args[] = {const_cast<GemmParams*>(&p)};
  const dim3 grid((unsigned)(p.tiles_m * p.tiles_n)), block(WM * WN * 64);
  return hipLaunchKernel(reinterpret_cast<const void*>(&gemm_tile_kernel<BM, BN, BK, WM, WN, ST, B_COL, DT>), grid,
                         block, args, 0, stream);
}

template <int BM, int BN, int BK, int WM, int WN, int ST>
static GemmVariant make_gemm_variant(int group_m) {
  GemmVariant v;
  v.cfg = tg_tile_config{0, TG_KERNEL_GEMM, BM, BN, BK, ST, WM * WN, 16, 16, 32, WM, WN, group_m, 1,
                         GemmShape<BM, BN, BK, WM, WN, ST, false>::LDS, -1};
  v.fn[0][0] = &launch_gemm<BM, BN, BK, WM, WN, ST, false, F16>;
  v.fn[0][1] = &launch_gemm<BM, BN, BK, WM, WN, ST, true, F16>;
  v.fn[1][0] = &launch_gemm<BM, BN, BK, WM, WN, ST, false, BF16>;
  v.fn[1][1] = &launch_gemm<BM, BN, BK, WM, WN, ST, true, BF16>;
  return v;
}

// The compiled GEMM tile configurations, in configuration-id order.  (A host
// function holding the table keeps host-only launcher addresses out of device
// compilation.)
__host__ const GemmVariant* gemm_variants(int* count) {
  static const GemmVariant table[] = {
      make_gemm_variant<128, 128, 64, 2, 2, 4>(4),  // 0
      make_gemm_variant<256, 128, 64, 2, 2, 3>(4),  // 1
      make_gemm_variant<256, 256, 32, 2, 4, 4>(8),  // 2
      make_gemm_variant<128, 128, 32, 2, 2, 4>(4),  // 3
      make_gemm_variant<256, 256, 64, 2, 4, 2>(8),  // 4
      make_gemm_variant<128, 128, 64, 2, 4, 4>(4),  // 5: two waves per SIMD
      make_gemm_variant<128, 128, 64, 4, 2, 4>(4),  // 6
  };
  *count = (int)(sizeof(table) / sizeof(table[0]));
  return table;
}

}  // namespace tg
