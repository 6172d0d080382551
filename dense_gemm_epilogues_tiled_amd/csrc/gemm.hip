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

#include "gemm_common.hpp"
#include "phases.hpp"

namespace tg {

TG_PHASE_BUFFER(gemm)

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
  static_assert(STAGES >= 2 && STAGES <= 5, "2 to 5 stages");
  static_assert(BK == 64 || STAGES >= 3, "one-slice steps reuse a slot one step late");
  static_assert((STAGES - 1) * DMA < 64, "vmcnt range");
  static_assert(BM * BN * 2 <= LDS, "the C image fits in the ring");
};

template <int BM, int BN, int BK, int WAVES_M, int WAVES_N, int STAGES, bool FRONT, bool B_COL, class DT>
__global__ __launch_bounds__(WAVES_M* WAVES_N * 64, 1) void gemm_tile_kernel(GemmParams p) {
  using S = GemmShape<BM, BN, BK, WAVES_M, WAVES_N, STAGES, B_COL>;
  constexpr int NW = S::NW, FM = S::FM, FN = S::FN;

  __shared__ __attribute__((aligned(1024))) unsigned char smem[S::LDS];

  TG_PHASE_DECL;
  TG_PHASE(0);
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

  CopyPlan<BM, BN, BK, NW, B_COL> plan;
  plan.init(wave, lane, m0, n0, M, N, K);
  const uint32_t smem_base = lds_addr(smem);

  // Copy K step kt into LDS slot `slot`: copies [from, from + count) of the
  // step's DA + DB wave-wide 1 KB copies (A chunks first, then B).  Steps at
  // or past the end of K have every chunk out of range: they only write zeros.
  auto issue_part = [&](int kt, int slot, auto from_c, auto count_c) {
    constexpr int FROM = decltype(from_c)::value, COUNT = decltype(count_c)::value;
    const uint32_t sbase = smem_base + slot * S::STAGE;
    static_for<COUNT>([&](auto c_c) {
      plan.template copy<FROM + decltype(c_c)::value>(wave, gA, gB, m0, n0, N, K, kt * BK, sbase);
    });
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
  FragAddr<BN, BK, S::WTM, S::WTN, FN, B_COL> fa;
  fa.init(wm, wn, fr, fk);

  // ---- fragments: one 32-deep slice (kk) of a stage ----
  struct Frags {
    u32x4 a[FM];
    u32x4 b[FN];
  };
  auto load_frags = [&](int slot, int kk, Frags& f) {
    const unsigned char* sA = smem + opaque_sgpr(slot * S::STAGE);
    const unsigned char* sB = sA + S::A_BYTES;
#pragma unroll
    for (int i = 0; i < FM; ++i) f.a[i] = fa.read_a(sA, i, kk);
#pragma unroll
    for (int j = 0; j < FN; ++j) f.b[j] = fa.read_b(sB, j, kk);
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
    const unsigned char* sA = smem + opaque_sgpr(rslot * S::STAGE);
    const unsigned char* sB = sA + S::A_BYTES;
    const uint32_t dbase = smem_base + dslot * S::STAGE;
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
          if constexpr (is_a)
            fill.a[ia] = fa.read_a(sA, ia, kk);
          else
            fill.b[r - 1] = fa.read_b(sB, r - 1, kk);
        }
      });
      // copies c with c * NMF / COUNT == t
      if constexpr (COUNT > 0) {
        static_for<COUNT>([&](auto c_c) {
          constexpr int c = decltype(c_c)::value;
          if constexpr ((c * NMF) / COUNT == t)
            plan.template copy<FROM + c>(wave, gA, gB, m0, n0, N, K, dkt * BK, dbase);
        });
      }
      __builtin_amdgcn_sched_barrier(0);
    });
  };

  // Publish a stage (two-slice steps): wait until at most STAGES-2 later
  // steps of this wave's copies are still in flight, then the workgroup
  // barrier.  Every wave waited for its own LDS reads before the barrier, so
  // passing it also means no wave reads any earlier stage's slot any more.
  auto publish_next = [&]() { wait_vm_barrier<(STAGES - 2) * S::DMA>(); };

  // ---- main loop ----
  // Two-slice steps (BK = 64): STAGES steps are in flight before the loop; at
  // every step boundary the slot just finished is refilled with the step
  // STAGES ahead, so STAGES-1 steps are always in flight while one is
  // computed.  Fragments of the next 32-deep slice are read from LDS while
  // the MFMAs of the current slice run (two register buffers F0 / F1 with
  // fixed roles).  One-slice steps (BK = 32) are described at their loop.
  constexpr int KK = BK / 32;
  Frags F0, F1;
  // FRONT: every copy of step kt+STAGES is issued in phase B of step kt,
  // as soon as its slot is free, so it has STAGES-1 whole steps to land (with
  // two stages this is what keeps the barrier that publishes step kt+1 from
  // waiting on copies issued just before it).  Otherwise the copies of a
  // step are split between phase B of one step and phase A of the next.
  constexpr int COPIES_A = FRONT ? 0 : S::DMA - S::DMA / 2;  // phase A: tail of step kt+STAGES-1
  constexpr int COPIES_B = FRONT ? S::DMA : S::DMA / 2;      // phase B: head of step kt+STAGES
  if constexpr (KK == 2) {
#pragma unroll
    for (int s = 0; s < STAGES - 1; ++s) issue_stage(s, s);
    issue_part(STAGES - 1, STAGES - 1, std::integral_constant<int, 0>{}, std::integral_constant<int, COPIES_B>{});
  } else {
#pragma unroll
    for (int s = 0; s < STAGES - 1; ++s) issue_stage(s, s);
  }
  TG_PHASE(1);
  if (KT > 0) {
    if constexpr (KK == 2)
      wait_vm_barrier<(STAGES - 2) * S::DMA + COPIES_B>();
    else
      wait_vm_barrier<(STAGES - 2) * S::DMA>();
    TG_PHASE(2);
    load_frags(0, 0, F0);
    if constexpr (KK == 2) {
      // Explicitly interleaved K step (two 32-deep slices):
      //   phase A: MFMAs on slice 0 of step kt, interleaved with the LDS reads
      //            of slice 1 and the tail of the copies of step kt+STAGES-1
      //            (into the slot step kt-1 used);
      //   publish step kt+1 (vmcnt wait + barrier);
      //   phase B: MFMAs on slice 1, interleaved with the LDS reads of slice 0
      //            of step kt+1 and the head of the copies of step kt+STAGES
      //            (into step kt's slot, free after the barrier).
      // Between two MFMAs the wave issues at most one LDS read and one copy,
      // so neither the LDS queue nor the copy queue stalls the MFMA stream;
      // scheduling fences keep the compiler from regrouping them.
      for (int kt = 0; kt < KT - 1; ++kt) {
        const int slot = kt % STAGES;
        const int prev = (kt + STAGES - 1) % STAGES;
        run_phase(F0, F1, slot, 1, kt + STAGES - 1, prev, std::integral_constant<int, COPIES_B>{},
                  std::integral_constant<int, COPIES_A>{});
        publish_next();
        run_phase(F1, F0, (kt + 1) % STAGES, 0, kt + STAGES, slot, std::integral_constant<int, 0>{},
                  std::integral_constant<int, COPIES_B>{});
      }
      run_phase(F0, F1, (KT - 1) % STAGES, 1, 0, 0, std::integral_constant<int, 0>{},
                std::integral_constant<int, 0>{});
      mfma_frags(F1);
    } else {
      // One 32-deep slice per K step, one barrier per step.  Step kt runs
      // its MFMAs (i-major) on the fragments in F and refills F in place
      // with step kt+1: A fragment i as soon as the MFMAs of row block i are
      // done, the B fragments in the last FN MFMAs, so one register buffer
      // serves both steps.  The copies of step kt+STAGES-1 go into the slot
      // of step kt-1, whose reads (issued during step kt-2) were consumed by
      // step kt-1's MFMAs: the barrier never waits for LDS reads, only for
      // the copies of step kt+1, and every copy has STAGES-2 steps to land.
      using All = std::integral_constant<int, S::DMA>;
      auto phase = [&](Frags& f, int rslot, int dkt, int dslot, auto count_c) {
        constexpr int COUNT = decltype(count_c)::value;
        constexpr int NMF = FM * FN;
        const unsigned char* sA = smem + opaque_sgpr(rslot * S::STAGE);
        const unsigned char* sB = sA + S::A_BYTES;
        const uint32_t dbase = smem_base + dslot * S::STAGE;
        static_for<NMF>([&](auto t_c) {
          constexpr int t = decltype(t_c)::value;
          constexpr int i = t / FN, j = t % FN;
          acc[i][j] = mfma16x16x32(DT{}, f.b[j], f.a[i], acc[i][j]);
          if constexpr (i == FM - 1) f.b[j] = fa.read_b(sB, j, 0);
          if constexpr (j == FN - 1) f.a[i] = fa.read_a(sA, i, 0);
          if constexpr (COUNT > 0) {
            static_for<COUNT>([&](auto c_c) {
              constexpr int c = decltype(c_c)::value;
              if constexpr ((c * NMF) / COUNT == t)
                plan.template copy<c>(wave, gA, gB, m0, n0, N, K, dkt * BK, dbase);
            });
          }
          __builtin_amdgcn_sched_barrier(0);
        });
      };
      constexpr int IN_FLIGHT = (STAGES - 3) * S::DMA;  // steps kt+2 .. kt+STAGES-2
      for (int kt = 0; kt + 1 < KT; ++kt) {
        wait_vm_barrier_only<IN_FLIGHT>();
        phase(F0, (kt + 1) % STAGES, kt + STAGES - 1, (kt + STAGES - 1) % STAGES, All{});
      }
      mfma_frags(F0);
    }
  }
  // ---- epilogue: finish the accumulators in registers, then write C once
  // through an LDS image of the tile.  Copies issued past the end of K may
  // still be writing LDS; once every wave is past the barrier the ring is
  // free for the image.
  TG_PHASE(3);
  with_epilogue(p.epilogue, [&](auto epi_c) {
    u32x2 out[FM][FN];
    finish_tile<decltype(epi_c)::value, DT>(p, acc, out, n0, wn * S::WTN, fk);
    TG_PHASE(4);
    wait_vm_barrier<0>();
    TG_PHASE(5);
    store_tile_staged<DT, BM, BN, S::NT, FM, FN>(p, out, smem, m0, n0, wm * S::WTM, wn * S::WTN, fr, fk, tid);
  });
  TG_PHASE(6);
  TG_PHASE_DRAINED(7);
  TG_PHASE_WRITE(gemm);
}

// ---------------------------------------------------------------------------
// K-split workgroup: 2 groups of WM x WN waves.  Wave s of group 0 and wave s
// of group 1 own the same (BM/WM) x (BN/WN) output block; in every 64-deep K
// step group g multiplies the 32-deep slice g, so a wave reads half a step's
// fragments from LDS: a third less LDS read traffic than 2*WM*WN waves tiling
// the output, for the same MFMA work per wave.  The loop is the one-slice
// loop of gemm_tile_kernel (in-place fragment refill, copies into the slot of
// step kt-1, barriers that wait only for copies).  At the end the two partial
// accumulators are summed through LDS, each group finishing half of the row
// blocks of its output block.
// ---------------------------------------------------------------------------
// MFMA order of one step over FM x FN tiles: 0 = j-major; 1 = 2x2 blocks of
// (i, j), block rows first.  Returns i (WHICH = 0) or j (WHICH = 1) of step t.
template <int ORDER, int FM, int FN>
constexpr int mfma_coord(int t, int which) {
  if (ORDER == 0) return which == 0 ? t % FM : t / FM;
  const int b = t / 4, w = t % 4, ib = b / (FN / 2), jb = b % (FN / 2);
  return which == 0 ? 2 * ib + w % 2 : 2 * jb + w / 2;
}
// Last step of the order that uses row block i (WHICH = 0) or column block j.
template <int ORDER, int FM, int FN>
constexpr int last_use(int x, int which) {
  int last = -1;
  for (int t = 0; t < FM * FN; ++t)
    if (mfma_coord<ORDER, FM, FN>(t, which) == x) last = t;
  return last;
}

template <int BM, int BN, int WM, int WN, int STAGES, int ORDER, bool B_COL, class DT>
__global__ __launch_bounds__(2 * WM * WN * 64, 1) void gemm_ksplit_kernel(GemmParams p) {
  constexpr int BK = 64;
  constexpr int NS = WM * WN, NW = 2 * NS, NT = NW * 64;
  constexpr int WTM = BM / WM, WTN = BN / WN, FM = WTM / 16, FN = WTN / 16, H = FM / 2;
  constexpr int A_BYTES = BM * BK * 2, STAGE = (BM + BN) * BK * 2, LDS = STAGES * STAGE;
  using Plan = CopyPlan<BM, BN, BK, NW, B_COL>;
  constexpr int DMA = Plan::DMA;
  constexpr int XBYTES = NS * 2 * H * FN * 1024;  // partial accumulators handed between the groups
  static_assert(STAGES >= 3 && LDS <= 160 * 1024 && (STAGES - 1) * DMA < 64, "ring");
  static_assert(FM % 2 == 0 && WTM % 16 == 0 && WTN % 16 == 0, "whole MFMA tiles, even row blocks");
  static_assert(ORDER == 0 || FN % 2 == 0, "2x2 blocks of MFMA tiles");
  static_assert(XBYTES + BM * BN * 2 <= LDS, "partials and the C image fit in the ring");

  __shared__ __attribute__((aligned(1024))) unsigned char smem[LDS];

  TG_PHASE_DECL;
  TG_PHASE(0);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = wave / NS, sw = wave % NS;
  const int wm = sw / WN, wn = sw % WN;

  int tile_m, tile_n;
  map_tile(blockIdx.x, p.tiles_m, p.tiles_n, p.group_m, p.xcd_remap, tile_m, tile_n);
  const int m0 = tile_m * BM, n0 = tile_n * BN;
  const int M = p.M, N = p.N, K = p.K;
  const int KT = (K + BK - 1) / BK;
  const uint16_t* __restrict__ gA = static_cast<const uint16_t*>(p.A);
  const uint16_t* __restrict__ gB = static_cast<const uint16_t*>(p.B);

  Plan plan;
  plan.init(wave, lane, m0, n0, M, N, K);
  const uint32_t smem_base = lds_addr(smem);
  const int fr = lane & 15, fk = lane >> 4;
  FragAddr<BN, BK, WTM, WTN, FN, B_COL> fa;
  fa.init(wm, wn, fr, fk);
  // this wave's slice: offsets of slice g (a select, not an indexed register array)
  const int a_lane = g ? fa.a[1] : fa.a[0];
  auto read_a = [&](const unsigned char* sA, int i) { return lds_read16(sA + a_lane, i * 16 * BK * 2); };
  auto read_b = [&](const unsigned char* sB, int j) -> u32x4 {
    if constexpr (B_COL) {
      return lds_read16(sB + (g ? fa.b[1] : fa.b[0]), j * 16 * BK * 2);
    } else {
      const unsigned char* q = sB + fa.b[j] + g * (32 * BN * 2);
      const u32x2 lo = lds_read_tr8(q, 0);
      const u32x2 hi = lds_read_tr8(q, 4 * BN * 2);
      return u32x4{lo.x, lo.y, hi.x, hi.y};
    }
  };

  auto issue_stage = [&](int kt, int slot) {
    const uint32_t sbase = smem_base + slot * STAGE;
    static_for<DMA>([&](auto c_c) {
      plan.template copy<decltype(c_c)::value>(wave, gA, gB, m0, n0, N, K, kt * BK, sbase);
    });
  };

  f32x4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // bias of this lane's output columns, fetched now so its latency hides
  // under the main loop (a bias is passed exactly when the epilogue uses one)
  u32x2 bias_raw[FN];
#pragma unroll
  for (int j = 0; j < FN; ++j) {
    const int n = n0 + wn * WTN + 16 * j + 4 * fk;
    bias_raw[j] = (p.bias != nullptr && n < N)
                      ? *reinterpret_cast<const u32x2*>(static_cast<const uint16_t*>(p.bias) + n)
                      : u32x2{0u, 0u};
  }

  struct Frags {
    u32x4 a[FM];
    u32x4 b[FN];
  } F;
  // MFMAs on F (j-major), refilling F in place with the slice of step kt+1
  // from slot rslot, and the copies of step dkt into slot dslot.
  auto phase = [&](int rslot, int dkt, int dslot, auto count_c) {
    constexpr int COUNT = decltype(count_c)::value;
    constexpr int NMF = FM * FN;
    const unsigned char* sA = smem + opaque_sgpr(rslot * STAGE);
    const unsigned char* sB = sA + A_BYTES;
    const uint32_t dbase = smem_base + dslot * STAGE;
    static_for<NMF>([&](auto t_c) {
      constexpr int t = decltype(t_c)::value;
      constexpr int i = mfma_coord<ORDER, FM, FN>(t, 0), j = mfma_coord<ORDER, FM, FN>(t, 1);
      acc[i][j] = mfma16x16x32(DT{}, F.b[j], F.a[i], acc[i][j]);
      // a fragment is refilled right after its last MFMA of the step: in the
      // j-major order the B fragments (two transposing reads each) go early,
      // one per column block, and the A fragments in the last FM MFMAs
      if constexpr (t == last_use<ORDER, FM, FN>(j, 1)) F.b[j] = read_b(sB, j);
      if constexpr (t == last_use<ORDER, FM, FN>(i, 0)) F.a[i] = read_a(sA, i);
      if constexpr (COUNT > 0) {
        static_for<COUNT>([&](auto c_c) {
          constexpr int c = decltype(c_c)::value;
          if constexpr ((c * NMF) / COUNT == t) plan.template copy<c>(wave, gA, gB, m0, n0, N, K, dkt * BK, dbase);
        });
      }
      __builtin_amdgcn_sched_barrier(0);
    });
  };

#pragma unroll
  for (int st = 0; st < STAGES - 1; ++st) issue_stage(st, st);
  TG_PHASE(1);
  if (KT > 0) {
    wait_vm_barrier<(STAGES - 2) * DMA>();
    TG_PHASE(2);
    {
      const unsigned char* sA = smem;
#pragma unroll
      for (int i = 0; i < FM; ++i) F.a[i] = read_a(sA, i);
#pragma unroll
      for (int j = 0; j < FN; ++j) F.b[j] = read_b(sA + A_BYTES, j);
    }
    for (int kt = 0; kt + 1 < KT; ++kt) {
      wait_vm_barrier_only<(STAGES - 3) * DMA>();
      phase((kt + 1) % STAGES, kt + STAGES - 1, (kt + STAGES - 1) % STAGES, std::integral_constant<int, DMA>{});
    }
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) acc[i][j] = mfma16x16x32(DT{}, F.b[j], F.a[i], acc[i][j]);
  }
  // every copy landed and every wave is done with the ring
  wait_vm_barrier<0>();
  TG_PHASE(3);

  // ---- sum the two groups' partials, then the epilogue: group g finishes
  // row blocks [H g, H g + H) of its output block.  The tile goes out in H
  // rounds, one row block per wave each: finish it, put it in the C image,
  // barrier, store those rows; the stores of one round drain while the next
  // round's activations run. ----
  f32x4* xbuf = reinterpret_cast<f32x4*>(smem);
  auto xidx = [&](int part, int i, int j) { return ((sw * 2 + part) * H * FN + i * FN + j) * 64 + lane; };
  unsigned char* cimg = smem + XBYTES;
  uint16_t* __restrict__ gC = static_cast<uint16_t*>(p.C);
  with_epilogue(p.epilogue, [&](auto epi_c) {
    constexpr int EPI = decltype(epi_c)::value;
    auto finish = [&](auto g_c) {
      constexpr int G = decltype(g_c)::value;
#pragma unroll
      for (int i = 0; i < H; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) xbuf[xidx(1 - G, i, j)] = acc[H * (1 - G) + i][j];
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
#pragma unroll
      for (int i = 0; i < H; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[H * G + i][j] += xbuf[xidx(G, i, j)];
      TG_PHASE(4);
      static_for<H>([&](auto ih_c) {
        constexpr int IH = decltype(ih_c)::value;
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const u32x2 bb = bias_raw[j];
          const f32x4 b{lo_to_f32(DT{}, bb.x), hi_to_f32(DT{}, bb.x), lo_to_f32(DT{}, bb.y), hi_to_f32(DT{}, bb.y)};
          const int r = wm * WTM + 16 * (H * G + IH) + fr;
          const int c = wn * WTN + 16 * j + 4 * fk;
          *reinterpret_cast<u32x2*>(cimg + c_image_off<BN>(r, c / 4)) =
              finish4<EPI, DT>(p.alpha, acc[H * G + IH][j], b);
        }
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
        // rows of round IH: row block (r / 16) % H == IH of every wave's block
        constexpr int PIECES_PER_ROW = BN / 8, ROWS = BM / H;
        static_assert(ROWS * PIECES_PER_ROW % NT == 0, "whole rounds of 16-byte pieces");
#pragma unroll
        for (int q = tid; q < ROWS * PIECES_PER_ROW; q += NT) {
          const int rr = q / PIECES_PER_ROW, v = q % PIECES_PER_ROW;
          const int r = (rr / 16) * (16 * H) + 16 * IH + rr % 16;
          const int m = m0 + r, n = n0 + 8 * v;
          const u32x4 val = *reinterpret_cast<const u32x4*>(cimg + c_image_off<BN>(r, 2 * v));
          if (m < M && n < N) store_nt(reinterpret_cast<u32x4*>(gC + (size_t)m * N + n), val);
        }
        if constexpr (IH == 0) TG_PHASE(5);
      });
    };
    if (g == 0)
      finish(std::integral_constant<int, 0>{});
    else
      finish(std::integral_constant<int, 1>{});
  });
  TG_PHASE(6);
  TG_PHASE_DRAINED(7);
  TG_PHASE_WRITE(gemm);
}

// ---------------------------------------------------------------------------
// Compiled variants.
// ---------------------------------------------------------------------------
template <int BM, int BN, int BK, int WM, int WN, int ST, bool FRONT, bool B_COL, class DT>
static hipError_t launch_gemm(const GemmParams& p, hipStream_t stream) {
  void* args[] = {const_cast<GemmParams*>(&p)};
  const dim3 grid((unsigned)(p.tiles_m * p.tiles_n)), block(WM * WN * 64);
  return hipLaunchKernel(reinterpret_cast<const void*>(&gemm_tile_kernel<BM, BN, BK, WM, WN, ST, FRONT, B_COL, DT>), grid,
                         block, args, 0, stream);
}

template <int BM, int BN, int WM, int WN, int ST, int OR, bool B_COL, class DT>
static hipError_t launch_ksplit(const GemmParams& p, hipStream_t stream) {
  void* args[] = {const_cast<GemmParams*>(&p)};
  const dim3 grid((unsigned)(p.tiles_m * p.tiles_n)), block(2 * WM * WN * 64);
  return hipLaunchKernel(reinterpret_cast<const void*>(&gemm_ksplit_kernel<BM, BN, WM, WN, ST, OR, B_COL, DT>), grid,
                         block, args, 0, stream);
}

// waves = 2 * wave_m * wave_n: two groups splitting each K step
template <int BM, int BN, int WM, int WN, int ST, int OR = 0>
static GemmVariant make_ksplit_variant(int group_m) {
  GemmVariant v;
  v.cfg = tg_tile_config{0, TG_KERNEL_GEMM, BM, BN, 64, ST, 2 * WM * WN, 16, 16, 32, WM, WN, group_m, 1,
                         ST * (BM + BN) * 64 * 2, -1};
  v.fn[0][0] = &launch_ksplit<BM, BN, WM, WN, ST, OR, false, F16>;
  v.fn[0][1] = &launch_ksplit<BM, BN, WM, WN, ST, OR, true, F16>;
  v.fn[1][0] = &launch_ksplit<BM, BN, WM, WN, ST, OR, false, BF16>;
  v.fn[1][1] = &launch_ksplit<BM, BN, WM, WN, ST, OR, true, BF16>;
  return v;
}

template <int BM, int BN, int BK, int WM, int WN, int ST, bool FRONT = ST == 2>
static GemmVariant make_gemm_variant(int group_m) {
  GemmVariant v;
  v.cfg = tg_tile_config{0, TG_KERNEL_GEMM, BM, BN, BK, ST, WM * WN, 16, 16, 32, WM, WN, group_m, 1,
                         GemmShape<BM, BN, BK, WM, WN, ST, false>::LDS, -1};
  v.fn[0][0] = &launch_gemm<BM, BN, BK, WM, WN, ST, FRONT, false, F16>;
  v.fn[0][1] = &launch_gemm<BM, BN, BK, WM, WN, ST, FRONT, true, F16>;
  v.fn[1][0] = &launch_gemm<BM, BN, BK, WM, WN, ST, FRONT, false, BF16>;
  v.fn[1][1] = &launch_gemm<BM, BN, BK, WM, WN, ST, FRONT, true, BF16>;
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
      make_gemm_variant<128, 128, 64, 2, 4, 4, true>(4),  // 7: as 5, copies issued a whole step earlier
      make_gemm_variant<256, 256, 32, 2, 4, 5>(8),        // 8: 4 slices of prefetch in the whole 160 KB
      make_gemm_variant<256, 256, 64, 2, 2, 2>(8),        // 9: one wave per SIMD, 128x128 per wave
      make_ksplit_variant<128, 128, 2, 2, 4>(8),          // 10: two groups of 4 waves split each K step
      make_ksplit_variant<128, 128, 2, 2, 4, 1>(8),       // 11: as 10, MFMAs in 2x2 blocks
  };
  *count = (int)(sizeof(table) / sizeof(table[0]));
  return table;
}

}  // namespace tg
