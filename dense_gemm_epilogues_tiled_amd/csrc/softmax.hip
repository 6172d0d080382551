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
// 128-bit buffer loads (no LDS: no two waves share a B column); all loads of
// a K chunk are issued together and two chunks are in flight.  The row max and row sum are reduced first inside each
// lane, then across the 4 lanes sharing a row (lane xor 16, xor 32), then
// across waves through a few bytes of LDS.  exp uses v_exp_f32 (2^x) on
// (x - max) * log2(e).  Each lane writes 4 consecutive fp32 per tile.

#include "device.hpp"
#include "kernels.hpp"
#include "phases.hpp"

namespace tg {

TG_PHASE_BUFFER(softmax)

template <int WAVES, int MAX_SUB, int KC, bool B_COL, class DT>
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
  // B offsets stay 32-bit: the descriptor is rebased at this wave's first
  // column (column-major B) or at the K step's first row (row-major B).
  const __amdgpu_buffer_rsrc_t rBc = make_rsrc(gB + (size_t)col0 * K);

  f32x4 acc[MAX_SUB];
#pragma unroll
  for (int s = 0; s < MAX_SUB; ++s) acc[s] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Operand fragments of one 32-deep MFMA step kb: A rows m0..m0+15, B columns
  // col0 + 16 s .. +15; zero outside the matrix.
  auto load_a = [&](int kb) -> u32x4 {
    const int k = kb * 32 + fk * 8;
    return buffer_load16(rA, (a_row_ok && k < K) ? (fr * K + k) * 2 : kOOB);
  };
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

  // K in chunks of KC steps; all loads of a chunk are issued together and two
  // chunks are in flight, so the wave waits on memory latency about once.
  struct Chunk {
    u32x4 a[KC];
    u32x4 b[KC][MAX_SUB];
  };
  auto load_chunk = [&](int c, Chunk& ch) {
#pragma unroll
    for (int q = 0; q < KC; ++q) {
      ch.a[q] = load_a(c * KC + q);
#pragma unroll
      for (int s = 0; s < MAX_SUB; ++s) ch.b[q][s] = load_b(c * KC + q, s);
    }
  };
  auto mfma_chunk = [&](const Chunk& ch) {
#pragma unroll
    for (int q = 0; q < KC; ++q)
#pragma unroll
      for (int s = 0; s < MAX_SUB; ++s) acc[s] = mfma16x16x32(DT{}, ch.b[q][s], ch.a[q], acc[s]);
  };
  const int NC = (K + 32 * KC - 1) / (32 * KC);
  if constexpr (!B_COL) {
    // Row-major B gathers 16-bit values: one K step at a time keeps the
    // gathered registers small (this layout is not the fast path).
    const int KB = (K + 31) / 32;
    for (int kb = 0; kb < KB; ++kb) {
      const u32x4 a = load_a(kb);
#pragma unroll
      for (int s = 0; s < MAX_SUB; ++s) acc[s] = mfma16x16x32(DT{}, load_b(kb, s), a, acc[s]);
    }
  } else if (NC > 0) {
    Chunk c0, c1;
    load_chunk(0, c0);
    if (NC > 1) load_chunk(1, c1);
    int c = 0;
    for (; c + 2 < NC; c += 2) {
      mfma_chunk(c0);
      load_chunk(c + 2, c0);
      mfma_chunk(c1);
      if (c + 3 < NC) load_chunk(c + 3, c1);
    }
    if (c < NC) mfma_chunk(c0);
    if (c + 1 < NC) mfma_chunk(c1);
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

// ---------------------------------------------------------------------------
// Column-major B fast path.  Each wave owns NSUB 16-column MFMA tiles of the
// row (B rows col0 .. col0 + 16 NSUB - 1 of the N x K storage, contiguous in
// memory) and streams them, one 32-deep K step at a time, HBM/L2 -> its own
// LDS region with 1 KB direct copies (two steps in flight), together with its
// own copy of the 16 x 32 A step.  No LDS is shared between waves during the
// product, so no workgroup barrier is needed there.  LDS rows are 64 bytes
// (32 k), 16-byte chunks XOR-swizzled by (row / 4) % 4 so 16 consecutive rows
// at one chunk hit 16 distinct slots.  The row softmax takes one workgroup
// barrier (per-wave (max, sum) pairs, combined after it).  The result is
// staged back through the same region so each store instruction writes two
// contiguous 512-byte row segments, non-temporal.
// Keeping B in registers instead (every operand of the wave's product loaded
// at once, the row assembled in LDS and stored as whole rows) measured
// slower: 13.5 us against 10.8 us at 4096 x 1024 x 128, its loads of the
// whole of B into 256 workgroups' registers arriving at half the rate of
// these copies.
// ---------------------------------------------------------------------------
// FULL_LINES: 64-deep K steps instead of 32-deep ones, one step in flight
// per wave (the same LDS as two 32-deep steps): each copy then reads whole
// 128-byte lines (8 rows x 128 bytes) instead of half lines (16 rows x 64
// bytes, the other halves read by the next step's copies).
template <int WAVES, int NSUB, bool FULL_LINES, class DT>
__global__ __launch_bounds__(WAVES * 64, 1) void gemm_softmax_lds_kernel(SoftmaxParams p) {
  constexpr int BKS = FULL_LINES ? 64 : 32;           // K per step
  constexpr int SLOT = (1 + NSUB) * 16 * BKS * 2;     // one K step: A (16 rows) + NSUB x 16 B rows
  constexpr int NSLOT = FULL_LINES ? 1 : 2;           // steps in flight per wave
  constexpr int WREG = NSLOT * SLOT;
  constexpr int DMA = SLOT / 1024;                    // 1 KB copies per wave per step
  constexpr int OUT_STRIDE = NSUB * 64 + 16;  // staged output row (floats of 16 columns x NSUB), padded
  static_assert(16 * OUT_STRIDE <= WREG, "output staging fits the wave region");
  static_assert(WAVES * WREG + 2 * WAVES * 16 * 4 <= 160 * 1024, "LDS of one CU");
  __shared__ __attribute__((aligned(1024))) unsigned char smem[WAVES * WREG];
  __shared__ float red_max[WAVES][16];
  __shared__ float red_sum[WAVES][16];

  TG_PHASE_DECL;
  TG_PHASE(0);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int fr = lane & 15, fk = lane >> 4;
  const int M = p.M, N = p.N, K = p.K;
  const int n_sub = p.n_sub;
  const int m0 = blockIdx.x * 16;
  // column block of this wave, rotated by workgroup so that the workgroups
  // running at the same time read different parts of B (measured 1.7% faster
  // on 4096 x 1024 x 128 than every workgroup reading B in the same order)
  const int col0 = ((wave + (int)blockIdx.x) % WAVES) * n_sub * 16;

  const uint16_t* __restrict__ gA = static_cast<const uint16_t*>(p.A);
  const uint16_t* __restrict__ gB = static_cast<const uint16_t*>(p.B);
  const __amdgpu_buffer_rsrc_t rA = make_rsrc(gA + (size_t)m0 * K);
  const __amdgpu_buffer_rsrc_t rB = make_rsrc(gB + (size_t)col0 * K);
  unsigned char* wreg = smem + wave * WREG;
  const uint32_t wbase = lds_addr(wreg);

  // Copy plan of one step, in the kc_off<BKS> layout (rows of 2 BKS bytes):
  // each 1 KB copy covers RPC = 64 / CPR rows; lane i fills the 16-byte
  // slot i % CPR of row i / CPR of its copy, i.e. logical chunk
  // (i % CPR) ^ ((row / (16 / CPR)) % CPR); its global source is that row's
  // 8 k values.  Copies 0 .. CA-1 hold the 16 A rows, then CB per B tile.
  constexpr int CPR = BKS / 8;         // 16-byte chunks per row
  constexpr int RPC = 64 / CPR;        // rows per 1 KB copy
  constexpr int CA = 16 / RPC;         // copies per 16 rows
  const int crow = lane / CPR;
  auto cchunk = [&](int row) { return (lane % CPR) ^ ((row / (16 / CPR)) % CPR); };
  auto issue_step = [&](int kb, int slot) {
    const uint32_t sb = wbase + slot * SLOT;
#pragma unroll
    for (int c = 0; c < CA; ++c) {
      const int row = RPC * c + crow;  // of the 16 A rows
      const int k = kb * BKS + cchunk(row) * 8;
      dma16(rA, sb + 1024 * c, ((m0 + row) < M && k < K) ? (row * K + k) * 2 : kOOB);
    }
#pragma unroll
    for (int s = 0; s < NSUB; ++s)
#pragma unroll
      for (int c = 0; c < CA; ++c) {
        const int row = RPC * c + crow;  // of B tile s
        const int nl = 16 * s + row;
        const int k = kb * BKS + cchunk(row) * 8;
        const bool ok = k < K && s < n_sub && (col0 + nl) < N;
        dma16(rB, sb + 1024 * (CA * (1 + s) + c), ok ? (nl * K + k) * 2 : kOOB);
      }
  };

  f32x4 acc[NSUB];
#pragma unroll
  for (int s = 0; s < NSUB; ++s) acc[s] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int KB = (K + BKS - 1) / BKS;
  constexpr int TILE = 16 * BKS * 2;  // bytes of 16 rows of one step
  if constexpr (!FULL_LINES) {
    issue_step(0, 0);
    issue_step(1, 1);
    TG_PHASE(1);
    for (int kb = 0; kb < KB; ++kb) {
      const int slot = kb & 1;
      // step kb is complete once only step kb+1's copies are in flight
      asm volatile("s_waitcnt vmcnt(%0)" : : "n"(DMA) : "memory");
      if (kb == 0) TG_PHASE(2);
      const unsigned char* sb = wreg + slot * SLOT;
      const u32x4 a = lds_read16(sb, kc_off<32>(fr, fk));
      u32x4 b[NSUB];
#pragma unroll
      for (int s = 0; s < NSUB; ++s) b[s] = lds_read16(sb + TILE * (1 + s), kc_off<32>(fr, fk));
#pragma unroll
      for (int s = 0; s < NSUB; ++s) acc[s] = mfma16x16x32(DT{}, b[s], a, acc[s]);
      // the slot is refilled with step kb+2 once this wave's reads of it are done
      // (steps past the end of K copy nothing but zeros)
      asm volatile("s_waitcnt lgkmcnt(0)" : : : "memory");
      issue_step(kb + 2, slot);
    }
  } else {
    // one 64-deep step in flight: its fragments are read into registers, the
    // next step's copies are issued into the freed slot, then the MFMAs run
    // while those copies travel
    issue_step(0, 0);
    TG_PHASE(1);
    for (int kb = 0; kb < KB; ++kb) {
      asm volatile("s_waitcnt vmcnt(0)" : : : "memory");
      if (kb == 0) TG_PHASE(2);
      u32x4 a[2], b[2][NSUB];
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        a[kk] = lds_read16(wreg, kc_off<64>(fr, 4 * kk + fk));
#pragma unroll
        for (int s = 0; s < NSUB; ++s) b[kk][s] = lds_read16(wreg + TILE * (1 + s), kc_off<64>(fr, 4 * kk + fk));
      }
      asm volatile("s_waitcnt lgkmcnt(0)" : : : "memory");
      if (kb + 1 < KB) issue_step(kb + 1, 0);
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int s = 0; s < NSUB; ++s) acc[s] = mfma16x16x32(DT{}, b[kk][s], a[kk], acc[s]);
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" : : : "memory");
  TG_PHASE(3);

  // ---- row softmax, base 2, with one workgroup barrier: each wave reduces
  // its part of a row to (m_w, l_w) = (max of x, sum of 2^(x - m_w)),
  // x = alpha log2(e) acc; the pairs combine as m = max_w m_w,
  // l = sum_w l_w 2^(m_w - m), and the wave's exponentials are rescaled by
  // 2^(m_w - m) / l instead of recomputed (2% faster than a barrier for the
  // max and another for the sum) ----
  const float c1 = p.alpha * 1.4426950408889634f;
  const float NEG_INF = -__builtin_inff();
  float mw = NEG_INF;
#pragma unroll
  for (int s = 0; s < NSUB; ++s) {
    const int nb = col0 + s * 16 + 4 * fk;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bool ok = (s < n_sub) && (nb + i) < N;
      const float x = ok ? acc[s][i] * c1 : NEG_INF;
      acc[s][i] = x;
      mw = __builtin_fmaxf(mw, x);
    }
  }
  mw = __builtin_fmaxf(mw, __shfl_xor(mw, 16));
  mw = __builtin_fmaxf(mw, __shfl_xor(mw, 32));
  // a wave with no column of this row (short rows) contributes l_w = 0
  const float ms = mw == NEG_INF ? 0.f : mw;
  float lw = 0.f;
#pragma unroll
  for (int s = 0; s < NSUB; ++s)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float e = __builtin_amdgcn_exp2f(acc[s][i] - ms);  // 2^-inf = 0 for columns past the row
      acc[s][i] = e;
      lw += e;
    }
  lw += __shfl_xor(lw, 16);
  lw += __shfl_xor(lw, 32);
  if (fk == 0) {
    red_max[wave][fr] = mw;
    red_sum[wave][fr] = lw;
  }
  __syncthreads();
  TG_PHASE(4);
  float mx = red_max[0][fr];
#pragma unroll
  for (int w = 1; w < WAVES; ++w) mx = __builtin_fmaxf(mx, red_max[w][fr]);
  float sum = 0.f;
#pragma unroll
  for (int w = 0; w < WAVES; ++w) sum += red_sum[w][fr] * __builtin_amdgcn_exp2f(red_max[w][fr] - mx);
  TG_PHASE(5);
  const float inv = __builtin_amdgcn_exp2f(ms - mx) * __builtin_amdgcn_rcpf(sum);

  // ---- stage the wave's 16 x 16NSUB block through its LDS region, write rows contiguously ----
#pragma unroll
  for (int s = 0; s < NSUB; ++s)
    *reinterpret_cast<f32x4*>(wreg + fr * OUT_STRIDE + (16 * s + 4 * fk) * 4) = acc[s] * inv;
  // reads below follow this wave's own writes in LDS order
  const int cols = (N - col0) < 16 * n_sub ? (N - col0) : 16 * n_sub;  // valid columns of this wave
  constexpr int LPR = NSUB * 4;          // lanes per staged row (4 floats each)
  constexpr int RPI = 64 / LPR;          // rows per store instruction
#pragma unroll
  for (int q = 0; q < 16 / RPI; ++q) {
    const int r = q * RPI + lane / LPR;
    const int c4 = lane % LPR;
    const f32x4 v = *reinterpret_cast<const f32x4*>(wreg + r * OUT_STRIDE + c4 * 16);
    if (m0 + r < M && 4 * c4 < cols) store_nt(reinterpret_cast<f32x4*>(p.C + (size_t)(m0 + r) * N + col0 + 4 * c4), v);
  }
  TG_PHASE(6);
  TG_PHASE_DRAINED(7);
  TG_PHASE_WRITE(softmax);
}

template <int WAVES, int NSUB, bool FULL, class DT>
static hipError_t launch_softmax_lds(const SoftmaxParams& p, hipStream_t stream) {
  void* args[] = {const_cast<SoftmaxParams*>(&p)};
  const dim3 grid((unsigned)((p.M + 15) / 16)), block(WAVES * 64);
  return hipLaunchKernel(reinterpret_cast<const void*>(&gemm_softmax_lds_kernel<WAVES, NSUB, FULL, DT>), grid, block,
                         args, 0, stream);
}

template <int WAVES, int MAX_SUB, int KC, bool B_COL, class DT>
static hipError_t launch_softmax(const SoftmaxParams& p, hipStream_t stream) {
  void* args[] = {const_cast<SoftmaxParams*>(&p)};
  const dim3 grid((unsigned)((p.M + 15) / 16)), block(WAVES * 64);
  return hipLaunchKernel(reinterpret_cast<const void*>(&gemm_softmax_kernel<WAVES, MAX_SUB, KC, B_COL, DT>), grid,
                         block, args, 0, stream);
}

template <int W, int S, int KC>
static SoftmaxVariant make_softmax_variant() {
  SoftmaxVariant v;
  // bm = 16 rows per workgroup, bn = longest row, bk = one K chunk, stages = chunks in flight
  v.cfg = tg_tile_config{0, TG_KERNEL_GEMM_SOFTMAX, 16, W * S * 16, 32 * KC, 2, W, 16, 16, 32, 1, W, 1, 0,
                         2 * W * 16 * 4, -1};
  v.fn[0][0] = &launch_softmax<W, S, KC, false, F16>;
  v.fn[0][1] = &launch_softmax<W, S, KC, true, F16>;
  v.fn[1][0] = &launch_softmax<W, S, KC, false, BF16>;
  v.fn[1][1] = &launch_softmax<W, S, KC, true, BF16>;
  return v;
}

template <int W, int S, bool FULL = false>
static SoftmaxVariant make_softmax_lds_variant() {
  SoftmaxVariant v;
  // bk = K per step, stages = steps in flight per wave
  v.cfg = tg_tile_config{0, TG_KERNEL_GEMM_SOFTMAX, 16, W * S * 16, FULL ? 64 : 32, FULL ? 1 : 2, W, 16, 16, 32, 1, W,
                         1, 0, W * 2 * (1 + S) * 1024 + 2 * W * 16 * 4, 1};
  v.fn[0][0] = nullptr;  // column-major B only
  v.fn[0][1] = &launch_softmax_lds<W, S, FULL, F16>;
  v.fn[1][0] = nullptr;
  v.fn[1][1] = &launch_softmax_lds<W, S, FULL, BF16>;
  return v;
}

// The compiled row-softmax configurations (ids follow the GEMM ones).
__host__ const SoftmaxVariant* softmax_variants(int* count) {
  static const SoftmaxVariant table[] = {
      make_softmax_variant<8, 8, 2>(),   // rows up to 1024, two waves per SIMD
      make_softmax_variant<8, 16, 1>(),  // rows up to 2048
      make_softmax_variant<4, 16, 1>(),  // rows up to 1024, one wave per SIMD
      make_softmax_lds_variant<8, 8>(),  // rows up to 1024, column-major B through LDS
      make_softmax_lds_variant<4, 16>(), // rows up to 1024, column-major B through LDS
      make_softmax_lds_variant<8, 8, true>(),  // as <8, 8>, 64-deep steps: copies of whole 128-byte lines
  };
  *count = (int)(sizeof(table) / sizeof(table[0]));
  return table;
}

}  // namespace tg
