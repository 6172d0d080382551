// attention.hip -- FlashAttention forward for gfx950 (fp16 / bf16, head dim 64
// or 128, causal or not):
//
//     O = softmax(scale * Q K^T [key j <= query i when causal]) V   per (batch, head)
//
// The tutorial's capstone ("TileLang: Criando Kernels ..." (noticiai.com.br),
// section "Softmax por linha e FlashAttention"; the edgex.exchange page's
// FlashAttention paragraph; spaxe.top, FlashAttention paragraph): query, key
// and value tiles are processed without writing the score matrix to memory;
// an online softmax keeps a running maximum and a running sum per query and
// rescales the partial output whenever the maximum grows; both products run
// on the matrix units.
//
// gfx950 design
// -------------
// A workgroup of 4 waves owns 128 consecutive queries of one (batch, head)
// (256 for the non-causal kernel at head dim 64): 32 (64) per wave, held in
// registers as MFMA operands for the whole kernel.  Key
// and value blocks of 64 rows stream through a two-stage LDS ring, copied
// HBM/L2 -> LDS with the direct 16-byte-per-lane copies (no VGPR staging);
// keys past the sequence end are zero-filled by the buffer range check.
//
// Each wave computes the transposed score tile S^T = K Q^T (64 keys x 32
// queries) with v_mfma_f32_16x16x32: lane l then holds, for query l % 16,
// four consecutive keys 4 (l / 16) .. +3 of each 16-key tile.  Those are
// exactly the values the second product needs from the lane, in that order:
// O^T += V^T P^T takes P^T as its B operand with the MFMA's 32-deep k axis
// mapped to keys {4g .. 4g+3} of one 16-key tile and {4g .. 4g+3} of the next
// (g = l / 16), and V^T as its A operand read with ds_read_b64_tr_b16 using
// the same key order (an MFMA sums over k in any order, as long as both
// operands agree).  So P never leaves the registers and is never shuffled;
// per-query statistics need only the 4 lanes that share a query (lane-swap
// instructions across rows of 16 and halves of 32 lanes).
// The online softmax works in base 2 (exp2 on scale * log2 e * score), keeps
// per-lane partial sums (the 4 lanes of a query are rescaled by the same
// factors) and reduces them once at the end.

#include "device.hpp"
#include "kernels.hpp"
#include "phases.hpp"

namespace tg {

TG_PHASE_BUFFER(attention)

namespace {

constexpr int kAttnWaves = 4;
// Queries per wave: 32, or 64 for the non-causal kernel at head dim 64,
// where the accumulators are half as large -- every wave reads the whole
// K / V block from LDS, so more queries per wave means fewer LDS bytes per
// FLOP.  (The causal kernel's masking state does not fit beside 64.)
template <int D, bool CAUSAL>
constexpr int attn_qw() { return D == 64 && !CAUSAL ? 64 : 32; }
template <int D, bool CAUSAL>
constexpr int attn_bm() { return kAttnWaves * attn_qw<D, CAUSAL>(); }  // queries per workgroup
constexpr int kAttnBN = 64;                      // keys per block

template <int D>
struct AttnShape {
  static_assert(D == 64 || D == 128, "head dim 64 or 128");
  static constexpr int KBYTES = kAttnBN * D * 2;           // one K block in LDS
  static constexpr int VBYTES = kAttnBN * D * 2;           // one V block in LDS
  static constexpr int STAGE = KBYTES + VBYTES;
  static constexpr int LDS = 2 * STAGE;                    // two-stage ring
  static constexpr int KCOPIES = KBYTES / 1024 / kAttnWaves;  // 1 KB copies per wave per block
  static constexpr int VCOPIES = VBYTES / 1024 / kAttnWaves;
  static_assert(KCOPIES * 1024 * kAttnWaves == KBYTES && VCOPIES * 1024 * kAttnWaves == VBYTES, "1 KB pieces");
};

// V tiles are n-contiguous (a key row of D values) with 32-byte pairs of
// 16-byte chunks XOR-swizzled per row.  The transposing reads of one wave
// touch 4 consecutive keys per 16-lane group and the groups start 4 keys
// apart; the 32 lanes served together (8 rows) must hit distinct banks.
//   D = 128: a row spans all 64 banks, so the 8 rows need 8 distinct pairs:
//            the swizzle takes key bits 0-1 and bit 2;
//   D = 64:  a row spans half of them (odd rows the other half), so rows of
//            one parity need distinct pairs: key bits 1-2.
template <int D>
__device__ __forceinline__ int v_swz(int key) {
  if constexpr (D == 128) return (key & 3) | (((key >> 2) & 1) << 2);
  return (key >> 1) & 3;
}
template <int D>
__device__ __forceinline__ int v_off(int key, int chunk) {
  return key * (D * 2) + 16 * ((((chunk >> 1) ^ v_swz<D>(key)) << 1) | (chunk & 1));
}

// x combined with the value of the same register in lanes l ^ 16 and l ^ 32
// (the four lanes that hold one query's scores), via the gfx950 lane-swap
// instructions (VALU, no LDS round trip).  The words pass by value: a bit
// cast of a vector element in place would read element 0.
__device__ __forceinline__ float w2f(uint32_t w) { return __builtin_bit_cast(float, w); }
__device__ __forceinline__ uint32_t f2w(float f) { return __builtin_bit_cast(uint32_t, f); }
template <bool MAX>
__device__ __forceinline__ float reduce_4lanes(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(f2w(x), f2w(x), false, false);  // rows of 16 lanes, pairwise
  const uint32_t a0 = a[0], a1 = a[1];
  x = MAX ? __builtin_fmaxf(w2f(a0), w2f(a1)) : w2f(a0) + w2f(a1);
  const auto b = __builtin_amdgcn_permlane32_swap(f2w(x), f2w(x), false, false);  // halves of 32 lanes
  const uint32_t b0 = b[0], b1 = b[1];
  return MAX ? __builtin_fmaxf(w2f(b0), w2f(b1)) : w2f(b0) + w2f(b1);
}

// Per-lane source offsets (bytes from the block's first key row) of this
// wave's copies, chosen so that the LDS image of a block is the swizzled
// layout the fragment reads expect: K rows k-contiguous (kc_off), V rows
// n-contiguous (v_off).
template <int D>
struct AttnCopies {
  int k_off[AttnShape<D>::KCOPIES], k_row[AttnShape<D>::KCOPIES];
  int v_src[AttnShape<D>::VCOPIES], v_row[AttnShape<D>::VCOPIES];

  __device__ __forceinline__ void init(int wave, int lane) {
    constexpr int KCH = D / 8;
#pragma unroll
    for (int j = 0; j < AttnShape<D>::KCOPIES; ++j) {
      const int pos = 1024 * (wave + kAttnWaves * j) + 16 * lane;
      const int row = pos / (D * 2);
      const int slot = (pos % (D * 2)) / 16;
      const int chunk = slot ^ ((row / (16 / KCH)) % KCH);
      k_off[j] = row * D * 2 + chunk * 16;
      k_row[j] = row;
    }
#pragma unroll
    for (int j = 0; j < AttnShape<D>::VCOPIES; ++j) {
      const int pos = 1024 * (wave + kAttnWaves * j) + 16 * lane;
      const int row = pos / (D * 2);
      const int slot = (pos % (D * 2)) / 16;
      const int chunk = (((slot >> 1) ^ v_swz<D>(row)) << 1) | (slot & 1);
      v_src[j] = row * D * 2 + chunk * 16;
      v_row[j] = row;
    }
  }

  // Copy key / value block starting at key kb into the stage at LDS byte
  // address `stage`; rows at or past n read zeros.
  __device__ __forceinline__ void issue(int wave, __amdgpu_buffer_rsrc_t kr, __amdgpu_buffer_rsrc_t vr, int kb, int n,
                                        uint32_t stage) const {
    const int rows_left = n - kb;
    const int base = kb * D * 2;
#pragma unroll
    for (int j = 0; j < AttnShape<D>::KCOPIES; ++j)
      dma16(kr, stage + 1024 * (wave + kAttnWaves * j), k_row[j] < rows_left ? base + k_off[j] : kOOB);
#pragma unroll
    for (int j = 0; j < AttnShape<D>::VCOPIES; ++j)
      dma16(vr, stage + AttnShape<D>::KBYTES + 1024 * (wave + kAttnWaves * j),
            v_row[j] < rows_left ? base + v_src[j] : kOOB);
  }
};

// Buffer resource over one head's N x D block (range = its bytes).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t head_rsrc(const void* base, int64_t head, int n, int d) {
  const unsigned char* p = static_cast<const unsigned char*>(base) + head * (int64_t)n * d * 2;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<unsigned char*>(p), (short)0, n * d * 2, 0x00020000);
}

}  // namespace

template <int D, class DT, bool CAUSAL>
__global__ __launch_bounds__(256, 2) void attention_fwd_kernel(AttnParams p) {
  using S = AttnShape<D>;
  constexpr int KT = kAttnBN / 16;  // 16-key tiles per block
  constexpr int kAttnQW = attn_qw<D, CAUSAL>(), kAttnBM = attn_bm<D, CAUSAL>();
  constexpr int QT = kAttnQW / 16;  // 16-query tiles per wave
  constexpr int DK = D / 32;        // 32-deep slices of the QK^T product
  constexpr int NDT = D / 16;       // 16-row tiles of O^T
  __shared__ __attribute__((aligned(1024))) unsigned char smem[S::LDS];

  TG_PHASE_DECL;  // per pass (slots 4 pass .. +3): start, first block landed, last block done, O stored
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: the copies' LDS base goes to m0
  const int fr = lane & 15, fk = lane >> 4;

  // workgroup -> (head, query block): each XCD takes a contiguous range of
  // heads (workgroups are dealt to the 8 XCDs round robin), so a head's K / V
  // stay in one L2; within a head the query blocks run last-to-first.
  // The causal kernel pairs query block t with block q_blocks - 1 - t (the
  // longest with the shortest), so every workgroup does the same work.
  const int groups = gridDim.x;
  int lin = blockIdx.x;
  if ((groups & 7) == 0) lin = (lin & 7) * (groups >> 3) + (lin >> 3);
  const int64_t head = lin / p.units;
  const int t = lin % p.units;
  const int qb_first = p.q_blocks - 1 - t;
  const int npass = CAUSAL && t != qb_first ? 2 : 1;
  const int n = p.N;

  const __amdgpu_buffer_rsrc_t qr = head_rsrc(p.Q, head, n, D);
  const __amdgpu_buffer_rsrc_t kr = head_rsrc(p.K, head, n, D);
  const __amdgpu_buffer_rsrc_t vr = head_rsrc(p.V, head, n, D);

  AttnCopies<D> cp;
  cp.init(wave, lane);
  const uint32_t lds0 = lds_addr(smem);

  for (int pass = 0; pass < npass; ++pass) {
  if (pass == 0) TG_PHASE(0); else TG_PHASE(4);
  const int qb = pass == 0 ? qb_first : t;
  const int q0 = qb * kAttnBM;
  const int q0w = q0 + wave * kAttnQW;
  const int kend = CAUSAL ? (q0 + kAttnBM < n ? q0 + kAttnBM : n) : n;
  const int nblk = (kend + kAttnBN - 1) / kAttnBN;
  cp.issue(wave, kr, vr, 0, n, lds0);

  // Q^T fragments (B operand of S^T = K Q^T): query q0w + 16 qt + fr, dims
  // 32 kk + 8 fk .. +7; queries past n read zeros.
  u32x4 qf[QT][DK];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt)
#pragma unroll
    for (int kk = 0; kk < DK; ++kk)
      qf[qt][kk] = buffer_load16(qr, (q0w + 16 * qt + fr) * D * 2 + (32 * kk + 8 * fk) * 2);

  f32x4 o[NDT][QT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) o[dt][qt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m[QT], l[QT];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    m[qt] = -__builtin_inff();
    l[qt] = 0.f;
  }
  // scores are scaled by |scale| log2 e > 0 (the host passes 2^-100 for a
  // zero scale: exp2 of anything that small is exactly 1, as for 0); a
  // negative scale flips the sign of Q instead (exact)
  const float sl2 = p.scale_log2;
  if (p.negate_q) {
#pragma unroll
    for (int qt = 0; qt < QT; ++qt)
#pragma unroll
      for (int kk = 0; kk < DK; ++kk) qf[qt][kk] ^= u32x4{0x80008000u, 0x80008000u, 0x80008000u, 0x80008000u};
  }

  wait_vm_barrier<0>();
  if (pass == 0) TG_PHASE(1); else TG_PHASE(5);
  // The Q loads are complete (the wait above), but the compiler does not see
  // through that asm and would wait for them again at their first use inside
  // the loop -- with vmcnt, which also counts the in-flight copies of the
  // next K / V block, stalling every block until its successor has landed.
  // Redefining the fragments here makes the compiler's wait happen once.
#pragma unroll
  for (int qt = 0; qt < QT; ++qt)
#pragma unroll
    for (int kk = 0; kk < DK; ++kk) asm volatile("" : "+v"(qf[qt][kk]));
  // One key / value block: issue the next block's copies, then the two
  // products and the online softmax on this one.  Blocks run as MASKED may
  // hold keys past the sequence end or (causal) after some of the
  // workgroup's queries; the other instantiation carries no masking code.
  auto run_block = [&]<bool MASKED>(int j) {
    if (j + 1 < nblk) cp.issue(wave, kr, vr, (j + 1) * kAttnBN, n, lds0 + ((j + 1) & 1) * S::STAGE);
    const int kb = j * kAttnBN;
    // a causal block entirely after this wave's last query adds nothing
    if (!CAUSAL || kb <= q0w + kAttnQW - 1) {
      const unsigned char* sK = smem + (j & 1) * S::STAGE;
      const unsigned char* sV = sK + S::KBYTES;

      // S^T = K Q^T: tile [kt][qt], lane holds query 16 qt + fr, keys 16 kt + 4 fk + r
      f32x4 st[KT][QT];
#pragma unroll
      for (int kt = 0; kt < KT; ++kt)
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) st[kt][qt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < DK; ++kk)
#pragma unroll
        for (int kt = 0; kt < KT; ++kt) {
          const u32x4 a = lds_read16(sK, kc_off<D>(16 * kt + fr, 4 * kk + fk));
#pragma unroll
          for (int qt = 0; qt < QT; ++qt) st[kt][qt] = mfma16x16x32(DT{}, a, qf[qt][kk], st[kt][qt]);
        }

      // masked keys (past the end; causal: after the query) get a raw score
      // of -inf; only blocks that hold such keys pay for it
      if (MASKED && __builtin_expect(kb + kAttnBN > n || (CAUSAL && kb + kAttnBN - 1 > q0w), 0)) {
#pragma unroll
        for (int qt = 0; qt < QT; ++qt)
#pragma unroll
          for (int kt = 0; kt < KT; ++kt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int key = kb + 16 * kt + 4 * fk + r;
              const bool ok = key < n && (!CAUSAL || key <= q0w + 16 * qt + fr);
              st[kt][qt][r] = ok ? st[kt][qt][r] : -__builtin_inff();
            }
      }

      // block max of the scaled scores per query (sl2 > 0: the max commutes
      // with the scaling; all keys masked: -inf)
      float bm[QT];
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) {
        float x = -__builtin_inff();
#pragma unroll
        for (int kt = 0; kt < KT; ++kt)
#pragma unroll
          for (int r = 0; r < 4; ++r) x = __builtin_fmaxf(x, st[kt][qt][r]);
        bm[qt] = reduce_4lanes<true>(x) * sl2;
      }

      // Lazy rescaling: the reference m of a query moves only when the block
      // max exceeds it by more than kLazy (log2 units), so p = exp2(s - m)
      // stays <= 2^kLazy; the output and the sum share the same stale m, so
      // their quotient is unchanged.  The wave rescales only when one of its
      // queries needs it.
      constexpr float kLazy = 8.f;
      bool need = false;
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) need |= bm[qt] > m[qt] + kLazy;
      if (__builtin_amdgcn_ballot_w64(need) != 0) {
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) {
          const bool up = bm[qt] > m[qt] + kLazy;
          const float corr = up ? __builtin_amdgcn_exp2f(m[qt] - bm[qt]) : 1.f;  // m = -inf: corr = 0
          m[qt] = up ? bm[qt] : m[qt];
          l[qt] *= corr;
#pragma unroll
          for (int dt = 0; dt < NDT; ++dt) o[dt][qt] *= corr;
        }
      }

      // P^T operands and the partial sums: p = exp2(s sl2 - m); a masked key
      // (s = -inf) gives 0
      u32x4 pb[QT][KT / 2];
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) {
        const float mu = m[qt] == -__builtin_inff() ? 0.f : m[qt];  // nothing visible yet
        float pv[KT][4];
        float ps = 0.f;
#pragma unroll
        for (int kt = 0; kt < KT; ++kt)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            pv[kt][r] = __builtin_amdgcn_exp2f(__builtin_fmaf(st[kt][qt][r], sl2, -mu));
            ps += pv[kt][r];
          }
        l[qt] += ps;
#pragma unroll
        for (int u = 0; u < KT / 2; ++u)
          pb[qt][u] = u32x4{pack2(DT{}, pv[2 * u][0], pv[2 * u][1]), pack2(DT{}, pv[2 * u][2], pv[2 * u][3]),
                            pack2(DT{}, pv[2 * u + 1][0], pv[2 * u + 1][1]),
                            pack2(DT{}, pv[2 * u + 1][2], pv[2 * u + 1][3])};
      }

      // O^T += V^T P^T: A operand = V^T rows 16 dt .. +15 (dims), k = keys
      // {32u + 4 fk .. +3} then {32u + 16 + 4 fk .. +3}, read transposed
#pragma unroll
      for (int u = 0; u < KT / 2; ++u)
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
          const int chunk = 2 * dt + ((fr & 3) >> 1);
          const int key = 32 * u + 4 * fk + (fr >> 2);
          const u32x2 lo = lds_read_tr8(sV, v_off<D>(key, chunk) + 8 * (fr & 1));
          const u32x2 hi = lds_read_tr8(sV, v_off<D>(key + 16, chunk) + 8 * (fr & 1));
          const u32x4 a = u32x4{lo.x, lo.y, hi.x, hi.y};
#pragma unroll
          for (int qt = 0; qt < QT; ++qt) o[dt][qt] = mfma16x16x32(DT{}, a, pb[qt][u], o[dt][qt]);
        }
    }
    // this wave's copies of block j + 1 have landed and every wave is done
    // with block j's stage before it is overwritten
    wait_vm_barrier<0>();
  };
  if constexpr (CAUSAL) {
    // the blocks before the workgroup's first query are visible to all of its
    // queries: a loop without the mask, then the two diagonal blocks with it
    // (11% faster at 4 x 16 x 4096 x 128 than one loop that tests every block,
    // the register pressure of the masking kept out of the long loop)
    const int jfull = q0 / kAttnBN < nblk ? q0 / kAttnBN : nblk;
    for (int j = 0; j < jfull; ++j) run_block.template operator()<false>(j);
    for (int j = jfull; j < nblk; ++j) run_block.template operator()<true>(j);
  } else {
    // non-causal: one loop, the test (for a last block past the sequence
    // end) taken per block -- 1-2% faster than peeling that block
    for (int j = 0; j < nblk; ++j) run_block.template operator()<true>(j);
  }

  if (pass == 0) TG_PHASE(2); else TG_PHASE(6);
  // finish: O = O^T / l, lane writes dims 16 dt + 4 fk .. +3 of its query
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const float inv = 1.0f / reduce_4lanes<false>(l[qt]);
    const int query = q0w + 16 * qt + fr;
    if (query < n) {
      uint16_t* orow = static_cast<uint16_t*>(p.O) + (head * n + query) * (int64_t)D;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        const f32x4 v = o[dt][qt];
        *reinterpret_cast<u32x2*>(orow + 16 * dt + 4 * fk) =
            u32x2{pack2(DT{}, v[0] * inv, v[1] * inv), pack2(DT{}, v[2] * inv, v[3] * inv)};
      }
    }
  }
  if (pass == 0) TG_PHASE_DRAINED(3); else TG_PHASE_DRAINED(7);
  }  // pass: the last block's barrier has released the LDS ring for the next pass
  TG_PHASE_WRITE(attention);
}

template <int D, class DT, bool CAUSAL>
static hipError_t launch_attention(const AttnParams& p, hipStream_t stream) {
  void* args[] = {const_cast<AttnParams*>(&p)};
  return hipLaunchKernel(reinterpret_cast<const void*>(&attention_fwd_kernel<D, DT, CAUSAL>),
                         dim3((unsigned)p.groups), dim3(256), args, 0, stream);
}

template <int D>
static AttnFn attention_launcher_d(int dtype, int causal) {
  if (dtype == TG_DTYPE_F16) return causal ? &launch_attention<D, F16, true> : &launch_attention<D, F16, false>;
  if (dtype == TG_DTYPE_BF16) return causal ? &launch_attention<D, BF16, true> : &launch_attention<D, BF16, false>;
  return nullptr;
}

__host__ AttnFn attention_launcher(int dtype, int head_dim, int causal) {
  if (head_dim == 128) return attention_launcher_d<128>(dtype, causal);
  if (head_dim == 64) return attention_launcher_d<64>(dtype, causal);
  return nullptr;
}

__host__ int attention_block_queries(int head_dim, int causal) {
  if (head_dim == 64) return causal ? attn_bm<64, true>() : attn_bm<64, false>();
  return causal ? attn_bm<128, true>() : attn_bm<128, false>();
}

}  // namespace tg
