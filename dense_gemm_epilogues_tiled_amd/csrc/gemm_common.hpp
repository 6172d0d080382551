// gemm_common.hpp -- pieces of the tiled GEMM kernel (gemm.hip): compile-time loops, the workgroup -> tile mapping, the
// direct-to-LDS copy plan of one K step and the register epilogue.
#pragma once

#include <type_traits>

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

// A wave-uniform value the optimiser may not look through.  Used for the
// byte offset of a ring slot: otherwise loop strength reduction rewrites
// (k step mod stages) * slot size into one induction variable per LDS read,
// each a live VGPR, which spills in the kernels with the largest tiles.
__device__ __forceinline__ int opaque_sgpr(int v) {
  asm volatile("" : "+s"(v));
  return v;
}

// Wait until at most N vector-memory operations of this wave are in flight,
// then join the workgroup barrier, without waiting for the wave's LDS
// operations: for a barrier that only publishes direct-to-LDS copies (tracked
// by vmcnt).
template <int N>
__device__ __forceinline__ void wait_vm_barrier_only() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" : : "n"(N) : "memory");
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

// Direct-to-LDS copy plan of one BM x BK (A) and BK x BN (B) K step for a
// workgroup of NW waves.  The A tile (and a k-contiguous B tile) is stored in
// the kc_off layout, an n-contiguous B tile in the nc_off layout.  Wave `wave`
// issues the 1 KB blocks q = wave + NW * j of each region; lane i of block q
// fills LDS bytes [1024 q + 16 i, +16) of the region, so the lane fetches the
// (row, chunk) the layout stores there.  Offsets are relative to the tile's
// first element of the step; rows / columns past the matrix get kOOB.
template <int BM, int BN, int BK, int NW, bool B_COL>
struct CopyPlan {
  static constexpr int A_BYTES = BM * BK * 2, B_BYTES = BN * BK * 2;
  static constexpr int DA = A_BYTES / 1024 / NW;
  static constexpr int DB = B_BYTES / 1024 / NW;
  static constexpr int DMA = DA + DB;  // 1 KB copies per wave per K step
  static_assert(DA * 1024 * NW == A_BYTES && DB * 1024 * NW == B_BYTES, "tiles must split into 1 KB per wave");
  static_assert(B_COL || BN >= 128, "n-contiguous B tiles need 128+ columns");

  int a_off[DA], a_kc[DA];  // byte offset, first k of the chunk
  int b_off[DB], b_kc[DB];

  __device__ __forceinline__ void init(int wave, int lane, int m0, int n0, int M, int N, int K) {
    constexpr int KCH = BK / 8;
#pragma unroll
    for (int j = 0; j < DA; ++j) {
      const int pos = 1024 * (wave + NW * j) + 16 * lane;
      const int row = pos / (BK * 2);
      const int slot = (pos % (BK * 2)) / 16;
      const int chunk = slot ^ ((row / (16 / KCH)) % KCH);
      a_off[j] = (m0 + row) < M ? row * K * 2 + chunk * 16 : kOOB;
      a_kc[j] = chunk * 8;
    }
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
  }

  // Copy number q (A copies first, then B) of K step starting at k0 into the
  // stage at LDS byte address `stage`.  Chunks at k >= K are zero-filled, so
  // steps at or past the end of K only write zeros.
  template <int Q>
  __device__ __forceinline__ void copy(int wave, const uint16_t* gA, const uint16_t* gB, int m0, int n0, int N, int K,
                                       int k0, uint32_t stage) const {
    const int k_left = K - k0;
    if constexpr (Q < DA) {
      const __amdgpu_buffer_rsrc_t r = make_rsrc(gA + (size_t)m0 * K + k0);
      dma16(r, stage + 1024 * (wave + NW * Q), a_kc[Q] < k_left ? a_off[Q] : kOOB);
    } else {
      constexpr int J = Q - DA;
      const __amdgpu_buffer_rsrc_t r = make_rsrc(B_COL ? gB + (size_t)n0 * K + k0 : gB + (size_t)k0 * N + n0);
      dma16(r, stage + A_BYTES + 1024 * (wave + NW * J), b_kc[J] < k_left ? b_off[J] : kOOB);
    }
  }
};

// Fragment reads of one 32-deep slice kk of a stage (A tile at sA, B tile at
// sB) for the wave at (wm, wn).  A fragment i: rows 16i .. 16i+15 of the
// wave's A rows; B fragment j: columns 16j .. 16j+15 of its B columns.  Each
// lane ends with the 8 k values of its MFMA operand (see mfma16x16x32).
//
// The per-lane byte offsets are computed once per kernel.  A block of 16 rows
// leaves the kc_off swizzle unchanged, so A fragment i (and B fragment j of a
// k-contiguous B) lies a constant 16*i rows past fragment 0.  For a row-major
// B the swizzle XORs into the column-block bits, so each 16-column block gets
// its own offset; k + 4 and k + 32 keep nc_swz(k), so the second half of a
// fragment and the next slice lie constant distances away.  Constant parts
// become the LDS instructions' immediate offsets: each read costs at most one
// address add for the stage slot.
template <int BN, int BK, int WTM, int WTN, int FN, bool B_COL>
struct FragAddr {
  static constexpr int KK = BK / 32;
  int a[KK];
  int b[B_COL ? KK : FN];

  __device__ __forceinline__ void init(int wm, int wn, int fr, int fk) {
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) a[kk] = kc_off<BK>(wm * WTM + fr, 4 * kk + fk);
    if constexpr (B_COL) {
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) b[kk] = kc_off<BK>(wn * WTN + fr, 4 * kk + fk);
    } else {
      // lanes 4q..4q+3 of each 16-lane group read row k = 8fk + 4h + q
#pragma unroll
      for (int j = 0; j < FN; ++j)
        b[j] = nc_off<BN>(8 * fk + (fr >> 2), (wn * WTN + 16 * j) / 8 + ((fr & 3) >> 1)) + 8 * (fr & 1);
    }
  }
  __device__ __forceinline__ u32x4 read_a(const unsigned char* sA, int i, int kk) const {
    return lds_read16(sA + a[kk], i * 16 * BK * 2);
  }
  __device__ __forceinline__ u32x4 read_b(const unsigned char* sB, int j, int kk) const {
    if constexpr (B_COL) {
      return lds_read16(sB + b[kk], j * 16 * BK * 2);
    } else {
      const unsigned char* q = sB + b[j];
      const u32x2 lo = lds_read_tr8(q, 32 * kk * BN * 2);
      const u32x2 hi = lds_read_tr8(q, (32 * kk + 4) * BN * 2);
      return u32x4{lo.x, lo.y, hi.x, hi.y};
    }
  }
};

// bias[n .. n+3] widened to fp32 (zeros without a bias epilogue).
template <int EPI, class DT>
__device__ __forceinline__ f32x4 load_bias4(const GemmParams& p, int n) {
  if constexpr (EPI == EPI_NONE) {
    return f32x4{0.f, 0.f, 0.f, 0.f};
  } else {
    const u32x2 bb = *reinterpret_cast<const u32x2*>(static_cast<const uint16_t*>(p.bias) + n);
    return f32x4{lo_to_f32(DT{}, bb.x), hi_to_f32(DT{}, bb.x), lo_to_f32(DT{}, bb.y), hi_to_f32(DT{}, bb.y)};
  }
}

// Four consecutive outputs of one row: x = alpha * acc + bias, the
// activation, one rounding to the output type, packed for one 8-byte store.
template <int EPI, class DT>
__device__ __forceinline__ u32x2 finish4(float alpha, const f32x4& a, const f32x4& b) {
  float x[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    x[e] = __builtin_fmaf(alpha, a[e], b[e]);
    if constexpr (EPI == EPI_RELU) x[e] = __builtin_fmaxf(x[e], 0.f);
    if constexpr (EPI == EPI_GELU) x[e] = gelu_erf(x[e]);
  }
  return u32x2{pack2(DT{}, x[0], x[1]), pack2(DT{}, x[2], x[3])};
}

// Epilogue through LDS.  Every wave finishes its 16x16 MFMA tiles in
// registers (lane (fr, fk) of tile (i, j) holds C[r0 + 16i + fr][c0 + 16j +
// 4fk + 0..3] of the tile), packs them to the output type and writes them into
// a BM x BN row-major image of the tile in LDS; after a workgroup barrier all
// NT threads copy the image to C as 16-byte pieces, consecutive lanes taking
// consecutive pieces of a row, so each store instruction writes whole rows of
// the tile instead of 16 scattered 32-byte pieces.  In the image the 8-byte
// unit u of row r sits at unit u ^ (2 (r % 16)): the fragment writes (16 rows
// at one unit) and the row reads (16 bytes per lane) are both free of bank
// conflicts, and a 16-byte piece (units 2v, 2v+1) stays contiguous.
// Requires BM * BN * 2 bytes of LDS no longer in use (the caller has waited
// for its copies and passed a barrier after its last fragment read).
template <int BN>
__device__ __forceinline__ int c_image_off(int r, int u) {
  return r * (BN * 2) + 8 * (u ^ ((r & 15) << 1));
}

// Bias, activation and the one rounding of a wave's accumulator tiles, in
// registers: out[i][j] holds the 4 results of acc[i][j] packed to 16 bits.
// It touches no LDS, so it can run before the barrier that frees the operand
// ring, overlapping other waves' last MFMAs.
template <int EPI, class DT, int FM, int FN>
__device__ __forceinline__ void finish_tile(const GemmParams& p, const f32x4 (&acc)[FM][FN], u32x2 (&out)[FM][FN],
                                            int n0, int c0, int fk) {
  const int N = p.N;
#pragma unroll
  for (int j = 0; j < FN; ++j) {
    const int n = n0 + c0 + 16 * j + 4 * fk;
    const f32x4 b = n < N ? load_bias4<EPI, DT>(p, n) : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < FM; ++i) out[i][j] = finish4<EPI, DT>(p.alpha, acc[i][j], b);
  }
}

// Write finished tiles to C through an LDS image of the BM x BN tile, so each
// lane stores whole 16-byte row pieces.  The ring must be free (barrier
// passed) when this starts.
template <class DT, int BM, int BN, int NT, int FM, int FN>
__device__ __forceinline__ void store_tile_staged(const GemmParams& p, const u32x2 (&out)[FM][FN],
                                                  unsigned char* smem, int m0, int n0, int r0, int c0, int fr,
                                                  int fk, int tid) {
  static_assert(BM * BN / 8 % NT == 0, "whole rounds of 16-byte pieces");
  const int M = p.M, N = p.N;
#pragma unroll
  for (int j = 0; j < FN; ++j) {
    const int c = c0 + 16 * j + 4 * fk;  // column inside the tile
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int r = r0 + 16 * i + fr;
      *reinterpret_cast<u32x2*>(smem + c_image_off<BN>(r, c / 4)) = out[i][j];
    }
  }
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  uint16_t* __restrict__ gC = static_cast<uint16_t*>(p.C);
  constexpr int PIECES_PER_ROW = BN / 8;
#pragma unroll
  for (int q = tid; q < BM * BN / 8; q += NT) {
    const int r = q / PIECES_PER_ROW, v = q % PIECES_PER_ROW;
    const int m = m0 + r, n = n0 + 8 * v;
    const u32x4 val = *reinterpret_cast<const u32x4*>(smem + c_image_off<BN>(r, 2 * v));
    // plain stores: for this kernel non-temporal ones measured the same at
    // 8192^3 and 4.6% slower at 3000 x 5000 x 1000 (one tile per CU)
    if (m < M && n < N) *reinterpret_cast<u32x4*>(gC + (size_t)m * N + n) = val;
  }
}

// Dispatch the runtime epilogue code to a compile-time one.
template <class F>
__device__ __forceinline__ void with_epilogue(int epi, F&& f) {
  switch (epi) {
    case EPI_RELU: f(std::integral_constant<int, EPI_RELU>{}); break;
    case EPI_GELU: f(std::integral_constant<int, EPI_GELU>{}); break;
    case EPI_BIAS: f(std::integral_constant<int, EPI_BIAS>{}); break;
    default: f(std::integral_constant<int, EPI_NONE>{}); break;
  }
}

}  // namespace tg
