// kernels.hpp -- interface between the host dispatch (api.cpp) and the
// compiled kernel variants (gemm.hip, softmax.hip, stream.hip, attention.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/tg.h"

namespace tg {

// Kernel arguments of the 2-D tiled GEMM (sizes already validated on the host
// to fit the kernels' 32-bit offsets).
struct GemmParams {
  const void* A;
  const void* B;
  const void* bias;
  void* C;
  int M, N, K;
  float alpha;
  int epilogue;
  int tiles_m, tiles_n;
  int group_m;
  int xcd_remap;
};

// Kernel arguments of the full-row GEMM + row softmax.
struct SoftmaxParams {
  const void* A;
  const void* B;
  float* C;
  int M, N, K;
  float alpha;
  int n_sub;  // 16-column MFMA tiles per wave: ceil(N / (16 * waves))
};

// Kernel arguments of the vector addition (stream.hip).
struct VectorAddParams {
  const void* A;
  const void* B;
  void* C;
  int64_t n;
};

// Kernel arguments of the standalone row softmax (stream.hip).
struct RowSoftmaxParams {
  const void* X;
  float* Y;
  int64_t rows, cols;
  float alpha;
};

// Kernel arguments of the attention forward (attention.hip).
struct AttnParams {
  const void* Q;
  const void* K;
  const void* V;
  void* O;
  int N;            // sequence length
  int q_blocks;     // query blocks per (batch, head)
  int units;        // workgroups per (batch, head): q_blocks, or ceil(q_blocks / 2) causal pairs
  int groups;       // workgroups: batch * heads * units
  float scale_log2; // |scale| * log2(e)
  int negate_q;     // scale < 0: the kernel flips the sign of Q
};

typedef hipError_t (*VectorAddFn)(const VectorAddParams&, hipStream_t);
typedef hipError_t (*RowSoftmaxFn)(const RowSoftmaxParams&, hipStream_t);

typedef hipError_t (*AttnFn)(const AttnParams&, hipStream_t);

// Launchers for a dtype (and row length / head dim); NULL when unsupported.
VectorAddFn vector_add_launcher(int dtype);
RowSoftmaxFn row_softmax_launcher(int dtype, int64_t cols);
AttnFn attention_launcher(int dtype, int head_dim, int causal);
int attention_block_queries(int head_dim, int causal);  // queries per attention workgroup

typedef hipError_t (*GemmLaunchFn)(const GemmParams&, hipStream_t);
typedef hipError_t (*SoftmaxLaunchFn)(const SoftmaxParams&, hipStream_t);

// One compiled GEMM tile configuration: its description and its launchers,
// indexed [dtype][b_col_major].
struct GemmVariant {
  tg_tile_config cfg;
  GemmLaunchFn fn[2][2];
};
// One compiled row-softmax configuration.
struct SoftmaxVariant {
  tg_tile_config cfg;
  SoftmaxLaunchFn fn[2][2];
};

// Tile-configuration registry (api.cpp) as seen by the autotuner.
int num_tile_configs();
const tg_tile_config* tile_config(int id);                            // NULL if out of range
bool tile_config_runs(int id, int dtype, int b_col_major, int64_t N);  // a kernel exists for this call
void default_choice(int64_t M, int64_t N, int64_t K, int dtype, int epilogue, int b_col_major, int* variant,
                    int* group_m, int* xcd_remap);                     // table / rule, no tuning cache
// Run-time autotune cache (autotune_cache.cpp): true and the tuned choice if
// the exact problem was tuned (or loaded from a cache file); insert or
// replace the entry of a problem.
bool autotune_lookup(int dtype, int b_col_major, int kind, int64_t M, int64_t N, int64_t K, int* variant,
                     int* group_m, int* xcd_remap);
void autotune_cache_put(const tg_autotune_entry& e);

// Variant tables (defined next to the kernels).
const GemmVariant* gemm_variants(int* count);
const SoftmaxVariant* softmax_variants(int* count);

}  // namespace tg
