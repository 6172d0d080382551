// api.cpp -- the C ABI of include/tg.h: argument validation, tile
// configuration lookup and kernel launch.
//
// The per-shape configuration choice mirrors the TileLang pages' autotuning
// (noticiai.com.br, section "Exploracao de schedules com autotuning": a search
// over tile sizes and warp counts keyed on (M, N, K), cached; spaxe.top,
// autotuning paragraph): here the search runs offline (sweep.py) and its
// winners are baked into config_table.inc; shapes without an entry fall back
// to a rule that keeps every compute unit busy with the largest tile.

#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "../../include/tg.h"
#include "kernels.hpp"

namespace tg {
namespace {

// Compute units of an MI355X; the fallback rule aims for at least one tile per CU.
constexpr int kNumCUs = 256;

// All compiled configurations: the GEMM variants (gemm.hip) with ids
// 0 .. G-1, then the row-softmax variants (softmax.hip) with ids G ...
constexpr int kMaxConfigs = 64;
struct Registry {
  const GemmVariant* gemm;
  const SoftmaxVariant* softmax;
  int n_gemm, n_softmax;
  tg_tile_config cfg[kMaxConfigs];
  int n;
};

const Registry& registry() {
  static const Registry r = [] {
    Registry x{};
    x.gemm = gemm_variants(&x.n_gemm);
    if (x.n_gemm > kMaxConfigs) x.n_gemm = kMaxConfigs;
    x.softmax = softmax_variants(&x.n_softmax);
    if (x.n_softmax > kMaxConfigs - x.n_gemm) x.n_softmax = kMaxConfigs - x.n_gemm;
    x.n = 0;
    for (int i = 0; i < x.n_gemm; ++i) x.cfg[x.n++] = x.gemm[i].cfg;
    for (int i = 0; i < x.n_softmax; ++i) x.cfg[x.n++] = x.softmax[i].cfg;
    for (int i = 0; i < x.n; ++i) x.cfg[i].id = i;
    return x;
  }();
  return r;
}

// Baked per-shape choices written by the offline sweep.
struct TableEntry {
  int dtype, b_col_major, epilogue_kind;  // epilogue_kind: 0 elementwise, 1 softmax
  int64_t M, N, K;
  int variant, group_m, xcd_remap;
};
#include "config_table.inc"
constexpr int kNumTable = sizeof(kTable) / sizeof(kTable[0]);

bool log_enabled() {
  const char* v = getenv("TG_LOG");
  return v && v[0] && v[0] != '0';
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct Choice {
  int variant;
  int group_m;
  int xcd_remap;
};

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Shape checks shared by the launch and the query (no pointers involved).
int check_shape(int64_t M, int64_t N, int64_t K, int dtype, int epilogue, int b_col_major) {
  if (dtype != TG_DTYPE_F16 && dtype != TG_DTYPE_BF16) return TG_ERR_INVALID_ARG;
  if (epilogue < TG_EPI_NONE || epilogue > TG_EPI_SOFTMAX) return TG_ERR_INVALID_ARG;
  if (b_col_major != 0 && b_col_major != 1) return TG_ERR_INVALID_ARG;
  if (M < 0 || N < 0 || K < 0) return TG_ERR_INVALID_ARG;
  if (M >= (int64_t(1) << 31) || N > (int64_t(1) << 24) || K > (int64_t(1) << 20)) return TG_ERR_UNSUPPORTED;
  if (epilogue == TG_EPI_SOFTMAX && N > TG_SOFTMAX_MAX_N) return TG_ERR_UNSUPPORTED;
  if ((N & 7) != 0 || (K & 7) != 0) return TG_ERR_MISALIGNED;
  return TG_OK;
}

int softmax_capacity(const tg_tile_config& v) { return v.bn; }

int64_t tiles_of(const tg_tile_config& c, int64_t M, int64_t N) { return cdiv(M, c.bm) * cdiv(N, c.bn); }

// Lookup: baked entry for the exact shape, else the fallback rule.
Choice choose_default(int64_t M, int64_t N, int64_t K, int dtype, int epilogue, int b_col_major) {
  const Registry& R = registry();
  const int kind = epilogue == TG_EPI_SOFTMAX ? 1 : 0;
  for (int i = 0; i < kNumTable; ++i) {
    const TableEntry& e = kTable[i];
    if (e.dtype == dtype && e.b_col_major == b_col_major && e.epilogue_kind == kind && e.M == M && e.N == N &&
        e.K == K && e.variant >= 0 && e.variant < R.n && R.cfg[e.variant].kind == kind &&
        (kind == 0 || R.softmax[e.variant - R.n_gemm].fn[dtype][b_col_major]))
      return {e.variant, e.group_m, e.xcd_remap};
  }
  if (kind == 1) {
    // a softmax variant whose row capacity covers N and that has a kernel for
    // this B layout; variants built for exactly this layout first, then the
    // fewest waves
    int best = -1;
    for (int i = R.n_gemm; i < R.n; ++i) {
      if (R.cfg[i].bn < N || !R.softmax[i - R.n_gemm].fn[dtype][b_col_major]) continue;
      const bool exact = R.cfg[i].b_col_major == b_col_major;
      if (best < 0) { best = i; continue; }
      const bool best_exact = R.cfg[best].b_col_major == b_col_major;
      if ((exact && !best_exact) || (exact == best_exact && R.cfg[i].waves < R.cfg[best].waves)) best = i;
    }
    return {best, 1, 0};
  }
  // the largest tile that still gives every CU at least one tile; failing
  // that (small problems), the variant with the most tiles
  int best = -1;
  for (int i = 0; i < R.n_gemm; ++i) {
    const tg_tile_config& c = R.cfg[i];
    if (tiles_of(c, M, N) < kNumCUs) continue;
    if (best < 0 || c.bm * c.bn > R.cfg[best].bm * R.cfg[best].bn ||
        (c.bm * c.bn == R.cfg[best].bm * R.cfg[best].bn && c.bk > R.cfg[best].bk))
      best = i;
  }
  if (best < 0) {
    best = 0;
    for (int i = 1; i < R.n_gemm; ++i)
      if (tiles_of(R.cfg[i], M, N) > tiles_of(R.cfg[best], M, N)) best = i;
  }
  return {best, R.cfg[best].group_m, R.cfg[best].xcd_remap};
}

// Lookup: a run-time autotuned entry for the exact shape first (autotune.hip),
// then the baked table and the fallback rule.
Choice choose(int64_t M, int64_t N, int64_t K, int dtype, int epilogue, int b_col_major) {
  const int kind = epilogue == TG_EPI_SOFTMAX ? 1 : 0;
  Choice c;
  if (autotune_lookup(dtype, b_col_major, kind, M, N, K, &c.variant, &c.group_m, &c.xcd_remap) &&
      c.variant >= 0 && c.variant < registry().n && registry().cfg[c.variant].kind == kind)
    return c;
  return choose_default(M, N, K, dtype, epilogue, b_col_major);
}

}  // namespace

// Internal interface for the autotuner (kernels.hpp).
int num_tile_configs() { return registry().n; }

const tg_tile_config* tile_config(int id) {
  return id >= 0 && id < registry().n ? &registry().cfg[id] : nullptr;
}

bool tile_config_runs(int id, int dtype, int b_col_major, int64_t N) {
  const Registry& R = registry();
  if (id < 0 || id >= R.n || (dtype != TG_DTYPE_F16 && dtype != TG_DTYPE_BF16) || (b_col_major & ~1)) return false;
  if (R.cfg[id].kind == TG_KERNEL_GEMM) return R.gemm[id].fn[dtype][b_col_major] != nullptr;
  return R.softmax[id - R.n_gemm].fn[dtype][b_col_major] != nullptr && N <= softmax_capacity(R.cfg[id]);
}

void default_choice(int64_t M, int64_t N, int64_t K, int dtype, int epilogue, int b_col_major, int* variant,
                    int* group_m, int* xcd_remap) {
  const Choice c = choose_default(M, N, K, dtype, epilogue, b_col_major);
  *variant = c.variant;
  *group_m = c.group_m;
  *xcd_remap = c.xcd_remap;
}

}  // namespace tg

using namespace tg;

extern "C" {

int tg_version(void) { return TG_VERSION_MAJOR * 100 + TG_VERSION_MINOR; }

const char* tg_status_string(int status) {
  switch (status) {
    case TG_OK: return "TG_OK: success";
    case TG_ERR_INVALID_ARG: return "TG_ERR_INVALID_ARG: invalid argument";
    case TG_ERR_UNSUPPORTED: return "TG_ERR_UNSUPPORTED: request outside the implemented kernels";
    case TG_ERR_MISALIGNED: return "TG_ERR_MISALIGNED: pointer not 16-byte aligned or N/K not a multiple of 8";
    case TG_ERR_HIP: return "TG_ERR_HIP: the HIP runtime rejected the launch";
    default: return "unknown tg status";
  }
}

int tg_num_configs(void) { return registry().n; }

int tg_get_config(int index, tg_tile_config* out) {
  if (!out || index < 0 || index >= registry().n) return TG_ERR_INVALID_ARG;
  *out = registry().cfg[index];
  return TG_OK;
}

int tg_gemm_query_config(int64_t M, int64_t N, int64_t K, int dtype, int epilogue, int b_col_major,
                         tg_tile_config* out) {
  if (!out) return TG_ERR_INVALID_ARG;
  const int rc = check_shape(M, N, K, dtype, epilogue, b_col_major);
  if (rc != TG_OK) return rc;
  const Choice c = choose(M, N, K, dtype, epilogue, b_col_major);
  if (c.variant < 0) return TG_ERR_UNSUPPORTED;
  *out = registry().cfg[c.variant];
  out->group_m = c.group_m;
  out->xcd_remap = c.xcd_remap;
  out->b_col_major = b_col_major;
  return TG_OK;
}

int tg_gemm_ex(const tg_gemm_args* a, void* stream) {
  if (!a) return TG_ERR_INVALID_ARG;
  int rc = check_shape(a->M, a->N, a->K, a->dtype, a->epilogue, a->b_col_major);
  if (rc != TG_OK) return rc;
  const bool wants_bias = a->epilogue == TG_EPI_BIAS || a->epilogue == TG_EPI_BIAS_RELU ||
                          a->epilogue == TG_EPI_BIAS_GELU;
  if (wants_bias != (a->bias != nullptr)) return TG_ERR_INVALID_ARG;
  const int kind = a->epilogue == TG_EPI_SOFTMAX ? TG_KERNEL_GEMM_SOFTMAX : TG_KERNEL_GEMM;

  const Registry& R = registry();
  Choice c;
  if (a->config_id >= 0) {
    if (a->config_id >= R.n || R.cfg[a->config_id].kind != kind) return TG_ERR_INVALID_ARG;
    if (kind == TG_KERNEL_GEMM_SOFTMAX && !R.softmax[a->config_id - R.n_gemm].fn[a->dtype][a->b_col_major])
      return TG_ERR_INVALID_ARG;  // variant built for the other B layout
    c = {a->config_id, R.cfg[a->config_id].group_m, R.cfg[a->config_id].xcd_remap};
    if (kind == TG_KERNEL_GEMM_SOFTMAX && a->N > softmax_capacity(R.cfg[a->config_id])) return TG_ERR_UNSUPPORTED;
  } else {
    c = choose(a->M, a->N, a->K, a->dtype, a->epilogue, a->b_col_major);
    if (c.variant < 0) return TG_ERR_UNSUPPORTED;
  }
  if (a->group_m < 0 || a->group_m > 4096 || a->xcd_remap < -1 || a->xcd_remap > 1) return TG_ERR_INVALID_ARG;
  if (a->group_m > 0) c.group_m = a->group_m;
  if (a->xcd_remap >= 0) c.xcd_remap = a->xcd_remap;

  if (a->M == 0 || a->N == 0) return TG_OK;  // empty output: nothing to launch
  if (!a->C || (a->K > 0 && (!a->A || !a->B))) return TG_ERR_INVALID_ARG;
  if (!aligned16(a->C) || (a->K > 0 && (!aligned16(a->A) || !aligned16(a->B))) ||
      (a->bias && !aligned16(a->bias)))
    return TG_ERR_MISALIGNED;

  const tg_tile_config& v = R.cfg[c.variant];
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t err;
  int grid = 0;
  if (kind == TG_KERNEL_GEMM) {
    GemmParams p;
    p.A = a->A;
    p.B = a->B;
    p.bias = a->bias;
    p.C = a->C;
    p.M = (int)a->M;
    p.N = (int)a->N;
    p.K = (int)a->K;
    p.alpha = a->alpha;
    p.epilogue = a->epilogue;
    p.tiles_m = (int)cdiv(a->M, v.bm);
    p.tiles_n = (int)cdiv(a->N, v.bn);
    p.group_m = c.group_m > 0 ? c.group_m : 1;
    p.xcd_remap = c.xcd_remap;
    if ((int64_t)p.tiles_m * p.tiles_n >= (int64_t(1) << 31)) return TG_ERR_UNSUPPORTED;
    grid = p.tiles_m * p.tiles_n;
    err = R.gemm[c.variant].fn[a->dtype][a->b_col_major](p, s);
  } else {
    SoftmaxParams p;
    p.A = a->A;
    p.B = a->B;
    p.C = static_cast<float*>(a->C);
    p.M = (int)a->M;
    p.N = (int)a->N;
    p.K = (int)a->K;
    p.alpha = a->alpha;
    p.n_sub = (int)cdiv(a->N, 16 * v.waves);
    grid = (int)cdiv(a->M, v.bm);
    err = R.softmax[c.variant - R.n_gemm].fn[a->dtype][a->b_col_major](p, s);
  }
  if (log_enabled())
    fprintf(stderr, "tg: M=%lld N=%lld K=%lld dtype=%d epi=%d bcol=%d cfg=%d (%dx%d) grid=%d group_m=%d xcd=%d -> %s\n",
            (long long)a->M, (long long)a->N, (long long)a->K, a->dtype, a->epilogue, a->b_col_major, c.variant, v.bm,
            v.bn, grid, c.group_m, c.xcd_remap, hipGetErrorString(err));
  return err == hipSuccess ? TG_OK : TG_ERR_HIP;
}

int tg_vector_add(const void* A, const void* B, void* C, int64_t n, int dtype, void* stream) {
  if (n < 0) return TG_ERR_INVALID_ARG;
  const VectorAddFn fn = vector_add_launcher(dtype);
  if (!fn) return TG_ERR_INVALID_ARG;
  if (n > (int64_t(1) << 36)) return TG_ERR_UNSUPPORTED;  // keeps the one-vector-per-thread grid < 2^31
  if (n == 0) return TG_OK;
  if (!A || !B || !C) return TG_ERR_INVALID_ARG;
  if (!aligned16(A) || !aligned16(B) || !aligned16(C)) return TG_ERR_MISALIGNED;
  const hipError_t err = fn(VectorAddParams{A, B, C, n}, static_cast<hipStream_t>(stream));
  if (log_enabled())
    fprintf(stderr, "tg: vector_add n=%lld dtype=%d -> %s\n", (long long)n, dtype, hipGetErrorString(err));
  return err == hipSuccess ? TG_OK : TG_ERR_HIP;
}

int tg_row_softmax(const void* X, float* Y, int64_t rows, int64_t cols, int dtype, float alpha, void* stream) {
  if (rows < 0 || cols < 0) return TG_ERR_INVALID_ARG;
  if (dtype != TG_DTYPE_F16 && dtype != TG_DTYPE_BF16 && dtype != TG_DTYPE_F32) return TG_ERR_INVALID_ARG;
  const int64_t esize = dtype == TG_DTYPE_F32 ? 4 : 2;
  if (rows >= (int64_t(1) << 31) || cols > TG_ROW_SOFTMAX_MAX_ROW_BYTES / esize) return TG_ERR_UNSUPPORTED;
  if ((cols * esize) % 16 != 0) return TG_ERR_MISALIGNED;
  if (rows == 0 || cols == 0) return TG_OK;
  if (!X || !Y) return TG_ERR_INVALID_ARG;
  if (!aligned16(X) || !aligned16(Y)) return TG_ERR_MISALIGNED;
  const RowSoftmaxFn fn = row_softmax_launcher(dtype, cols);
  if (!fn) return TG_ERR_UNSUPPORTED;
  const hipError_t err = fn(RowSoftmaxParams{X, Y, rows, cols, alpha}, static_cast<hipStream_t>(stream));
  if (log_enabled())
    fprintf(stderr, "tg: row_softmax rows=%lld cols=%lld dtype=%d -> %s\n", (long long)rows, (long long)cols, dtype,
            hipGetErrorString(err));
  return err == hipSuccess ? TG_OK : TG_ERR_HIP;
}

int tg_attention_fwd(const void* Q, const void* K, const void* V, void* O, int64_t batch, int64_t heads,
                     int64_t seq_len, int64_t head_dim, int dtype, int causal, float scale, void* stream) {
  if (batch < 0 || heads < 0 || seq_len < 0 || head_dim < 0) return TG_ERR_INVALID_ARG;
  if (dtype != TG_DTYPE_F16 && dtype != TG_DTYPE_BF16) return TG_ERR_INVALID_ARG;
  if (causal != 0 && causal != 1) return TG_ERR_INVALID_ARG;
  if (!isfinite(scale)) return TG_ERR_INVALID_ARG;
  const AttnFn fn = attention_launcher(dtype, (int)(head_dim > 1024 ? 0 : head_dim), causal);
  if (!fn || seq_len > TG_ATTN_MAX_SEQ) return TG_ERR_UNSUPPORTED;
  const int64_t bm = attention_block_queries((int)head_dim, causal);
  const int64_t q_blocks = cdiv(seq_len, bm);
  if (heads > 0 && batch > ((int64_t(1) << 31) - 1) / heads) return TG_ERR_UNSUPPORTED;
  const int64_t units = causal ? (q_blocks + 1) / 2 : q_blocks;  // causal: pairs of query blocks
  const int64_t groups = batch * heads * units;
  if (groups >= (int64_t(1) << 31)) return TG_ERR_UNSUPPORTED;
  if (groups == 0) return TG_OK;
  if (!Q || !K || !V || !O) return TG_ERR_INVALID_ARG;
  if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O)) return TG_ERR_MISALIGNED;
  AttnParams p;
  p.Q = Q;
  p.K = K;
  p.V = V;
  p.O = O;
  p.N = (int)seq_len;
  p.q_blocks = (int)q_blocks;
  p.units = (int)units;
  p.groups = (int)groups;
  // |scale| log2 e, kept strictly positive: a masked score is -inf and
  // -inf * 0 would be NaN; 2^-100 times any finite score is below 2^-25, whose
  // exp2 is exactly 1, the same as for a zero scale
  p.scale_log2 = fabsf(scale) * 1.4426950408889634f;
  if (!(p.scale_log2 >= 0x1p-100f)) p.scale_log2 = 0x1p-100f;
  p.negate_q = scale < 0.f ? 1 : 0;
  const hipError_t err = fn(p, static_cast<hipStream_t>(stream));
  if (log_enabled())
    fprintf(stderr, "tg: attention_fwd B=%lld H=%lld N=%lld D=%lld dtype=%d causal=%d grid=%lld -> %s\n",
            (long long)batch, (long long)heads, (long long)seq_len, (long long)head_dim, dtype, causal,
            (long long)groups, hipGetErrorString(err));
  return err == hipSuccess ? TG_OK : TG_ERR_HIP;
}

int tg_gemm(const void* A, const void* B, const void* bias, void* C, int64_t M, int64_t N, int64_t K, int dtype,
            int epilogue, void* stream) {
  tg_gemm_args a;
  a.A = A;
  a.B = B;
  a.bias = bias;
  a.C = C;
  a.M = M;
  a.N = N;
  a.K = K;
  a.dtype = dtype;
  a.epilogue = epilogue;
  a.b_col_major = 0;
  a.alpha = 1.0f;
  a.config_id = -1;
  a.group_m = 0;
  a.xcd_remap = -1;
  return tg_gemm_ex(&a, stream);
}

}  // extern "C"
