// autotune_cache.cpp -- the run-time autotuner's cache of tuned problems
// (host code only): lookup by problem, insertion, and the text file it is
// saved to and loaded from.  The search that fills it is in autotune.hip.
//
// The TileLang pages keep the winner of a schedule search per (M, N, K) so
// that the search is paid for once ("TileLang: Criando Kernels ..."
// (noticiai.com.br), section "Exploracao de schedules com autotuning";
// spaxe.top, autotuning paragraph).  tg_gemm / tg_gemm_ex /
// tg_gemm_query_config consult this cache before the baked table.

#include <stdio.h>
#include <string.h>

#include <atomic>
#include <mutex>
#include <vector>

#include "../../include/tg.h"
#include "kernels.hpp"

namespace tg {
namespace {

std::mutex g_mu;
std::vector<tg_autotune_entry> g_cache;  // one entry per tuned problem
std::atomic<int> g_count{0};             // g_cache.size(): lets a lookup skip the lock while empty

bool same_key(const tg_autotune_entry& e, int dtype, int b_col_major, int kind, int64_t M, int64_t N, int64_t K) {
  return e.dtype == dtype && e.b_col_major == b_col_major && e.kind == kind && e.M == M && e.N == N && e.K == K;
}

}  // namespace

void autotune_cache_put(const tg_autotune_entry& e) {
  std::lock_guard<std::mutex> lock(g_mu);
  for (auto& x : g_cache)
    if (same_key(x, e.dtype, e.b_col_major, e.kind, e.M, e.N, e.K)) {
      x = e;
      return;
    }
  g_cache.push_back(e);
  g_count.store((int)g_cache.size(), std::memory_order_release);
}

bool autotune_lookup(int dtype, int b_col_major, int kind, int64_t M, int64_t N, int64_t K, int* variant,
                     int* group_m, int* xcd_remap) {
  if (g_count.load(std::memory_order_acquire) == 0) return false;  // every launch asks; usually nothing tuned
  std::lock_guard<std::mutex> lock(g_mu);
  for (const auto& e : g_cache)
    if (same_key(e, dtype, b_col_major, kind, M, N, K)) {
      *variant = e.config.id;
      *group_m = e.config.group_m;
      *xcd_remap = e.config.xcd_remap;
      return true;
    }
  return false;
}

}  // namespace tg

using namespace tg;

extern "C" {

int tg_autotune_cache_size(void) {
  std::lock_guard<std::mutex> lock(g_mu);
  return (int)g_cache.size();
}

int tg_autotune_cache_get(int index, tg_autotune_entry* out) {
  std::lock_guard<std::mutex> lock(g_mu);
  if (!out || index < 0 || index >= (int)g_cache.size()) return TG_ERR_INVALID_ARG;
  *out = g_cache[index];
  return TG_OK;
}

int tg_autotune_cache_clear(void) {
  std::lock_guard<std::mutex> lock(g_mu);
  g_cache.clear();
  g_count.store(0, std::memory_order_release);
  return TG_OK;
}

// File format: a first line "tg-autotune-cache 1", then one line per entry:
//   dtype b_col_major kind M N K id bm bn bk stages waves group_m xcd_remap us
// The tile fields identify the variant; an entry whose id does not describe
// the same variant in this library (another build) is skipped on load.
int tg_autotune_cache_save(const char* path) {
  if (!path) return TG_ERR_INVALID_ARG;
  std::vector<tg_autotune_entry> copy;
  {
    std::lock_guard<std::mutex> lock(g_mu);
    copy = g_cache;
  }
  FILE* f = fopen(path, "w");
  if (!f) return TG_ERR_INVALID_ARG;
  int ok = fprintf(f, "tg-autotune-cache 1\n") > 0;
  for (const auto& e : copy)
    ok &= fprintf(f, "%d %d %d %lld %lld %lld %d %d %d %d %d %d %d %d %.3f\n", e.dtype, e.b_col_major, e.kind,
                  (long long)e.M, (long long)e.N, (long long)e.K, e.config.id, e.config.bm, e.config.bn, e.config.bk,
                  e.config.stages, e.config.waves, e.config.group_m, e.config.xcd_remap, e.us) > 0;
  ok &= fclose(f) == 0;
  return ok ? TG_OK : TG_ERR_INVALID_ARG;
}

int tg_autotune_cache_load(const char* path, int* loaded, int* skipped) {
  if (!path) return TG_ERR_INVALID_ARG;
  FILE* f = fopen(path, "r");
  if (!f) return TG_ERR_INVALID_ARG;
  char line[512];
  int version = 0;
  if (!fgets(line, sizeof line, f) || sscanf(line, "tg-autotune-cache %d", &version) != 1 || version != 1) {
    fclose(f);
    return TG_ERR_INVALID_ARG;
  }
  int n_ok = 0, n_skip = 0;
  while (fgets(line, sizeof line, f)) {
    int dtype, bcol, kind, id, bm, bn, bk, stages, waves, gm, xcd;
    long long M, N, K;
    float us;
    if (line[0] == '\n' || line[0] == '#') continue;
    const int got = sscanf(line, "%d %d %d %lld %lld %lld %d %d %d %d %d %d %d %d %f", &dtype, &bcol, &kind, &M, &N,
                           &K, &id, &bm, &bn, &bk, &stages, &waves, &gm, &xcd, &us);
    const tg_tile_config* cfg = got == 15 ? tile_config(id) : nullptr;
    tg_tile_config probe;
    const bool ok = cfg && cfg->kind == kind && cfg->bm == bm && cfg->bn == bn && cfg->bk == bk &&
                    cfg->stages == stages && cfg->waves == waves && gm >= 1 && gm <= 4096 && (xcd == 0 || xcd == 1) &&
                    tile_config_runs(id, dtype, bcol, N) &&
                    tg_gemm_query_config(M, N, K, dtype, kind == TG_KERNEL_GEMM_SOFTMAX ? TG_EPI_SOFTMAX : TG_EPI_NONE,
                                         bcol, &probe) == TG_OK;
    if (!ok) {
      ++n_skip;
      continue;
    }
    tg_autotune_entry e;
    memset(&e, 0, sizeof(e));
    e.dtype = dtype;
    e.b_col_major = bcol;
    e.kind = kind;
    e.M = M;
    e.N = N;
    e.K = K;
    e.config = *cfg;
    e.config.group_m = gm;
    e.config.xcd_remap = xcd;
    e.config.b_col_major = bcol;
    e.us = us;
    autotune_cache_put(e);
    ++n_ok;
  }
  fclose(f);
  if (loaded) *loaded = n_ok;
  if (skipped) *skipped = n_skip;
  return TG_OK;
}

}  // extern "C"
