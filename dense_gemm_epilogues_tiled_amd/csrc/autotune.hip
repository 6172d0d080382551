// autotune.hip -- run-time per-shape tile-configuration search.
//
// The TileLang pages tune a GEMM's schedule per matrix shape: a search space
// over tile sizes, warp counts and pipelining, keyed on (M, N, K); every
// candidate is compiled, benchmarked and validated, and the winner is cached
// so the search is paid for once ("TileLang: Criando Kernels ..."
// (noticiai.com.br), section "Exploracao de schedules com autotuning"; the
// edgex.exchange page's autotuning paragraph; spaxe.top, autotuning
// paragraph).  Here every candidate is already compiled (the variants of
// gemm.hip / softmax.hip), so a search times each compatible variant -- and,
// for the 2-D tiled kernels, each raster band height and the per-XCD
// regrouping -- on the caller's own buffers, checks its output against the
// output of the default choice on the device, and stores the fastest valid
// one in the cache (autotune_cache.cpp, host code only), which tg_gemm /
// tg_gemm_ex / tg_gemm_query_config consult before the baked table.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdio.h>
#include <string.h>

#include <mutex>

#include "../../include/tg.h"
#include "kernels.hpp"

namespace tg {
namespace {

// ---------------------------------------------------------------------------
// Validation on the device: the number of elements of C that differ from the
// reference output by more than atol + rtol |ref| (or that are not finite
// where the reference is, or the other way round).  Each block writes its
// own count; the host adds them.
// ---------------------------------------------------------------------------
constexpr int kCmpBlocks = 1024;

__device__ __forceinline__ float out_value(const void* p, int64_t i, int out_kind) {
  if (out_kind == 2) return static_cast<const float*>(p)[i];
  const uint32_t w = static_cast<const uint16_t*>(p)[i];
  if (out_kind == 1) return __builtin_bit_cast(float, w << 16);
  return (float)__builtin_bit_cast(_Float16, (uint16_t)w);
}

__global__ __launch_bounds__(256) void count_mismatch_kernel(const void* c, const void* r, int64_t n, int out_kind,
                                                             float atol, float rtol, unsigned* partial) {
  unsigned bad = 0;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    const float x = out_value(c, i, out_kind), y = out_value(r, i, out_kind);
    const bool fx = __builtin_isfinite(x), fy = __builtin_isfinite(y);
    if (fx != fy || (fx && !(__builtin_fabsf(x - y) <= atol + rtol * __builtin_fabsf(y))) ||
        (!fx && !fy && !(x == y || (x != x && y != y))))
      ++bad;
  }
  __shared__ unsigned red[256];
  red[threadIdx.x] = bad;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if ((int)threadIdx.x < o) red[threadIdx.x] += red[threadIdx.x + o];
    __syncthreads();
  }
  if (threadIdx.x == 0) partial[blockIdx.x] = red[0];
}

// Reads of the GPU's constant 100 MHz clock, in stream order: one thread
// writes the counter (vector store) where the host asked.  Two such reads
// around a candidate's launches time them without HIP events (whose creation
// allocates).
__global__ __launch_bounds__(64) void clock_stamp_kernel(unsigned long long* out) {
  const unsigned long long t = __builtin_amdgcn_s_memrealtime();
  if (threadIdx.x == 0) out[0] = t;
}

int64_t out_bytes(int64_t M, int64_t N, int epilogue) { return M * N * (epilogue == TG_EPI_SOFTMAX ? 4 : 2); }
int64_t align256(int64_t x) { return (x + 255) & ~int64_t(255); }
// workspace layout: reference output | kCmpBlocks mismatch counts | 2 clock stamps
constexpr int64_t kTailBytes = kCmpBlocks * sizeof(unsigned) + 256;

}  // namespace
}  // namespace tg

using namespace tg;

extern "C" {

int tg_gemm_autotune_workspace_size(int64_t M, int64_t N, int epilogue, int64_t* bytes) {
  if (!bytes || M < 0 || N < 0 || epilogue < TG_EPI_NONE || epilogue > TG_EPI_SOFTMAX) return TG_ERR_INVALID_ARG;
  if (M >= (int64_t(1) << 31) || N > (int64_t(1) << 24)) return TG_ERR_UNSUPPORTED;  // the GEMM's own limits
  *bytes = align256(out_bytes(M, N, epilogue)) + kTailBytes;
  return TG_OK;
}

}  // extern "C"

namespace tg {
namespace {

// Argument checks shared by both entry points (no HIP call); *need receives
// the workspace bytes the problem takes.
int autotune_check(const tg_gemm_args* args, int iters, const tg_autotune_entry* result, int64_t* need) {
  if (!args || !result || iters < 1 || iters > 1000) return TG_ERR_INVALID_ARG;
  tg_tile_config probe;
  int rc = tg_gemm_query_config(args->M, args->N, args->K, args->dtype, args->epilogue, args->b_col_major, &probe);
  if (rc != TG_OK) return rc;
  rc = tg_gemm_autotune_workspace_size(args->M, args->N, args->epilogue, need);
  if (rc != TG_OK) return rc;
  if (args->M == 0 || args->N == 0) return TG_ERR_INVALID_ARG;  // nothing to time
  return TG_OK;
}

// The search, on a checked problem, with `workspace` (256-byte aligned, at
// least the problem's workspace size) for the reference output, the
// mismatch counts and the clock stamps.
int autotune_run(const tg_gemm_args* args, void* workspace, int iters, tg_autotune_entry* result, void* stream) {
  int rc;
  const int kind = args->epilogue == TG_EPI_SOFTMAX ? TG_KERNEL_GEMM_SOFTMAX : TG_KERNEL_GEMM;
  hipStream_t s = static_cast<hipStream_t>(stream);

  // the reference: the default choice (baked table / rule), written to the workspace
  int dv, dg, dx;
  default_choice(args->M, args->N, args->K, args->dtype, args->epilogue, args->b_col_major, &dv, &dg, &dx);
  tg_gemm_args ref = *args;
  ref.C = workspace;
  ref.config_id = dv;
  ref.group_m = dg > 0 ? dg : 1;
  ref.xcd_remap = dx;
  rc = tg_gemm_ex(&ref, stream);
  if (rc != TG_OK) return rc;

  const int64_t n_out = args->M * args->N;
  const int out_kind = args->epilogue == TG_EPI_SOFTMAX ? 2 : args->dtype;
  const float tol = args->epilogue == TG_EPI_SOFTMAX ? 1e-4f : 1e-2f;
  unsigned* partial = reinterpret_cast<unsigned*>(static_cast<unsigned char*>(workspace) +
                                                  align256(out_bytes(args->M, args->N, args->epilogue)));
  unsigned long long* stamps = reinterpret_cast<unsigned long long*>(partial + kCmpBlocks);
  const int cmp_blocks = (int)(n_out / 2048 + 1 < kCmpBlocks ? n_out / 2048 + 1 : kCmpBlocks);
  unsigned host_partial[kCmpBlocks];
  unsigned long long host_stamps[2];

  static const int kGroups[] = {1, 4, 8, 16};
  tg_gemm_args best = *args;
  float best_us = -1.f;
  int tried = 0, valid = 0;
  for (int id = 0; id < num_tile_configs(); ++id) {
    const tg_tile_config* cfg = tile_config(id);
    if (cfg->kind != kind || !tile_config_runs(id, args->dtype, args->b_col_major, args->N)) continue;
    const int ng = kind == TG_KERNEL_GEMM ? 4 : 1, nx = kind == TG_KERNEL_GEMM ? 2 : 1;
    for (int gi = 0; gi < ng; ++gi)
      for (int x = 0; x < nx; ++x) {
        tg_gemm_args c = *args;
        c.config_id = id;
        c.group_m = kind == TG_KERNEL_GEMM ? kGroups[gi] : 1;
        c.xcd_remap = kind == TG_KERNEL_GEMM ? x : 0;
        ++tried;
        if (tg_gemm_ex(&c, stream) != TG_OK) continue;  // e.g. a variant the problem cannot use
        // validate against the reference
        hipLaunchKernelGGL(count_mismatch_kernel, dim3(cmp_blocks), dim3(256), 0, s, args->C, workspace, n_out,
                           out_kind, tol, tol, partial);
        if (hipGetLastError() != hipSuccess) return TG_ERR_HIP;
        if (hipMemcpyAsync(host_partial, partial, cmp_blocks * sizeof(unsigned), hipMemcpyDeviceToHost, s) !=
                hipSuccess ||
            hipStreamSynchronize(s) != hipSuccess)
          return TG_ERR_HIP;
        uint64_t bad = 0;
        for (int b = 0; b < cmp_blocks; ++b) bad += host_partial[b];
        if (bad != 0) continue;
        ++valid;
        // time: one more warm launch, then `iters` launches between two clock stamps
        if (tg_gemm_ex(&c, stream) != TG_OK) continue;
        hipLaunchKernelGGL(clock_stamp_kernel, dim3(1), dim3(64), 0, s, stamps);
        for (int i = 0; i < iters; ++i) (void)tg_gemm_ex(&c, stream);
        hipLaunchKernelGGL(clock_stamp_kernel, dim3(1), dim3(64), 0, s, stamps + 1);
        if (hipGetLastError() != hipSuccess ||
            hipMemcpyAsync(host_stamps, stamps, sizeof host_stamps, hipMemcpyDeviceToHost, s) != hipSuccess ||
            hipStreamSynchronize(s) != hipSuccess)
          return TG_ERR_HIP;
        const float us = (float)(host_stamps[1] - host_stamps[0]) * 0.01f / iters;  // 100 MHz ticks
        if (best_us < 0.f || us < best_us) {
          best_us = us;
          best = c;
        }
      }
  }
  if (best_us < 0.f) return TG_ERR_UNSUPPORTED;  // no candidate ran and matched the reference

  tg_autotune_entry e;
  memset(&e, 0, sizeof(e));
  e.dtype = args->dtype;
  e.b_col_major = args->b_col_major;
  e.kind = kind;
  e.M = args->M;
  e.N = args->N;
  e.K = args->K;
  e.config = *tile_config(best.config_id);
  e.config.group_m = best.group_m;
  e.config.xcd_remap = best.xcd_remap;
  e.config.b_col_major = args->b_col_major;
  e.us = best_us;
  e.candidates = tried;
  e.valid = valid;
  autotune_cache_put(e);
  *result = e;
  // leave the winner's result in C
  rc = tg_gemm_ex(&best, stream);
  if (rc != TG_OK) return rc;
  return hipStreamSynchronize(s) == hipSuccess ? TG_OK : TG_ERR_HIP;
}

}  // namespace
}  // namespace tg

extern "C" {

int tg_gemm_autotune(const tg_gemm_args* args, void* workspace, int64_t workspace_bytes, int iters,
                     tg_autotune_entry* result, void* stream) {
  int64_t need = 0;
  const int rc = autotune_check(args, iters, result, &need);
  if (rc != TG_OK) return rc;
  if (!workspace || workspace_bytes < need) return TG_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(workspace) & 255) != 0) return TG_ERR_MISALIGNED;
  return autotune_run(args, workspace, iters, result, stream);
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Allocation-free variant: the workspace is a fixed device array of this
// library, TG_AUTOTUNE_NOALLOC_MAX_BYTES long, which every GPU the library
// runs on holds until the process ends.  Host code never passes the array's
// name to a kernel or a copy (on the host it is only a stand-in): the first
// call on a device, with that device current, asks the runtime for the
// array's device address on that device and keeps it.
// ---------------------------------------------------------------------------
static __device__ __align__(256) unsigned char scratch[TG_AUTOTUNE_NOALLOC_MAX_BYTES];

namespace tg {
namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices];  // device address of `scratch` on each device, once looked up

// The current device's copy of the scratch array, or NULL (status in *rc).
void* scratch_address(int* rc) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
    *rc = TG_ERR_HIP;
    return nullptr;
  }
  if (dev >= kMaxDevices) {
    *rc = TG_ERR_UNSUPPORTED;
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
      *rc = TG_ERR_HIP;
      return nullptr;
    }
    g_scratch[dev] = p;
  }
  *rc = TG_OK;
  return g_scratch[dev];
}

}  // namespace
}  // namespace tg

extern "C" {

int tg_gemm_autotune_noalloc(const tg_gemm_args* args, int iters, tg_autotune_entry* result, void* stream) {
  int64_t need = 0;
  int rc = autotune_check(args, iters, result, &need);
  if (rc != TG_OK) return rc;
  if (need > (int64_t)TG_AUTOTUNE_NOALLOC_MAX_BYTES) return TG_ERR_UNSUPPORTED;
  void* ws = scratch_address(&rc);
  if (!ws) return rc;
  return autotune_run(args, ws, iters, result, stream);
}


}  // extern "C"
