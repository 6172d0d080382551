// phases.hpp -- phase stamps for profiling builds.
//
// Compiled in only with -DTG_PHASE_STAMPS (dense_gemm_epilogues_tiled_amd/phases.py
// builds such a library beside the product one); in the product build every
// macro below expands to nothing.  An instrumented kernel reads the GPU's
// constant 100 MHz clock (s_memrealtime, identical on every XCD) at named
// points of its schedule -- a stamp only reads a counter, it changes no work
// -- and thread 0 of each workgroup writes its stamps, with vector stores,
// to a per-source-file device array at the end.  The host reads the array of
// the last launch with tg_phases_<file>(), a function only profiling builds
// export.  Stamps are those of wave 0 of each workgroup.
#pragma once

#include <hip/hip_runtime.h>

#ifdef TG_PHASE_STAMPS

namespace tg {
constexpr int kPhaseSlots = 8;            // stamps per workgroup
constexpr int kPhaseMaxGroups = 1 << 16;  // workgroups recorded per launch
}  // namespace tg

// One stamp array per source file, and its host reader:
//   int tg_phases_<name>(unsigned long long* host, int groups)
// copies groups x kPhaseSlots stamps (workgroup-major) into host memory.
#define TG_PHASE_BUFFER(name)                                                                            \
  static __device__ unsigned long long name##_phase_buf[tg::kPhaseMaxGroups * tg::kPhaseSlots];        \
  extern "C" int tg_phases_##name(unsigned long long* host, int groups) {                               \
    if (!host || groups <= 0 || groups > tg::kPhaseMaxGroups) return -1;                                \
    return (int)hipMemcpyFromSymbol(host, HIP_SYMBOL(name##_phase_buf),                                  \
                                    sizeof(unsigned long long) * tg::kPhaseSlots * groups, 0,            \
                                    hipMemcpyDeviceToHost);                                              \
  }
#define TG_PHASE_DECL unsigned long long tg_phase_t_[tg::kPhaseSlots] = {0, 0, 0, 0, 0, 0, 0, 0}
#define TG_PHASE(i) (tg_phase_t_[(i)] = __builtin_amdgcn_s_memrealtime())
// wait for this wave's outstanding stores, then stamp (the last phase of a kernel)
#define TG_PHASE_DRAINED(i)                                   \
  do {                                                        \
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");          \
    TG_PHASE(i);                                              \
  } while (0)
#define TG_PHASE_WRITE(name)                                                                  \
  do {                                                                                        \
    if (threadIdx.x == 0 && blockIdx.x < (unsigned)tg::kPhaseMaxGroups) {                     \
      _Pragma("unroll") for (int tg_i_ = 0; tg_i_ < tg::kPhaseSlots; ++tg_i_)                 \
          name##_phase_buf[blockIdx.x * tg::kPhaseSlots + tg_i_] = tg_phase_t_[tg_i_];        \
    }                                                                                         \
  } while (0)

#else

#define TG_PHASE_BUFFER(name)
#define TG_PHASE_DECL
#define TG_PHASE(i) ((void)0)
#define TG_PHASE_DRAINED(i) ((void)0)
#define TG_PHASE_WRITE(name) ((void)0)

#endif
