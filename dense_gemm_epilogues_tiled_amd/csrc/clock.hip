// clock.hip -- measurement aid: the shader clock the matrix units run at
// under sustained load with data-like operands.
//
// The dense MFMA peak of a gfx950 is 256 CUs x 4096 FLOP/clk x the shader
// clock; the published 2.5 PFLOP/s assumes 2.4 GHz, but sustained MFMA work
// runs the chip at a lower clock.  This kernel keeps every SIMD's matrix unit
// busy with independent MFMA chains for `iters` iterations and records, per
// workgroup, the elapsed shader-clock cycles (s_memtime) and the elapsed ticks
// of the constant 100 MHz counter (s_memrealtime) around the loop; their
// ratio is the clock under that load.

#include "device.hpp"
#include "kernels.hpp"

namespace tg {

__global__ __launch_bounds__(256) void clock_probe_kernel(unsigned long long* out, int iters) {
  // Operands change every iteration (a per-lane xorshift): the power drawn,
  // and so the clock, depends on how many operand bits toggle, and real GEMM
  // data toggles most of them.  Every operand is a finite fp16 value of
  // magnitude in [0.5, 1), sign random; accumulators stay finite.
  uint32_t x = 0x9e3779b9u ^ (blockIdx.x * 256u + threadIdx.x) * 0x85ebca6bu;
  f32x4 acc[4] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f},
                  f32x4{0.f, 0.f, 0.f, 0.f}};
  const unsigned long long t0 = __builtin_amdgcn_s_memtime();
  const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
  for (int i = 0; i < iters; ++i) {
    x ^= x << 13;
    x ^= x >> 17;
    x ^= x << 5;
    const uint32_t w = (x & 0x83ff83ffu) | 0x38003800u;  // two fp16 in +-[0.5, 1)
    const u32x4 a = u32x4{w, w ^ 0x00ff00ffu, w ^ 0x03300330u, w ^ 0x80008000u};
    const u32x4 b = u32x4{w ^ 0x80000000u, w ^ 0x01550155u, w, w ^ 0x02aa02aau};
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[j] = mfma16x16x32(F16{}, a, b, acc[j]);
  }
  // the counters are read after the last MFMA has retired
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j) s += acc[j][0] + acc[j][1] + acc[j][2] + acc[j][3];
  asm volatile("" : "+v"(s));
  const unsigned long long t1 = __builtin_amdgcn_s_memtime();
  const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
  if (threadIdx.x == 0) {
    out[2 * blockIdx.x] = t1 - t0;
    out[2 * blockIdx.x + 1] = (s != s ? 1ull : 0ull) + (r1 - r0);  // s is never NaN; keeps it live
  }
}

}  // namespace tg

using namespace tg;

extern "C" int tg_clock_probe(unsigned long long* out, int blocks, int iters, void* stream) {
  if (!out || blocks < 1 || blocks > 65536 || iters < 1 || iters > (1 << 24)) return TG_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(out) & 15u) != 0) return TG_ERR_MISALIGNED;
  hipLaunchKernelGGL(clock_probe_kernel, dim3(blocks), dim3(256), 0, static_cast<hipStream_t>(stream), out, iters);
  return hipGetLastError() == hipSuccess ? TG_OK : TG_ERR_HIP;
}
