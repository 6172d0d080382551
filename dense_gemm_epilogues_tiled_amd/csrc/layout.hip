// layout.hip -- measurement aid: the register layouts the GEMM and attention
// kernels rely on, read back from the hardware so that a test can pin them.
//
// The kernels feed v_mfma_f32_16x16x32_{f16,bf16} with operand fragments
// whose lane layout (device.hpp, mfma16x16x32) is taken as: lane l holds
// row (A) / column (B) l % 16 and 8 k values of k-group l / 16, in the same
// k order for both operands; the accumulator lane l holds column l % 16 and
// rows 4 (l / 16) + r, r = 0..3.  Row-major B is read with the transposing
// ds_read_b64_tr_b16 (device.hpp, lds_read_tr8).  The probes below run those
// instructions on known data and write what every lane received; they take
// no input and depend on no other kernel.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/tg.h"
#include "device.hpp"

namespace tg {
namespace {

// The code of B element (lane lb, element eb), v = 8 lb + eb: distinct for
// every v and exact in the operand type -- v + 1 in fp16; (16 + v % 16) x
// 2^(v / 16) in bf16, whose 8-bit significand cannot hold 1 .. 512.
__device__ __forceinline__ float b_code(F16, int v) { return (float)(v + 1); }
__device__ __forceinline__ float b_code(BF16, int v) { return (float)(16 + (v & 15)) * (float)(1u << (v >> 4)); }

// One wave.  For every A position (lane la, element ea) in turn: A is one-hot
// (1 there, 0 elsewhere), B element (lb, eb) holds b_code(8 lb + eb), the
// accumulator starts at zero, and the 4 accumulator registers of every lane
// are written to out[((la * 8 + ea) * 64 + lane) * 4 + r].  With the layout
// above the only non-zero outputs are row la % 16, i.e. register
// r = la % 4 of lanes 16 (la % 16 / 4) + j, j = 0..15, each equal to the code
// of B lane j + 16 (la / 16), element ea.
template <class DT>
__global__ __launch_bounds__(64) void mfma_layout_kernel(float* out) {
  const int lane = threadIdx.x;
  u32x4 b;
#pragma unroll
  for (int h = 0; h < 4; ++h)
    b[h] = pack2(DT{}, b_code(DT{}, 8 * lane + 2 * h), b_code(DT{}, 8 * lane + 2 * h + 1));
  for (int pos = 0; pos < 64 * 8; ++pos) {
    const int la = pos >> 3, ea = pos & 7;
    u32x4 a = {0u, 0u, 0u, 0u};
    if (lane == la) {
#pragma unroll
      for (int h = 0; h < 4; ++h)
        a[h] = pack2(DT{}, ea == 2 * h ? 1.0f : 0.0f, ea == 2 * h + 1 ? 1.0f : 0.0f);
    }
    const f32x4 d = mfma16x16x32(DT{}, a, b, f32x4{0.f, 0.f, 0.f, 0.f});
    float* o = out + ((size_t)pos * 64 + lane) * 4;
#pragma unroll
    for (int r = 0; r < 4; ++r) o[r] = d[r];
  }
}

// One wave.  LDS holds the 16-bit values 0 .. 2047 in order; lane j supplies
// the byte address 8 j (four consecutive values each, 512 bytes in all) to
// one ds_read_b64_tr_b16, and out[4 lane + i] receives element i of what the
// lane got.
__global__ __launch_bounds__(64) void tr_read_layout_kernel(uint32_t* out) {
  __shared__ __attribute__((aligned(16))) uint16_t lds[2048];
  const int lane = threadIdx.x;
  for (int i = lane; i < 2048; i += 64) lds[i] = (uint16_t)i;
  __syncthreads();
  const u32x2 v = lds_read_tr8(reinterpret_cast<const unsigned char*>(lds), 8 * lane);
  out[4 * lane + 0] = v.x & 0xffffu;
  out[4 * lane + 1] = v.x >> 16;
  out[4 * lane + 2] = v.y & 0xffffu;
  out[4 * lane + 3] = v.y >> 16;
}

}  // namespace
}  // namespace tg

using namespace tg;

extern "C" int tg_layout_probe(int kind, void* out, void* stream) {
  if (!out || kind < 0 || kind > 2) return TG_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(out) & 15) != 0) return TG_ERR_MISALIGNED;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (kind == 0)
    hipLaunchKernelGGL(mfma_layout_kernel<F16>, dim3(1), dim3(64), 0, s, static_cast<float*>(out));
  else if (kind == 1)
    hipLaunchKernelGGL(mfma_layout_kernel<BF16>, dim3(1), dim3(64), 0, s, static_cast<float*>(out));
  else
    hipLaunchKernelGGL(tr_read_layout_kernel, dim3(1), dim3(64), 0, s, static_cast<uint32_t*>(out));
  return hipGetLastError() == hipSuccess ? TG_OK : TG_ERR_HIP;
}
