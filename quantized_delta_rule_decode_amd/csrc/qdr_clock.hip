// qdr_clock.hip -- shader-clock probe (diagnostic, not part of the decode
// step).  One wave runs independent fma chains between two reads of the
// shader-clock counter (s_memtime) and of the constant 100 MHz counter
// (s_memrealtime); their ratio is the shader clock while the probe ran, so a
// probe launched on a second stream during decode steps measures the clock
// the step runs at (a VALU-bound kernel's time scales with it).
#include "../../include/qdr.h"

#include <hip/hip_runtime.h>

namespace {

__global__ void __launch_bounds__(64) k_clock_probe(uint64_t *out, int32_t iters) {
  float a0 = 1.0f + (float)threadIdx.x, a1 = a0 + 1.0f, a2 = a0 + 2.0f, a3 = a0 + 3.0f;
  const uint64_t t0 = __builtin_amdgcn_s_memtime();
  const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
  for (int32_t i = 0; i < iters; ++i) {
#pragma unroll
    for (int j = 0; j < 64; ++j) {
      a0 = __builtin_fmaf(a0, 0.999f, 0.5f);
      a1 = __builtin_fmaf(a1, 0.999f, 0.5f);
      a2 = __builtin_fmaf(a2, 0.999f, 0.5f);
      a3 = __builtin_fmaf(a3, 0.999f, 0.5f);
    }
  }
  const uint64_t t1 = __builtin_amdgcn_s_memtime();
  const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
  if (threadIdx.x == 0) {
    out[0] = t0;
    out[1] = r0;
    out[2] = t1;
    out[3] = r1;
    out[4] = (uint64_t)__float_as_uint(a0 + a1 + a2 + a3);   // keeps the chains
  }
}

}  // namespace

extern "C" qdr_status qdr_clock_probe(uint64_t *out, int32_t iters, void *stream) {
  if (!out || iters <= 0) return QDR_E_INVAL;
  hipLaunchKernelGGL(k_clock_probe, dim3(1), dim3(64), 0, (hipStream_t)stream, out, iters);
  return hipGetLastError() == hipSuccess ? QDR_OK : QDR_E_DEVICE;
}
