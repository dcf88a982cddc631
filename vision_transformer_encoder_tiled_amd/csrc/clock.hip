// Core-clock probe for the measurements.  The published bf16 peak assumes
// the 2.4 GHz peak engine clock; under MFMA load the clock is lower, so the
// benchmark also reports each roofline fraction against the clock measured
// while the kernel runs.  One wavefront reads the shader-clock counter
// (s_memtime, one tick per core clock) and the constant-rate real-time
// counter (s_memrealtime), waits until the real-time counter has advanced by
// `ticks` (it always advances, so the wait ends), and reads both again.
// Launched on a second stream beside a busy kernel, clock ticks / real-time
// ticks x the real-time rate is the core clock under that load.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "vt_kernels.h"

namespace vt {

__global__ void __launch_bounds__(64) clock_probe_kernel(uint64_t ticks, unsigned long long* out) {
  const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
  const uint64_t c0 = __builtin_amdgcn_s_memtime();
  uint64_t r1 = r0;
  while (r1 - r0 < ticks) {
    __builtin_amdgcn_s_sleep(8);
    r1 = __builtin_amdgcn_s_memrealtime();
  }
  const uint64_t c1 = __builtin_amdgcn_s_memtime();
  r1 = __builtin_amdgcn_s_memrealtime();
  if (threadIdx.x == 0) {
    out[0] = c0;
    out[1] = c1;
    out[2] = r0;
    out[3] = r1;
  }
}

hipError_t launch_clock_probe(uint64_t ticks, unsigned long long* out, hipStream_t s) {
  hipLaunchKernelGGL(clock_probe_kernel, dim3(1), dim3(64), 0, s, ticks, out);
  return hipGetLastError();
}

}  // namespace vt
