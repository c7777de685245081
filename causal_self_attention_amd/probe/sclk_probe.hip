// Shader-clock probe for the benchmark (not part of the attention library).
//
// One wave spins until the 100 MHz real-time counter (s_memrealtime) has
// advanced by a given number of ticks, and reports how many shader-clock
// cycles (s_memtime) passed meanwhile: their ratio times 100 MHz is the
// clock of the CU the wave ran on, averaged over the span. Launched on its
// own stream beside the timed steps, it measures the clock those steps ran
// at while taking one wave slot of one CU. The wait ends by real time, so
// the kernel always finishes.
#include <hip/hip_runtime.h>

#include <stdint.h>

namespace {

__global__ __launch_bounds__(64) void sclk_probe_kernel(unsigned long long* out,
                                                        unsigned long long ticks) {
  const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
  const unsigned long long c0 = __builtin_amdgcn_s_memtime();
  unsigned long long r = r0;
  while (r - r0 < ticks) {
    __builtin_amdgcn_s_sleep(1);
    r = __builtin_amdgcn_s_memrealtime();
  }
  const unsigned long long c1 = __builtin_amdgcn_s_memtime();
  // Lanes 0 and 1 write the two counts (a per-lane vector store).
  if (threadIdx.x < 2) out[threadIdx.x] = threadIdx.x == 0 ? c1 - c0 : r - r0;
}

}  // namespace

// Enqueue the probe on `stream`: out (device, 2 x uint64) receives the
// shader cycles and the 100 MHz ticks of the span. Returns 0, or the HIP
// error of the launch.
extern "C" int sclk_probe_launch(unsigned long long* out, unsigned long long ticks,
                                 void* stream) {
  hipLaunchKernelGGL(sclk_probe_kernel, dim3(1), dim3(64), 0,
                     static_cast<hipStream_t>(stream), out, ticks);
  return (int)hipGetLastError();
}
