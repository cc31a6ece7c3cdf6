// Shader-clock probe, a measurement aid: the chip lowers its clock under a
// heavy load (power), so a kernel's time alone does not say how busy its
// units were.  One wavefront, launched on its own stream beside the work to be
// measured, reads the shader-clock counter and the fixed-rate counter, sleeps
// until the fixed-rate counter has advanced by the requested span, and reads
// both again: the ratio of the two differences, times the fixed rate, is the
// clock the chip ran at meanwhile.  The wave holds a few registers and no LDS,
// so it takes nothing from the work beside it.
#include <hip/hip_runtime.h>

#include "launch.h"

namespace sla {

__global__ __launch_bounds__(64) void clock_probe_kernel(int64_t* __restrict__ out, uint64_t ticks,
                                                         uint32_t max_iter) {
  const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
  const uint64_t c0 = __builtin_amdgcn_s_memtime();
  uint64_t r1 = r0;
  // bounded twice: by the fixed-rate span and by an iteration count
  for (uint32_t it = 0; r1 - r0 < ticks && it < max_iter; ++it) {
    __builtin_amdgcn_s_sleep(4);
    r1 = __builtin_amdgcn_s_memrealtime();
  }
  const uint64_t c1 = __builtin_amdgcn_s_memtime();
  if (threadIdx.x == 0) {
    out[0] = (int64_t)c0;
    out[1] = (int64_t)c1;
    out[2] = (int64_t)r0;
    out[3] = (int64_t)r1;
  }
}

hipError_t launch_clock_probe(int64_t* out, uint64_t ticks, uint32_t max_iter, hipStream_t s) {
  clock_probe_kernel<<<dim3(1), 64, 0, s>>>(out, ticks, max_iter);
  return hipGetLastError();
}

}  // namespace sla
