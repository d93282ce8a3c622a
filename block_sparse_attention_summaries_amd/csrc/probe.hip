// probe.hip -- a measurement aid beside the attention path: the time of a
// chain of dependent device-memory loads.  One lane follows a cyclic list of
// indices, each load waiting for the one before, so the kernel's duration
// over `steps` loads is the round-trip latency of the memory level the list
// lives in (L2, the MALL or HBM, by the list's footprint).  A decode step is a
// short chain of such round trips, so this figure bounds it from below.
#include "spa_device.h"
#include "spa_launch.h"

namespace spa {

// `zero` is 0 at run time: it keeps the index per lane, so the loads take the
// vector memory path the attention kernels use.  Every index is masked to the
// power-of-two list length, so any list contents stay in bounds.
__global__ __launch_bounds__(64) void load_chase_kernel(const uint32_t* __restrict__ next, uint32_t mask,
                                                        int steps, uint32_t start, uint32_t zero,
                                                        uint32_t* __restrict__ out) {
  uint32_t i = (start + threadIdx.x * zero) & mask;
  for (int s = 0; s < steps; ++s) i = next[i] & mask;
  if (threadIdx.x == 0) out[0] = i;
}

hipError_t launch_load_chase(const uint32_t* next, uint32_t mask, int steps, uint32_t start, uint32_t* out,
                             hipStream_t st) {
  return launch(true, load_chase_kernel, dim3(1), dim3(1), st, next, mask, steps, start, 0u, out);
}

}  // namespace spa
