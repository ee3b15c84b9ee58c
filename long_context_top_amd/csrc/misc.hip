// Small utility kernels.
#include "common.h"
#include "kernels.h"

namespace lct {

// Plain fill kernel used instead of hipMemsetAsync so that callers may
// capture it in a graph.
__global__ __launch_bounds__(256) void k_zero(uint8_t* __restrict__ p, size_t bytes) {
  const size_t n16 = bytes / 16;
  uintx4* p16 = reinterpret_cast<uintx4*>(p);
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += (size_t)gridDim.x * 256)
    p16[i] = uintx4{0u, 0u, 0u, 0u};
  if (blockIdx.x == 0)
    for (size_t i = n16 * 16 + threadIdx.x; i < bytes; i += 256) p[i] = 0;
}

hipError_t launch_zero(void* p, size_t bytes, hipStream_t st) {
  size_t blocks = (bytes / 16 + 255) / 256;
  if (blocks < 1) blocks = 1;
  if (blocks > 4096) blocks = 4096;
  k_zero<<<(unsigned)blocks, 256, 0, st>>>(reinterpret_cast<uint8_t*>(p), bytes);
  return hipGetLastError();
}

}  // namespace lct
