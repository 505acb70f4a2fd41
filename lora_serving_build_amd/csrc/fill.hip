// Zero fill of a 16-byte-aligned buffer with vector stores (used for the
// shrink workspace; a kernel rather than a memset node so that captured
// graphs replay it reliably).
#include "lora_device.h"
#include "lora_kernels.h"

namespace lora {

namespace {

__global__ __launch_bounds__(256) void fill_zero_kernel(u32x4* p, size_t n16) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride)
    p[i] = u32x4{0u, 0u, 0u, 0u};
}

}  // namespace

hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t s) {
  const size_t n16 = bytes / 16;
  size_t blocks = (n16 + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)blocks), dim3(256), 0, s,
                     static_cast<u32x4*>(p), n16);
  return hipGetLastError();
}

}  // namespace lora
