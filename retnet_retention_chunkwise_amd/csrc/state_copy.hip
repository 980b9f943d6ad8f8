// state_out <- state_in (or zeros): the carried state of an empty sequence.
// A plain fill/copy kernel (no hipMemsetAsync/hipMemcpyAsync node), so the
// call can also sit inside a captured HIP graph.
#include "common.h"
#include "kernels.h"

namespace ret {
namespace {
__global__ __launch_bounds__(256) void state_copy_kernel(const float* __restrict__ src, float* __restrict__ dst,
                                                         size_t n) {
  for (size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
       i += static_cast<size_t>(gridDim.x) * blockDim.x)
    dst[i] = src != nullptr ? src[i] : 0.0f;
}
}  // namespace

hipError_t launch_state_copy(const float* state_in, float* state_out, size_t n, hipStream_t s) {
  size_t blocks = (n + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(state_copy_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, state_in, state_out, n);
  return hipGetLastError();
}
}  // namespace ret
