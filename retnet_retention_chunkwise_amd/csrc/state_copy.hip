// state_out <- state_in (or zeros): the carried state of an empty sequence,
// and a 32-bit fill.  Plain kernels (no hipMemsetAsync/hipMemcpyAsync node),
// so the calls can also sit inside a captured HIP graph.
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

// n 32-bit words: 16-byte stores over the first n/4 groups, then the tail;
// thread 0 also sets one separate word (when word is not null)
__global__ __launch_bounds__(256) void fill_u32_kernel(unsigned int* __restrict__ p, size_t n, unsigned int val,
                                                       unsigned int* word, unsigned int word_val) {
  const size_t n4 = n / 4;
  const size_t stride = static_cast<size_t>(gridDim.x) * blockDim.x;
  const size_t i0 = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  typedef unsigned int u4 __attribute__((ext_vector_type(4)));
  for (size_t i = i0; i < n4; i += stride) reinterpret_cast<u4*>(p)[i] = u4{val, val, val, val};
  for (size_t i = 4 * n4 + i0; i < n; i += stride) p[i] = val;
  if (word != nullptr && i0 == 0) *word = word_val;
}
}  // namespace

hipError_t launch_fill_u32(void* p, size_t n, unsigned int val, hipStream_t s, unsigned int* word,
                           unsigned int word_val) {
  size_t blocks = (n / 4 + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  if (blocks == 0) blocks = 1;
  if (n == 0 && word == nullptr) return hipSuccess;
  hipLaunchKernelGGL(fill_u32_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s,
                     static_cast<unsigned int*>(p), n, val, word, word_val);
  return hipGetLastError();
}

hipError_t launch_state_copy(const float* state_in, float* state_out, size_t n, hipStream_t s) {
  size_t blocks = (n + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(state_copy_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, state_in, state_out, n);
  return hipGetLastError();
}
}  // namespace ret
