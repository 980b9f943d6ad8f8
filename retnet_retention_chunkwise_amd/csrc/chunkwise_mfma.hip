#include "common.h"
#include "kernels.h"
namespace ret {
bool chunkwise_mfma_supports(int, int, int, int, int) { return false; }
hipError_t launch_chunkwise_mfma(const void*, const void*, const void*, const float*, float*, void*, int, int, int,
                                 int, int, int, const HeadGroup&, hipStream_t) {
  return hipErrorNotSupported;
}
}  // namespace ret
