// retention_chunkwise_fwd_noalloc: the chunkwise forward with its workspace in
// a static device array of the library instead of caller memory, for callers
// that cannot allocate device memory (code under HIP graph capture, tight
// serving loops, harnesses that forbid hipMalloc).  It shares the validation,
// kernel choice and kernels of retention_chunkwise_fwd; only the workspace
// pointer differs.  Nothing here allocates.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <mutex>

#include "abi_internal.h"
#include "libretention.h"

namespace {

constexpr size_t kScratchBytes = RET_NOALLOC_SCRATCH_BYTES;

// The workspace of segmented calls.  Each GPU the library runs on holds its
// own copy until the process ends.  In host code `scratch` is a host-side
// stand-in, not a device address: kernels get the address that
// hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices];  // device address of `scratch` per device, found on first use

// Address of this device's copy of `scratch`; looked up once per device, with
// that device current.
hipError_t device_scratch(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_scratch[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return hipSuccess;
}

}  // namespace

extern "C" ret_status retention_chunkwise_fwd_noalloc(const void* q, const void* k, const void* v,
                                                      const float* gamma, const float* state_in, float* state_out,
                                                      void* y, int B, int H, int T, int dk, int dv, int C,
                                                      ret_dtype dt, void* stream) {
  const ret::ChunkwiseFwdArgs a{q, k, v, gamma, state_in, state_out, y, B, H, T, dk, dv, C, static_cast<int>(dt)};
  ret_status st = ret::chunkwise_fwd_check(a, nullptr, 0, false, "retention_chunkwise_fwd_noalloc");
  if (st != RET_OK) return st;
  const size_t need = retention_chunkwise_workspace_bytes(B, H, T, dk, dv, C, dt);
  char msg[256];
  if (need > kScratchBytes) {
    std::snprintf(msg, sizeof(msg),
                  "retention_chunkwise_fwd_noalloc: this call needs %zu bytes of workspace, more than the %zu bytes "
                  "of static scratch (use retention_chunkwise_fwd with a workspace)",
                  need, kScratchBytes);
    ret::set_last_error(msg);
    return RET_ERR_UNSUPPORTED;
  }
  void* ws = nullptr;
  if (need > 0) {
    const hipError_t e = device_scratch(&ws);
    if (e != hipSuccess) {
      std::snprintf(msg, sizeof(msg), "retention_chunkwise_fwd_noalloc: scratch address lookup: HIP error %d (%s)",
                    static_cast<int>(e), hipGetErrorString(e));
      ret::set_last_error(msg);
      return RET_ERR_HIP;
    }
  }
  return ret::chunkwise_fwd_run(a, ws, stream);
}
