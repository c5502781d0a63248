// The Mamba-2 SSD scan for callers that cannot allocate device memory (code under
// HIP graph capture, serving loops, harnesses that forbid hipMalloc): the segment
// states that ssm_ssd_scan_fwd keeps in the caller's workspace live here in a
// file-scope device array instead, one copy per GPU, held until the process ends.
//
// In host code `scratch` names a host-side stand-in, not device memory: its device
// address on each GPU is obtained once per device with hipGetSymbolAddress (with that
// device current) and only that address is ever passed to kernels.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/ssm.h"
#include "kernels.hpp"

namespace {

constexpr size_t kScratchBytes = size_t(64) << 20;    // SSM_SSD_NOALLOC_SCRATCH_BYTES
static_assert(kScratchBytes == SSM_SSD_NOALLOC_SCRATCH_BYTES, "header and library agree on the scratch size");

__device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};                 // device address of `scratch`, per device

// The current device's address of `scratch`, looked up on the first call on that
// device; nullptr with *err set when the lookup fails.
void* scratch_on_current_device(hipError_t* err) {
  int dev = -1;
  *err = hipGetDevice(&dev);
  if (*err != hipSuccess) return nullptr;
  if (dev < 0 || dev >= kMaxDevices) {
    *err = hipErrorInvalidDevice;
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    *err = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (*err != hipSuccess || !ptr) {
      if (*err == hipSuccess) *err = hipErrorInvalidSymbol;
      return nullptr;
    }
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

ssm_status ssm_ssd_scan_fwd_noalloc(const void* x, const void* dt, const float* A, const void* Bm, const void* Cm,
                                    const float* Dskip, const float* dt_bias, int dt_softplus,
                                    const float* initial_state, void* y, float* final_state, int64_t batch,
                                    int64_t L, int64_t H, int64_t P, int64_t N, ssm_dtype dtype, void* stream) {
  ssm::SsdArgs a;
  ssm_status st = ssm::ssd_check(x, dt, A, Bm, Cm, Dskip, dt_bias, dt_softplus, initial_state, y, final_state, batch,
                                 L, H, P, N, dtype, nullptr, 0, &a);
  if (st != SSM_OK) return st;
  const size_t need = ssm_ssd_scan_workspace_size(batch, L, H, P, N, dtype);
  if (need > kScratchBytes) return SSM_ERR_TOO_LARGE;
  if (batch == 0 || H == 0) return SSM_OK;
  if (need == 0) return ssm::ssd_run(a, nullptr, 0, stream);   // one segment per sequence: no scratch
  hipError_t he = hipSuccess;
  void* ptr = scratch_on_current_device(&he);
  if (!ptr) {
    (void)hipGetLastError();
    return SSM_ERR_HIP;
  }
  return ssm::ssd_run(a, ptr, need, stream);
}

}  // extern "C"
