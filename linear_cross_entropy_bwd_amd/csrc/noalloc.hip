// flce_fwd_noalloc: the forward (loss and per-row LSE) in a fixed scratch area
// of device memory, so that a call allocates nothing.  The area is a
// file-scope device array, one copy per device, held until the process ends;
// host code reaches it only through the address hipGetSymbolAddress returns
// for the current device (the array's name is a host-side stand-in).
#include <hip/hip_runtime.h>

#include <mutex>

#include "flce.h"
#include "flce_internal.h"

namespace flce {
namespace {

constexpr size_t kScratchBytes = FLCE_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

// The current device's address of `scratch`, looked up once per device.
int scratch_address(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return FLCE_ERR_HIP;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) {
      (void)hipGetLastError();
      return FLCE_ERR_HIP;
    }
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return FLCE_OK;
}

}  // namespace
}  // namespace flce

extern "C" int flce_fwd_noalloc(const void* h, const void* w, const int64_t* labels, int64_t n, int64_t d, int64_t v,
                                flce_dtype dtype, int64_t ignore_index, flce_reduction reduction, float* loss_out,
                                float* lse_out, hipStream_t stream) {
  void* ws = nullptr;
  const int st = flce::scratch_address(&ws);
  if (st != FLCE_OK) return st;
  return flce::fwd_in_workspace(h, w, labels, n, d, v, dtype, ignore_index, reduction, loss_out, lse_out, ws,
                                flce::kScratchBytes, stream);
}
