// Static device scratch for the allocation-free backward (attn_bwd_noalloc).
//
// The backward's workspace (the FP32 delta row vector and, in the FP32-output
// mode, the BF16 copy of dO) lives here in a file-scope device array instead
// of caller memory, for callers that cannot allocate.  Each GPU the library
// runs on holds its own copy of the array until the process ends.  Host code
// never passes the array's name to a kernel (on the host it only stands for
// the symbol): the device address comes from hipGetSymbolAddress, looked up
// once per device with that device current, and kept per device.
#include <mutex>

#include "pfa_attn.h"
#include "pfa_internal.h"

namespace pfa {

namespace {

__device__ __align__(256) char scratch[kNoallocScratchBytes];

constexpr int kMaxDevices = 64;
void* g_scratch[kMaxDevices];
hipError_t g_status[kMaxDevices];
std::once_flag g_once[kMaxDevices];

}  // namespace

int noalloc_scratch(void* stream, void** ptr) {
  *ptr = nullptr;
  int dev = 0;
  if (stream) {
    if (hipStreamGetDevice(static_cast<hipStream_t>(stream), &dev) != hipSuccess) return PFA_ERR_HIP;
  } else if (hipGetDevice(&dev) != hipSuccess) {
    return PFA_ERR_HIP;
  }
  if (dev < 0 || dev >= kMaxDevices) return PFA_ERR_UNSUPPORTED;
  std::call_once(g_once[dev], [dev] {
    int cur = 0;
    hipError_t e = hipGetDevice(&cur);
    if (e == hipSuccess && cur != dev) e = hipSetDevice(dev);
    void* p = nullptr;
    if (e == hipSuccess) e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev) {
      const hipError_t r = hipSetDevice(cur);
      if (e == hipSuccess) e = r;
    }
    g_status[dev] = e;
    g_scratch[dev] = e == hipSuccess ? p : nullptr;
  });
  if (g_status[dev] != hipSuccess || !g_scratch[dev]) return PFA_ERR_HIP;
  *ptr = g_scratch[dev];
  return PFA_OK;
}

}  // namespace pfa
