// Forward of the deformable convolution layer for callers that cannot
// allocate device memory (code under HIP graph capture, tight serving loops,
// harnesses that forbid hipMalloc): the scratch that deft_forward takes from
// the caller's workspace (re-laid weights, channel-minor copy of x, deformed
// columns) lives instead in a fixed device array of this library.
//
// The array's name is only a host-side stand-in in host code: its device
// address is looked up once per device with hipGetSymbolAddress and that
// pointer is what the kernels receive.  Nothing here allocates.
#include <hip/hip_runtime.h>

#include <mutex>

#include "deft.h"
#include "deft_internal.h"

namespace {

constexpr size_t kScratchBytes = DEFT_NOALLOC_SCRATCH_BYTES;
static_assert(kScratchBytes % 256 == 0, "scratch size");

// One copy per GPU, held until the process ends.
__device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
struct DeviceScratch {
  std::once_flag once;
  void* ptr = nullptr;
  hipError_t err = hipSuccess;
};
DeviceScratch g_dev[kMaxDevices];

// Device address of this device's scratch (looked up on the first call made
// with that device current).
hipError_t scratch_ptr(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  DeviceScratch& s = g_dev[dev];
  std::call_once(s.once, [&s]() {
    void* p = nullptr;
    s.err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (s.err == hipSuccess && p == nullptr) s.err = hipErrorInvalidSymbol;
    if (s.err == hipSuccess) s.ptr = p;
  });
  if (s.err != hipSuccess) return s.err;
  *out = s.ptr;
  return hipSuccess;
}

}  // namespace

extern "C" int deft_forward_noalloc(const deft_plan* p, const void* x, const void* w_off, const void* b_off,
                                    const void* w, const void* b, void* y, float* offsets_out, void* stream) {
  if (!p) return DEFT_ERR_NULLPTR;
  if (p->d.n == 0) return DEFT_OK;  // empty batch: nothing is read or written
  if (p->ws_fwd_end > kScratchBytes) return DEFT_ERR_SCRATCH;
  void* ws = nullptr;
  const hipError_t e = scratch_ptr(&ws);
  if (e != hipSuccess) return deft::report_hip_error(e);
  // every scratch byte the forward reads it has written earlier in the same
  // call, so the previous call's contents need no clearing
  return deft_forward(p, x, w_off, b_off, w, b, y, offsets_out, ws, kScratchBytes, stream);
}
