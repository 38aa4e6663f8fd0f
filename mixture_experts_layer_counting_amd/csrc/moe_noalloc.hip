// moe_forward_noalloc: the whole forward of moe_forward with its workspace
// in a library-owned device array instead of a caller buffer, for callers
// that cannot allocate device memory (code under HIP graph capture, tight
// serving loops, harnesses that forbid hipMalloc).
//
// `scratch` is a file-scope device array, one copy per GPU the library runs
// on, held until the process ends.  Its name is only a host-side stand-in on
// the host, so the host never passes it anywhere: the first call on a device
// (with that device current) asks the runtime for the array's device address
// with hipGetSymbolAddress and keeps it per device; every later use on that
// device takes that address.  Nothing here allocates.
//
// The forward needs no zeroed workspace: every kernel writes what it later
// reads within the same call (the device-error word included), so the
// array's contents left by an earlier call never matter.  Calls that overlap
// on one device (other streams, other threads) share the one array and race.
#include <hip/hip_runtime.h>

#include <mutex>
#include <vector>

#include "../../include/moe_mi355x.h"

namespace {

static __device__ __align__(256) unsigned char scratch[MOE_NOALLOC_SCRATCH_BYTES];

// Device address of this device's `scratch`, looked up once per device.
int scratch_of_current_device(void** out) {
  static std::mutex mu;
  static std::vector<void*> addr;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
    (void)hipGetLastError();
    return MOE_E_DEVICE;
  }
  std::lock_guard<std::mutex> lock(mu);
  if (static_cast<size_t>(dev) >= addr.size()) addr.resize(dev + 1, nullptr);
  if (!addr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
      (void)hipGetLastError();
      return MOE_E_DEVICE;
    }
    addr[dev] = p;
  }
  *out = addr[dev];
  return MOE_OK;
}

}  // namespace

extern "C" int moe_forward_noalloc(const moe_dims* dims, const moe_weights* w, const uint16_t* x,
                                   moe_routes* routes, moe_saved* saved, float* out_f32,
                                   uint16_t* out_bf16, hipStream_t stream) {
  const size_t need = moe_workspace_bytes(dims, MOE_OP_FORWARD);
  if (need == 0) return dims ? MOE_E_SHAPE : MOE_E_NULL;
  if (need > MOE_NOALLOC_SCRATCH_BYTES) return MOE_E_WORKSPACE;
  if (dims->tokens == 0) return MOE_OK;
  void* ws = nullptr;
  const int st = scratch_of_current_device(&ws);
  if (st != MOE_OK) return st;
  return moe_forward(dims, w, x, routes, saved, out_f32, out_bf16, ws, MOE_NOALLOC_SCRATCH_BYTES, stream);
}
