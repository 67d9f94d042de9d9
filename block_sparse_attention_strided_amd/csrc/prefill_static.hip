// xattn_prefill_chunk_static: the resident-K/V prefill with the library's
// scratch in a fixed per-device array instead of a caller workspace, for
// callers that cannot allocate device memory.
//
// The array is a file-scope __device__ variable: every GPU the library runs
// on holds its own copy, from the code object's load until the process ends.
// On the host its name is only a stand-in, never a device address; the
// address comes from hipGetSymbolAddress, once per device with that device
// current, and is kept per device.  Every call on one device shares that
// device's array (the previous call's contents stay in it); the prefill
// path itself clears the one piece of state that must start at zero (the
// attention's work counter, cleared by the selection or the plan kernel
// before the attention launch reads it).  Calls that overlap in time on one
// device race on the array.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include <mutex>

#include "../../include/xattn.h"
#include "xattn_internal.h"

namespace {

constexpr size_t kScratchBytes = (size_t)XATTN_STATIC_SCRATCH_BYTES;
static_assert(kScratchBytes % 256 == 0, "scratch size must keep the 256-byte workspace alignment");

__device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices];  // device address of `scratch` per device (nullptr: not looked up yet)

// Device address of the current device's scratch array; looked up on the
// first call on each device.  Returns nullptr on failure with *err set.
void* scratch_ptr(hipError_t* err) {
  int dev = -1;
  *err = hipGetDevice(&dev);
  if (*err != hipSuccess) return nullptr;
  if (dev < 0 || dev >= kMaxDevices) {
    *err = hipErrorInvalidDevice;
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    void* ptr = nullptr;
    *err = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (*err != hipSuccess) return nullptr;
    g_ptr[dev] = ptr;
  }
  return g_ptr[dev];
}

}  // namespace

extern "C" int xattn_prefill_chunk_static(const XattnShape* shape, const XattnParams* params, const void* q,
                                          const void* k, const void* v, void* out, float* lse, int32_t* counts,
                                          const XattnAux* aux, void* stream) {
  size_t need = 0;
  const int rc = xattn::workspace_bytes(shape, params, &need);  // validates shape and params
  if (rc) return rc;
  if (need > kScratchBytes)
    return xattn::fail_message(XATTN_ERR_UNSUPPORTED,
                               "this call needs %zu bytes of scratch; the static scratch holds %zu (use "
                               "xattn_prefill_chunk with a workspace)", need, kScratchBytes);
  hipError_t e = hipSuccess;
  void* ws = scratch_ptr(&e);
  if (!ws) return xattn::fail_message(XATTN_ERR_HIP, "static scratch address: %s", hipGetErrorString(e));
  if (((uintptr_t)ws) & 255)
    return xattn::fail_message(XATTN_ERR_HIP, "static scratch address %p is not 256-byte aligned", ws);
  return xattn_prefill_chunk(nullptr, shape, params, q, k, v, nullptr, nullptr, 0, out, lse, counts, aux, ws,
                             kScratchBytes, stream);
}
