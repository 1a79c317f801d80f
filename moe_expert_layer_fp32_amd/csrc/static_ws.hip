// moe_layer_static: the whole layer with the library's own device scratch
// instead of a caller workspace, for callers that cannot allocate (code under
// stream capture that must not call hipMalloc, tight serving loops, hosts
// that forbid allocation).
//
// The scratch is one file-scope device array of MOE_STATIC_WORKSPACE_BYTES,
// held by every device the library runs on until the process ends. Host code
// never passes the array's name to a kernel (on the host it is only a
// stand-in symbol): the first call on a device, with that device current,
// asks the runtime for the array's device address on that device and keeps
// it; every later call on the device uses that address. The call itself
// allocates nothing; it is moe_layer with that address as the workspace.
//
// moe_layer needs no zeroed workspace (every region it reads is written
// earlier in the same call), so nothing is cleared between calls. Calls that
// overlap on one device (two host threads, or two streams running at once)
// share the one array and race; calls on different devices do not.
#include <hip/hip_runtime.h>

#include <mutex>

#include "moe.h"

static __device__ __align__(256) unsigned char scratch[MOE_STATIC_WORKSPACE_BYTES];

namespace {

constexpr int MAX_DEVICES = 64;
std::mutex g_mutex;
void* g_scratch[MAX_DEVICES] = {};

// Device address of the scratch array on the current device (looked up once
// per device). Returns MOE_OK and sets *out, or MOE_ERR_HIP.
moe_status device_scratch(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES) return MOE_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_mutex);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MOE_ERR_HIP;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return MOE_OK;
}

}  // namespace

extern "C" moe_status moe_layer_static(const moe_desc* desc, const moe_weights* w, const void* x, void* y,
                                       moe_aux* aux, void* stream) {
  // Checks first, before any HIP call: moe_workspace_bytes is 0 only for an
  // invalid descriptor, which moe_layer rejects with its own status; a layer
  // whose workspace exceeds the array is refused.
  const size_t need = moe_workspace_bytes(desc, MOE_OP_LAYER);
  if (need == 0) return moe_layer(desc, w, x, y, aux, nullptr, 0, stream);
  if (need > MOE_STATIC_WORKSPACE_BYTES) return MOE_ERR_WORKSPACE;
  void* ws = nullptr;
  const moe_status st = device_scratch(&ws);
  if (st != MOE_OK) return st;
  return moe_layer(desc, w, x, y, aux, ws, MOE_STATIC_WORKSPACE_BYTES, stream);
}
