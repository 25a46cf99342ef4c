// moe_forward_noalloc: the layer forward for callers that cannot allocate device memory (code
// under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).  The
// workspace moe_forward takes from the caller lives here in one static device array per GPU,
// so the call allocates nothing; it runs the same kernels as moe_forward.
#include <hip/hip_runtime.h>

#include <mutex>

#include "moe.h"
#include "moe_internal.h"

namespace {

// The forward's workspace for every call of this entry point on one GPU.  In host code the
// name `scratch` is only a host-side stand-in for the symbol: its device address comes from
// hipGetSymbolAddress, once per device, and only that address is ever passed to a kernel.
static __device__ __align__(256) unsigned char scratch[MOE_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices];   // device address of `scratch` on each device (null: not yet)

// Device address of this library's scratch array on the current device.
int scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MOE_EHIP;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MOE_EHIP;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return MOE_OK;
}

}  // namespace

extern "C" int moe_forward_noalloc(const moe_cfg* cfg, const void* x, const void* Wg,
                                   const float* bg, const void* W1, const void* W2,
                                   const float* u, void* y, float* aux_loss,
                                   const moe_meta* meta, void* stream) {
  size_t need = 0;
  int rc = moe_workspace_size(cfg, &need);
  if (rc) return rc;
  if (need > MOE_NOALLOC_SCRATCH_BYTES) return MOE_ESCRATCH;
  // every other host check of moe_forward first (a stand-in workspace address: nothing is
  // enqueued), so that a rejected call touches no HIP state
  rc = moe::forward_workspace(cfg, x, Wg, bg, W1, W2, u, y, aux_loss, meta,
                              reinterpret_cast<void*>(uintptr_t{256}),
                              MOE_NOALLOC_SCRATCH_BYTES, stream, true);
  if (rc) return rc;
  void* ws = nullptr;
  if (scratch_address(&ws)) return MOE_EHIP;
  return moe::forward_workspace(cfg, x, Wg, bg, W1, W2, u, y, aux_loss, meta, ws,
                                MOE_NOALLOC_SCRATCH_BYTES, stream, false);
}
