// Allocation-free decode entry point: topo_attn_decode with its workspace in a file-scope device
// array instead of a caller buffer, for callers that cannot allocate device memory (code under HIP
// graph capture, tight serving loops, harnesses that forbid hipMalloc). The kernels and their
// results are those of topo_attn_decode; only where the scratch lives differs.
//
// The array `scratch` exists once per GPU the library runs on and stays allocated until the
// process ends. In host code its name is only a host-side stand-in, never a device address: the
// device address is looked up once per device with hipGetSymbolAddress (with that device current)
// and kept in `g_scratch`; every use below goes through that pointer.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/topo_attn.h"

namespace {

static __device__ __align__(256) unsigned char scratch[TOPO_NOALLOC_MAX_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_lock;
void* g_scratch[kMaxDevices] = {};

// Device address of the current device's `scratch`, looked up on the first call on that device.
// Returns nullptr if the lookup fails.
void* device_scratch() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> hold(g_lock);
  if (!g_scratch[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
    g_scratch[dev] = ptr;
  }
  return g_scratch[dev];
}

}  // namespace

extern "C" int topo_attn_decode_noalloc(const topo_params_t* p, const void* q, const void* k, const void* v,
                                        float* out, int32_t* sel_idx, int32_t* sel_count, hipStream_t stream) {
  // Parameters are checked first (no device call on an invalid argument): topo_attn_decode
  // returns their error before it looks at the workspace.
  const size_t need = topo_workspace_bytes(p, TOPO_OP_DECODE);
  if (need == 0) return topo_attn_decode(p, q, k, v, out, sel_idx, sel_count, nullptr, 0, stream);
  if (need > (size_t)TOPO_NOALLOC_MAX_BYTES) return TOPO_ESCRATCH;
  void* ws = device_scratch();
  if (!ws) return TOPO_EHIP;
  return topo_attn_decode(p, q, k, v, out, sel_idx, sel_count, ws, (size_t)TOPO_NOALLOC_MAX_BYTES, stream);
}
