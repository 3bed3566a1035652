// nt_decode_layer_noalloc: the decode layer for callers that cannot allocate device memory
// (code under HIP graph capture, tight serving loops, harnesses that forbid allocation).
// Its workspace is a file-scope device array, one copy per device, instead of a caller
// buffer; everything else is nt_decode_layer.
#include <hip/hip_runtime.h>

#include <stdio.h>

#include <mutex>

#include "../../include/nt.h"
#include "errors.h"

// The workspace of every nt_decode_layer_noalloc call on a device (each device holds its own
// copy until the process ends).  Host code never passes this name to a kernel or a copy: on
// the host it is only a stand-in for the symbol, so its device address is looked up once per
// device and kept below.
__device__ __align__(256) unsigned char scratch[NT_NOALLOC_WS_BYTES];

namespace {

constexpr int MAX_DEVICES = 64;
std::mutex g_mu;
void* g_scratch[MAX_DEVICES];  // device address of `scratch` on each device, once looked up

// The device address of the current device's copy of `scratch`, looked up with that device
// current on the first call there.
int scratch_here(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return nt::set_error(NT_EHIP, "hipGetDevice failed");
  if (dev < 0 || dev >= MAX_DEVICES) return nt::set_error(NT_EINVAL, "device index out of range");
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      char msg[160];
      snprintf(msg, sizeof(msg), "hipGetSymbolAddress(scratch): %s (%d)", hipGetErrorString(e), (int)e);
      return nt::set_error(NT_EHIP, msg);
    }
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return NT_OK;
}

}  // namespace

extern "C" int nt_decode_layer_noalloc(const nt_layer_weights* w, const nt_layer_shape* shp, int pos, float* h,
                                       uint16_t* k_cache, uint16_t* v_cache, void* stream) {
  if (!shp) return nt::set_error(NT_EINVAL, "shape is null");
  const size_t need = nt_decode_layer_ws_bytes(shp);  // 0 for a shape nt_decode_layer rejects
  if (need > (size_t)NT_NOALLOC_WS_BYTES) {
    char msg[200];
    snprintf(msg, sizeof(msg), "layer workspace of %zu bytes exceeds the static %d bytes of nt_decode_layer_noalloc",
             need, NT_NOALLOC_WS_BYTES);
    return nt::set_error(NT_ESHAPE, msg);
  }
  void* ws = nullptr;
  const int rc = scratch_here(&ws);
  if (rc != NT_OK) return rc;
  return nt_decode_layer(w, shp, pos, h, k_cache, v_cache, ws, (size_t)NT_NOALLOC_WS_BYTES, stream);
}
