// noalloc.hip -- coli_moe_forward_noalloc: the layer forward with its
// workspace in a static device array, for callers that cannot allocate
// (code under stream capture, serving loops, harnesses that forbid hipMalloc).
//
// The array `scratch` lives in this library's code object: every GPU the
// library runs on holds its own copy, allocated when the code object is loaded
// on that device and kept until the process ends.  In host code the name is a
// host-side stand-in, not a device address; the device address is looked up
// once per device with hipGetSymbolAddress, with that device current, and only
// that address is handed to the kernels.
#include <hip/hip_runtime.h>

#include <mutex>

#include "coli.h"
#include "kernels.h"

namespace {

__device__ __attribute__((aligned(256))) uint8_t scratch[COLI_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void *g_scratch[kMaxDevices];  // device address of `scratch` on each device (host copy)

// The scratch array's device address on the current device (looked up on the
// first call made on that device).
int scratch_address(void **out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return COLI_EDEVICE;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch[dev]) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return COLI_EDEVICE;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return COLI_OK;
}

}  // namespace

extern "C" int coli_moe_forward_noalloc(const coli_moe_layer *L, coli_mode mode, const void *x,
                                        int T, void *y, int32_t *topk_idx_out,
                                        float *topk_gate_out, int32_t *status, void *stream) {
  // argument errors first, exactly as coli_moe_forward reports them, then the
  // size limit; nothing touches the device before both pass
  size_t need = 0;
  const int chk = coli::forward_arg_check(L, mode, x, T, y, topk_idx_out, topk_gate_out, status,
                                          &need);
  if (chk != COLI_OK) return chk;
  if (need > size_t(COLI_NOALLOC_SCRATCH_BYTES)) return COLI_ESCRATCH;
  if (T == 0) return COLI_OK;
  void *ws = nullptr;
  const int rc = scratch_address(&ws);
  if (rc != COLI_OK) return rc;
  return coli_moe_forward(L, mode, x, T, y, topk_idx_out, topk_gate_out, status, ws,
                          size_t(COLI_NOALLOC_SCRATCH_BYTES), stream);
}
