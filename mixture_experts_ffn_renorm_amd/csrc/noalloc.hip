// moe_forward_noalloc: moe_forward with its scratch memory in a device array
// of this library instead of a caller workspace, for callers that cannot
// allocate device memory.  The array is a file-scope __device__ object, so
// every GPU the library runs on holds its own copy (at its own address) from
// the first call on that device until the process ends.  Host code never
// uses the array's name as an address: the first call on a device looks up
// that device's address with hipGetSymbolAddress and keeps it.
#include <mutex>

#include "moe_common.h"
#include "moe_mi355x.h"

static __device__ __align__(256) uint8_t scratch[MOE_NOALLOC_SCRATCH_BYTES];

namespace {

std::mutex g_scratch_mu;
void* g_scratch_ptr[moe_host::kMaxDevices] = {};

// Device address of `scratch` on the current device (looked up once per
// device, with that device current).
hipError_t scratch_on_current_device(void** out) {
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  if (dev < 0 || dev >= moe_host::kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (err != hipSuccess) return err;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace

extern "C" int moe_forward_noalloc(const uint16_t* x, const uint16_t* w_router,
                                   const float* logit_bias, const uint16_t* w13,
                                   const uint16_t* w2, int M, int E, int top_k, int H, int I,
                                   int renormalize, uint16_t* out, int32_t* topk_ids_out,
                                   float* topk_weights_out, moe_dispatch_info* info,
                                   void* stream) {
  const size_t need = moe_workspace_size(M, E, top_k, H, I);
  if (need == 0) {
    // unsupported sizes: moe_forward reports which error (nothing launched)
    return moe_forward(x, w_router, logit_bias, w13, w2, M, E, top_k, H, I, renormalize, out,
                       topk_ids_out, topk_weights_out, nullptr, 0, info, stream);
  }
  if (need > (size_t)MOE_NOALLOC_SCRATCH_BYTES) return MOE_ERR_WORKSPACE;
  void* ws = nullptr;
  if (scratch_on_current_device(&ws) != hipSuccess) return MOE_ERR_HIP;
  return moe_forward(x, w_router, logit_bias, w13, w2, M, E, top_k, H, I, renormalize, out,
                     topk_ids_out, topk_weights_out, ws, (size_t)MOE_NOALLOC_SCRATCH_BYTES, info,
                     stream);
}
