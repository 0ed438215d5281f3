// forward_noalloc.hip -- moe_forward for callers that cannot allocate device
// memory: its workspace is one file-scope device array of fixed size.
//
// Each GPU the library runs on holds its own copy of `scratch` for the life
// of the process.  Host code never passes the array's name to a kernel (on
// the host it is a stand-in, not a device address): the device address is
// taken once per device with hipGetSymbolAddress, with that device current,
// and kept in g_scratch_ptr.
#include <hip/hip_runtime.h>

#include <mutex>

#include "moe_internal.h"

namespace moe {
namespace {

__device__ __align__(256) unsigned char scratch[MOE_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void *g_scratch_ptr[kMaxDevices];

// Device address of this device's scratch array (nullptr on a HIP error).
void *scratch_for_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    g_scratch_ptr[dev] = p;
  }
  return g_scratch_ptr[dev];
}

}  // namespace
}  // namespace moe

extern "C" int moe_forward_noalloc(const moe_layer_desc *desc, int32_t T, const void *x, const moe_weights *w,
                                   void *y, int32_t out_dtype, int32_t *topk_idx_out, float *topk_w_out,
                                   void *stream) {
  using namespace moe;
  int s;
  if ((s = validate_desc(desc)) || (s = validate_T(T))) return s;
  if (workspace_layout(desc, T).total > size_t(MOE_NOALLOC_SCRATCH_BYTES)) return MOE_E_WORKSPACE;
  void *ws = scratch_for_current_device();
  if (!ws) return MOE_E_HIP;
  // moe_forward needs no zeroed workspace: every section it reads is written
  // earlier in the same call.
  return moe_forward(desc, T, x, w, y, out_dtype, topk_idx_out, topk_w_out, ws, size_t(MOE_NOALLOC_SCRATCH_BYTES),
                     stream);
}
