// The attention launch for callers that cannot allocate device memory: vc_attn_mixed with its
// workspace taken from a device array the library holds, instead of a caller's buffer.
//
// The array is a file-scope __device__ variable, so every device the library runs on holds its
// own copy (VC_SCRATCH_BYTES) from the first use until the process ends.  In host code the
// variable's name is only a host-side handle: its device address is looked up once per device
// with hipGetSymbolAddress (with that device current) and that address is what the kernels get.
#include <stdio.h>

#include <mutex>

#include "vc_internal.h"

namespace vc {

static __device__ __attribute__((aligned(256))) uint8_t scratch[VC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

// Device address of the current device's copy of `scratch` (NULL and a recorded error on failure).
void* scratch_address() {
  int dev = 0;
  if (hip_check(hipGetDevice(&dev), "hipGetDevice")) return nullptr;
  if (dev < 0 || dev >= kMaxDevices) {
    fail(VC_EUNSUPPORTED, "device index beyond the library's table");
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hip_check(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), "hipGetSymbolAddress (scratch)")) return nullptr;
    g_scratch_ptr[dev] = p;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

}  // namespace vc

using namespace vc;

extern "C" {

int vc_attn_mixed_noalloc(const vc_shape* shape, int num_reqs, const vc_req* reqs, const void* q,
                          const void* blk_k, const void* blk_v, int num_pools, const vc_pool* pools,
                          float* out, int split_pages, void* stream) {
  set_error("");
  if (!pools) return fail(VC_EINVAL, "pools is NULL");
  if (num_reqs < 0 || num_reqs > VC_MAX_REQS) return fail(VC_EINVAL, "num_reqs must be in [0, 1024]");
  if (num_reqs == 0) return VC_OK;
  if (!reqs) return fail(VC_EINVAL, "reqs is NULL");
  // the same sizing as the workspace of vc_attn_mixed; checked before anything touches a device
  const size_t need = vc_attn_workspace_size(shape, num_reqs, reqs, split_pages);
  if (need > (size_t)VC_SCRATCH_BYTES) {
    char buf[200];
    snprintf(buf, sizeof buf,
             "this launch needs %zu bytes of workspace; the library's scratch holds %zu "
             "(use vc_attn_mixed with a workspace, or fewer context splits)",
             need, (size_t)VC_SCRATCH_BYTES);
    return fail(VC_ENOSPACE, buf);
  }
  void* ws = need > 0 ? scratch_address() : nullptr;
  if (need > 0 && !ws) return VC_EHIP;
  return vc_attn_mixed(shape, num_reqs, reqs, q, blk_k, blk_v, num_pools, pools, out, ws,
                       need > 0 ? (size_t)VC_SCRATCH_BYTES : 0, split_pages, stream);
}

}  // extern "C"
