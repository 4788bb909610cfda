// The TLR product with the library's own static device workspace, for callers
// that cannot allocate device memory (HIP graph capture, serving loops,
// harnesses that forbid hipMalloc).  Same plan, same launches and kernels as
// plan_execute; only the workspace differs.
//
// The workspace is one file-scope device array per GPU.  In host code the
// array's name is only a host-side stand-in: its device address is looked up
// with hipGetSymbolAddress once per device, with that device current, and
// only that address is ever handed to kernels.  Every call on one GPU shares
// the array and leaves its last contents in it; no product reads workspace it
// has not written first (the planner's self-check proves it per plan), so
// nothing is cleared.  Calls that overlap on one GPU (different streams, no
// ordering between them) race on the array.
#include <hip/hip_runtime.h>

#include <mutex>
#include <string>

#include "tlr_plan.h"

namespace tlr {

namespace {

__device__ __align__(256) unsigned char scratch[TLR_STATIC_WORKSPACE_BYTES];

constexpr int MAX_DEVICES = 64;
std::mutex g_mu;
void *g_scratch[MAX_DEVICES] = {};

// Device address of this device's copy of the array (looked up on the first
// call on the device, with the device current).
tlr_status scratch_of(int dev, void **out) {
  if (dev < 0 || dev >= MAX_DEVICES) return fail(TLR_ERR_INVALID_ARG, "execute_noalloc: device index out of range");
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_scratch[dev]) {
    void *p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(TLR_ERR_HIP, std::string("execute_noalloc: hipGetSymbolAddress of the static workspace: ") +
                                   hipGetErrorString(e));
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return TLR_OK;
}

}  // namespace

tlr_status plan_execute_noalloc(Plan *p, double alpha, const tlr_buffers *A, const tlr_buffers *B,
                                const void *B_dense, int64_t ldb, double beta, void *C, int64_t ldc,
                                void *const *streams, int n_streams) {
  if (!p->dev_desc) return fail(TLR_ERR_NOT_BOUND, "execute_noalloc: plan is not bound");
  if (p->ws_bytes > (size_t)TLR_STATIC_WORKSPACE_BYTES)
    return fail(TLR_ERR_WORKSPACE, "execute_noalloc: the plan needs " + std::to_string(p->ws_bytes) +
                                       " bytes of workspace, more than the static workspace of " +
                                       std::to_string((size_t)TLR_STATIC_WORKSPACE_BYTES) +
                                       " bytes; analyse it with workspace_budget <= TLR_STATIC_WORKSPACE_BYTES");
  int dev = 0;
  const hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(TLR_ERR_HIP, std::string("execute_noalloc: hipGetDevice: ") + hipGetErrorString(e));
  void *ws = nullptr;
  const tlr_status st = scratch_of(dev, &ws);
  if (st != TLR_OK) return st;
  return plan_execute(p, alpha, A, B, B_dense, ldb, beta, C, ldc, ws, (size_t)TLR_STATIC_WORKSPACE_BYTES, streams,
                      n_streams);
}

}  // namespace tlr
