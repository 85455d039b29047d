// rola_noalloc.hip -- rola_forward_noalloc: the fused forward on the library's
// own device scratch instead of a caller workspace, for callers that cannot
// allocate device memory (code under HIP graph capture, tight serving loops,
// harnesses that forbid hipMalloc).
//
// The scratch is one file-scope device array per GPU, of a fixed maximum size
// (ROLA_NOALLOC_SCRATCH_BYTES).  Its device address is taken once per device,
// with that device current, by hipGetSymbolAddress and kept; the kernels only
// ever see that address.  Every call on a GPU shares the array, which keeps
// the last call's contents (the forward writes every scratch byte it reads,
// so nothing needs clearing); calls that overlap on one GPU race on it.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/rola.h"

namespace {

static __device__ __align__(256) uint8_t scratch[ROLA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
void *g_scratch[kMaxDevices];
hipError_t g_status[kMaxDevices];
std::once_flag g_once[kMaxDevices];

// the scratch address on device `dev` (taken on the first call for that device)
void *scratch_on(int dev) {
  std::call_once(g_once[dev], [dev] {
    int cur = -1;
    g_status[dev] = hipGetDevice(&cur);
    if (g_status[dev] != hipSuccess) return;
    if (cur != dev && (g_status[dev] = hipSetDevice(dev)) != hipSuccess) return;
    void *ptr = nullptr;
    g_status[dev] = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    g_scratch[dev] = g_status[dev] == hipSuccess ? ptr : nullptr;
    if (cur != dev) (void)hipSetDevice(cur);
  });
  return g_status[dev] == hipSuccess ? g_scratch[dev] : nullptr;
}

}  // namespace

extern "C" int32_t rola_forward_noalloc(const rola_problem *prob, const rola_config *cfg, const void *q,
                                        const void *k, const void *v, const float *wq, const float *wk,
                                        const float *gate, int32_t *block_idx_out, void *out, void *stream) {
  rola_plan_info info;
  const int32_t st = rola_plan(prob, cfg, &info);
  if (st != ROLA_OK) return st;
  if (info.workspace_bytes > (int64_t)ROLA_NOALLOC_SCRATCH_BYTES) return ROLA_ERR_WORKSPACE;
  // the kernels run on the stream's device, so the scratch of that device is used
  int dev = -1;
  if (hipStreamGetDevice((hipStream_t)stream, &dev) != hipSuccess) return ROLA_ERR_DEVICE;
  if (dev < 0 || dev >= kMaxDevices) return ROLA_ERR_UNSUPPORTED;
  void *ws = scratch_on(dev);
  if (!ws) return ROLA_ERR_DEVICE;
  return rola_forward(prob, cfg, q, k, v, wq, wk, gate, block_idx_out, out, ws,
                      (size_t)ROLA_NOALLOC_SCRATCH_BYTES, stream);
}
