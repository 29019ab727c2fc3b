// zl_attn_bwd_noalloc: the backward with its scratch in a fixed device array instead of a
// caller workspace, for callers that cannot allocate device memory (code under HIP graph
// capture, tight serving loops, harnesses that forbid hipMalloc).
//
// The backward's scratch (queue counters, -D and -LSE / tau per query row, sentinel rows,
// split-item counters and partials, visit counters) lives in `scratch`, a file-scope device
// array of kNoallocScratchBytes. Each device holds its own copy for the life of the process.
// Its address is looked up once per device (hipGetSymbolAddress, with that device current) on
// the first call there and kept; the host-side name of the array is never passed to a kernel.
// The pre-pass rewrites every part of the scratch the later launches read (it clears the
// counters and writes the row values and sentinels), so the contents a previous call left
// behind do not matter. Calls that overlap on one device race on the array.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>
#include <string>

#include "zl_internal.h"

namespace {

constexpr size_t kNoallocScratchBytes = ZL_NOALLOC_SCRATCH_BYTES;
static_assert(kNoallocScratchBytes % 256 == 0, "the scratch size keeps 256-byte alignment");

static __device__ __align__(256) char scratch[kNoallocScratchBytes];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];  // device address of `scratch` per device, once known
std::mutex g_scratch_mu;

zl_status fail(zl_status st, const std::string& msg) {
  zl::set_error(msg);
  return st;
}

// The current device's copy of `scratch` (dev is the current device).
zl_status scratch_on(int dev, void** out) {
  if (dev < 0 || dev >= kMaxDevices)
    return fail(ZL_ERR_UNSUPPORTED, "zl_attn_bwd_noalloc: device index " + std::to_string(dev) + " out of range");
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch[dev].load(std::memory_order_relaxed);
    if (!p) {
      const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess || !p) {
        (void)hipGetLastError();
        return fail(ZL_ERR_HIP, std::string("zl_attn_bwd_noalloc: hipGetSymbolAddress(scratch) failed: ") +
                                    hipGetErrorString(e));
      }
      g_scratch[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return ZL_OK;
}

}  // namespace

extern "C" zl_status zl_attn_bwd_noalloc(const zl_plan* plan, const void* q, const void* k, const void* v,
                                         const float* o, const float* lse, const void* d_o, float* dq, float* dk,
                                         float* dv, void* stream) {
  if (!plan) return fail(ZL_ERR_INVALID, "zl_attn_bwd_noalloc: plan is NULL");
  zl_plan_info_t info;
  zl_status st = zl_plan_info(plan, &info);
  if (st != ZL_OK) return st;
  if (info.ws_bwd > kNoallocScratchBytes)
    return fail(ZL_ERR_UNSUPPORTED, "zl_attn_bwd_noalloc: the plan's backward needs " + std::to_string(info.ws_bwd) +
                                        " bytes of scratch, more than the fixed " +
                                        std::to_string(kNoallocScratchBytes) +
                                        "; use zl_attn_bwd with a workspace");
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return fail(ZL_ERR_HIP, "zl_attn_bwd_noalloc: hipGetDevice failed");
  void* ws = nullptr;
  st = scratch_on(dev, &ws);
  if (st != ZL_OK) return st;
  return zl_attn_bwd_stages(plan, q, k, v, o, lse, d_o, dq, dk, dv, ws, ZL_BWD_ALL, stream);
}
