// noalloc.hip -- moe_route_noalloc: the router with its scratch memory in a
// fixed device array instead of a caller workspace, for callers that cannot
// allocate (code under HIP graph capture, tight serving loops, harnesses that
// forbid allocation).
//
// The router's kernels need scratch for the partial logits of its fixed
// split of the reduction over d (splits x T x E_global fp32; the fp32 router
// writes the whole logits there, splits = 1).  Here that scratch is the file
// array `scratch`, kNoallocScratchBytes per GPU, held by each GPU the library
// runs on until the process ends.  Its device address is taken once per
// device with hipGetSymbolAddress (in host code the array's name is only a
// host-side stand-in) and every launch receives that address.  Every entry
// of the partial logits a call reads is written by the same call first, so
// nothing has to start at zero; calls that overlap on one GPU share the
// array and race.
#include <mutex>

#include "moe_internal.h"

namespace moe {
namespace {

constexpr size_t kNoallocScratchBytes = MOE_ROUTE_NOALLOC_MAX_BYTES;  // 16 MiB
constexpr int kNoallocMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kNoallocMaxDevices] = {};

// The device address of `scratch` on the current device (looked up once per
// device, with that device current).
hipError_t scratch_of_current_device(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kNoallocMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if ((e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch))) != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace

size_t noalloc_route_bytes(const moe_problem_t& p) {
  const int splits = router_splits(p.d, p.E_global, p.x_dtype == MOE_BF16);
  return static_cast<size_t>(splits) * static_cast<size_t>(p.T) * p.E_global * sizeof(float);
}

size_t noalloc_scratch_bytes() { return kNoallocScratchBytes; }

hipError_t launch_route_noalloc(const moe_problem_t& p, const void* x, const void* packed, const float* bias,
                                int32_t* topk_idx, float* topk_w, float* logits, hipStream_t s) {
  void* ptr = nullptr;
  hipError_t e = scratch_of_current_device(&ptr);
  if (e != hipSuccess) return e;
  return launch_route(p, x, packed, bias, topk_idx, topk_w, logits, static_cast<float*>(ptr), s);
}

}  // namespace moe
