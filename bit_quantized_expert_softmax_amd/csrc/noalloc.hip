// Routing without a caller workspace, for callers that cannot allocate
// device memory (code under HIP graph capture, tight serving loops, harnesses
// that forbid hipMalloc).
//
// The fp64 logits that moe_route keeps in its workspace live here in one
// file-scope device array instead. Each GPU the library runs on holds its own
// copy of the array, at its own address, until the process ends; the host
// looks that address up once per device (hipGetSymbolAddress with the device
// current) and passes it to the kernels like any workspace pointer. The
// array's name in host code is only a host-side stand-in, never a device
// address. Every call on one GPU shares that GPU's array, so calls that
// overlap on one GPU (on different streams, or from different threads) race;
// the logits are written in full before they are read, so nothing needs
// clearing between calls.
#include <hip/hip_runtime.h>

#include <mutex>

#include "host_common.h"
#include "launch.h"

namespace {

constexpr int kScratchDoubles = MOE_ROUTE_NOALLOC_MAX;  // 1 MiB of fp64 logits
constexpr int kMaxDevices = 64;

static __device__ __align__(256) double scratch[kScratchDoubles];

std::mutex g_mu;
double* g_scratch[kMaxDevices] = {};

// The current device's copy of the scratch array (looked up on first use).
hipError_t scratch_on_current_device(double** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch[dev] = static_cast<double*>(p);
  }
  *out = g_scratch[dev];
  return hipSuccess;
}

}  // namespace

namespace moe {
moe_status check_shape(const moe_shape* sh, const char* fn);
}

using moe::fail;

extern "C" {

moe_status moe_route_noalloc(const moe_shape* sh, const float* x, const uint16_t* wr, const float* bias,
                             const float* logits_in, int32_t B, int32_t* ids, float* w, void* stream) {
  moe::clear_error();
  const char* fn = "moe_route_noalloc";
  moe_status st = moe::check_shape(sh, fn);
  if (st) return st;
  if (B < 0) return fail(MOE_ESHAPE, "%s: B=%d is negative", fn, B);
  if (B == 0) return MOE_OK;
  if (!ids || !w) return fail(MOE_EINVAL, "%s: ids and w must not be NULL", fn);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (logits_in) {
    const hipError_t e = moe::launch_route_topk(nullptr, logits_in, B, sh->n_experts, sh->top_k, ids, w,
                                                nullptr, nullptr, s);
    if (e != hipSuccess) return fail(MOE_EHIP, "%s: %s", fn, hipGetErrorString(e));
    return MOE_OK;
  }
  if (!x || !wr) return fail(MOE_EINVAL, "%s: x and wr must not be NULL without logits_in", fn);
  if (!moe::aligned16(x) || !moe::aligned16(wr)) return fail(MOE_EALIGN, "%s: x and wr must be 16-byte aligned", fn);
  if (static_cast<int64_t>(B) * sh->n_experts > kScratchDoubles)
    return fail(MOE_ESHAPE, "%s: B * n_experts = %lld exceeds the scratch limit %d", fn,
                static_cast<long long>(B) * sh->n_experts, kScratchDoubles);
  double* z = nullptr;
  hipError_t e = scratch_on_current_device(&z);
  if (e != hipSuccess) return fail(MOE_EHIP, "%s: scratch address: %s", fn, hipGetErrorString(e));
  e = moe::launch_route_logits(x, B, sh->hidden, wr, bias, sh->n_experts, z, s);
  if (e == hipSuccess)
    e = moe::launch_route_topk(z, nullptr, B, sh->n_experts, sh->top_k, ids, w, nullptr, nullptr, s);
  if (e != hipSuccess) return fail(MOE_EHIP, "%s: %s", fn, hipGetErrorString(e));
  return MOE_OK;
}

}  // extern "C"
