// mhc_pre_static: mhc_pre for callers that cannot allocate device memory
// (code under stream capture, tight serving loops, harnesses that forbid
// hipMalloc). The workspace mhc_pre takes from its caller (the status words,
// the packed fn of the two-pass path, the split-K partials or the single-pass
// exchange words) lives here in one file-scope device array per GPU, of
// kStaticScratchBytes bytes, held from the library's load until the process
// ends.
//
// In host code `scratch` names a host-side stand-in, not the device array:
// every use goes through the address hipGetSymbolAddress returns for the
// current device, looked up once per device and kept.
//
// Every call on a GPU shares that GPU's array. The status words at its start
// carry the single-pass exchange's epoch and shape marker from one call to the
// next (as in a caller's workspace that only mhc_pre uses); they are zero when
// the library is loaded and are cleared once more, by a one-block kernel on the
// first call's stream, when a device is first used. Calls that overlap on one
// GPU (on different streams, or from different host threads without ordering)
// race on the array and must not be made.

#include <atomic>
#include <mutex>

#include "mhc_internal.h"

namespace mhc {
namespace {

constexpr size_t kStaticScratchBytes = MHC_PRE_STATIC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

__global__ void clear_status_kernel(unsigned long long* status) {
  if (threadIdx.x < kStatusBytes / 8) status[threadIdx.x] = 0ull;
}

std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_setup;

// The scratch array's device address on the current device (set up on first
// use: looked up, and its status words cleared on `s`). A WorkspaceProvider.
int scratch_address(hipStream_t s, void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e);
  if (dev < 0 || dev >= kMaxDevices) return fail_with(MHC_ERR_UNSUPPORTED, "mhc_pre_static: device index above 63");
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(g_setup);
    p = g_scratch[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return hip_fail(e);
      if (p == nullptr) return fail_with(MHC_ERR_HIP, "mhc_pre_static: no device address for the scratch array");
      hipLaunchKernelGGL(clear_status_kernel, dim3(1), dim3(64), 0, s, static_cast<unsigned long long*>(p));
      e = hipGetLastError();
      if (e != hipSuccess) return hip_fail(e);
      g_scratch[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return MHC_OK;
}

}  // namespace
}  // namespace mhc

using namespace mhc;

extern "C" {

MHC_API int mhc_pre_static(float* post, float* comb, void* y, const void* residual, mhc_dtype dt, const float* fn,
                           const float* hc_scale, const float* bias, int64_t T, int n, int64_t D,
                           int sinkhorn_repeat, float eps, int n_splits, void* stream) {
  if (mhc_pre_workspace_bytes(T, n, D, n_splits, dt) > kStaticScratchBytes)
    return fail_with(MHC_ERR_WORKSPACE,
                     "mhc_pre_static: these sizes need more workspace than the 32 MiB static scratch; call mhc_pre "
                     "with a workspace of mhc_pre_workspace_bytes() bytes");
  // every argument check of mhc_pre runs first; the scratch is looked up (and
  // set up on a device's first call) only for a call that will launch
  return pre_call(post, comb, y, residual, dt, fn, hc_scale, bias, T, n, D, sinkhorn_repeat, eps, n_splits, nullptr,
                  kStaticScratchBytes, static_cast<hipStream_t>(stream), scratch_address);
}

}  // extern "C"
