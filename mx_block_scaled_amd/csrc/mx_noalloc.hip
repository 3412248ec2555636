// mx_noalloc.hip — mxfp8_linear for callers that cannot allocate device memory (code under HIP
// graph capture, tight serving loops, harnesses that forbid hipMalloc).
//
// mxfp8_linear takes a caller-provided workspace: the counters of the split-K decode kernel's
// cross-workgroup sum, its fp32 partial sums, the quantized activations of the two-launch path,
// and the tiled GEMM's split-K parts.  This entry point takes none: the same kernels use
// `scratch`, a file-scope device array that every GPU the library runs on holds until the
// process ends.  Its address on the current device is taken once per device with
// hipGetSymbolAddress (the array's name in host code is only a host-side stand-in) and kept in
// g_scratch[device]; kernels are only ever given that address.
//
// Every call on one GPU shares that GPU's array and leaves its contents behind.  The counters at
// its start must be zero before a call; every call leaves them zero, and the first call on a
// device clears them with a fill kernel on the caller's stream.  Calls that overlap on one GPU
// (two streams, or two threads) race on the array; callers must serialize them.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/mxfp8.h"
#include "mx_launch.h"

static constexpr int64_t kScratchBytes = (int64_t)64 << 20;
static_assert(kScratchBytes == MXFP8_NOALLOC_SCRATCH_BYTES, "header and source disagree");

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices];   // per device: that device's address of `scratch`, or null

// zero the counter prefix (kWorkspacePrefix bytes, 16 per thread)
__global__ void __launch_bounds__(256) k_zero_prefix(uint4* p, int n16) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n16) p[i] = make_uint4(0u, 0u, 0u, 0u);
}

int scratch_for_current_device(hipStream_t s, void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return mx::api_fail(MX_EHIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return mx::api_fail(MX_EINVAL, "device %d: the static scratch is kept for devices 0..%d", dev,
                        kMaxDevices - 1);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return mx::api_fail(MX_EHIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev,
                          hipGetErrorString(e));
    constexpr int n16 = (int)(mx::kWorkspacePrefix / 16);
    hipLaunchKernelGGL(k_zero_prefix, dim3((n16 + 255) / 256), dim3(256), 0, s, (uint4*)p, n16);
    e = hipGetLastError();
    if (e != hipSuccess)
      return mx::api_fail(MX_EHIP, "clearing the scratch counters: %s", hipGetErrorString(e));
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return MX_OK;
}

}  // namespace

extern "C" int mxfp8_linear_noalloc(const void* x_bf16, int64_t M, int64_t K, const void* packed,
                                    int64_t N, int fmt, const void* bias, void* y, void* stream) {
  int64_t need = 0;
  int rc = mx::linear_check(x_bf16, M, K, packed, N, fmt, y, &need);
  if (rc) return rc;
  if (M == 0) return mx::api_ok();
  if (need > kScratchBytes)
    return mx::api_fail(MX_EWORKSPACE,
                        "M x N x K = %lld x %lld x %lld needs %lld bytes of scratch; the static "
                        "scratch holds %lld (use mxfp8_linear with a workspace)",
                        (long long)M, (long long)N, (long long)K, (long long)need,
                        (long long)kScratchBytes);
  if ((rc = mx::api_check_arch())) return rc;
  void* ws = nullptr;
  if ((rc = scratch_for_current_device((hipStream_t)stream, &ws))) return rc;
  return mx::linear_launch(x_bf16, M, K, packed, N, fmt, bias, y, ws, stream);
}
