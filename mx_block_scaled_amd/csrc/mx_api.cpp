// mx_api.cpp — the C-ABI front of libmxfp8 (declared in include/mxfp8.h).
//
// Every entry point validates its arguments first (no HIP call on a bad argument, so the error
// paths are testable without a GPU), then checks once per device that it is a gfx950, then
// enqueues its kernels on the caller's stream.  Nothing here allocates or synchronizes.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "../../include/mxfp8.h"
#include "mx_launch.h"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_err[0] = 0;
  return MX_OK;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
bool valid_fmt(int f) { return f == MX_FMT_E4M3 || f == MX_FMT_E2M3 || f == MX_FMT_E3M2; }

// 32-bit index arithmetic in the GEMM kernels: keep every dimension and every operand below
// 2^31 elements.
constexpr int64_t kMaxDim = (int64_t)1 << 30;

int check_mk(int64_t M, int64_t K) {
  if (M < 0) return fail(MX_ESHAPE, "M = %lld is negative", (long long)M);
  if (K <= 0 || K % 32 != 0) return fail(MX_ESHAPE, "K = %lld must be a positive multiple of 32 (the MX block)", (long long)K);
  if (M > kMaxDim || K > kMaxDim || M * K >= ((int64_t)1 << 31))
    return fail(MX_ESHAPE, "M x K = %lld x %lld exceeds the supported size", (long long)M, (long long)K);
  return MX_OK;
}

int check_nk(int64_t N, int64_t K) {
  if (N <= 0 || N % 16 != 0) return fail(MX_ESHAPE, "N = %lld must be a positive multiple of 16", (long long)N);
  if (K <= 0 || K % 32 != 0) return fail(MX_ESHAPE, "K = %lld must be a positive multiple of 32 (the MX block)", (long long)K);
  if (N > kMaxDim || K > kMaxDim || N * K >= ((int64_t)1 << 31))
    return fail(MX_ESHAPE, "N x K = %lld x %lld exceeds the supported size", (long long)N, (long long)K);
  return MX_OK;
}

// gfx950 check, cached per device (the first query per device is a HIP call).
std::mutex g_arch_mu;
int g_arch[64];
bool g_arch_init = false;

int check_arch() {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(MX_EHIP, "hipGetDevice: %s", hipGetErrorString(e));
  int s = mxfp8_device_supported(dev);
  if (s < 0) return s;
  if (s == 0) return fail(MX_EARCH, "device %d is not a gfx950 (CDNA4) GPU", dev);
  return MX_OK;
}

int hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(MX_EHIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

// bytes per K step of an FP6 activation row as the library quantizes it for its own GEMM: every
// step's 96 bytes at the start of a 128-byte slice where K % 128 == 0 (a packed 96-byte slice
// spans two 128-byte lines for every other step, and the GEMM's copies then fetch 1.5 lines per
// row and step: W6A6 512 x 8192 x 8192 41.0-41.5 us packed, 36.6-37.1 us in 128-byte slices)
int fp6_act_step(int64_t K) { return K % 128 == 0 ? 128 : 96; }

int64_t quant_ws_bytes(int64_t M, int64_t K, int afmt = MX_FMT_E4M3) {
  // the counter prefix, xq [M, K] (E4M3) or FP6 rows of K / 128 slices (fp6_act_step), then
  // xs [M, K/32] at a 256-byte boundary
  const int64_t row = afmt == MX_FMT_E4M3 ? K : (fp6_act_step(K) == 128 ? K : K / 4 * 3);
  return mx::kWorkspacePrefix + ((M * row + 255) / 256) * 256 + M * (K / 32);
}

// decode shapes that mxfp8_linear runs on the kernel splitting K across workgroups (outside
// batch-invariant mode).  Its cross-workgroup sum costs about 2 us of memory round trips at
// the end (store, count, load), so the role-split small-M kernel takes every shape it holds:
// up to 16 rows with K <= 8192, and with K <= 4096 up to 64 rows in row tiles (4096 x 4096:
// 6.9 against 9.0 us at M = 32, 8.8 against 12.9 at M = 64).  The split-K kernel keeps 17 to
// 64 rows with a longer K (16 rows from K > 8192) while one workgroup's share of x (M rows x
// K / P bf16) stays within 256 KiB; above that the tiled GEMM with K split across workgroups
// is faster (8192 x 8192, M = 64: 28.1 against 24.5 us)
constexpr int64_t kSkMinM = 16;
bool sk_shape(int64_t M, int64_t N, int64_t K) {
  if (M < kSkMinM || !mx::decode_sk_ok(M, N, K)) return false;
  if (mx::small_m_rs(M, N, K)) return false;   // the role-split small-M kernel
  return M <= 32 || M * (K / mx::decode_sk_parts(N, K)) * 2 <= (256 << 10);
}

// the split-K partial sums of the tiled GEMM follow the quantized activations
int64_t split_offset(int64_t M, int64_t K, int afmt = MX_FMT_E4M3) {
  return (quant_ws_bytes(M, K, afmt) + 255) / 256 * 256;
}
int64_t quant_split_ws_bytes(int64_t M, int64_t N, int64_t K, int afmt = MX_FMT_E4M3) {
  const int64_t sb = mx::gemm_split_bytes(M, N, K);
  return sb ? split_offset(M, K, afmt) + sb : quant_ws_bytes(M, K, afmt);
}

// mxfp8_linear's workspace: the split-K decode kernel's partial sums on its shapes (or, in
// batch-invariant mode, the quantized activations), otherwise the quantized activations and,
// where the tiled GEMM splits K, its partial sums
int64_t linear_ws_bytes(int64_t M, int64_t N, int64_t K) {
  if (sk_shape(M, N, K)) {
    const int64_t sk = mx::kWorkspacePrefix + mx::decode_sk_workspace(M, N, K);
    const int64_t q = quant_ws_bytes(M, K);
    return sk > q ? sk : q;
  }
  // the small-M kernels need none; batch-invariant mode quantizes first and never splits K
  if (mx::small_m_fused(M, N, K)) return quant_ws_bytes(M, K);
  return quant_split_ws_bytes(M, N, K);
}

// (weight, activation) format pairs with kernels: E4M3 activations with any weight format,
// FP6 activations with FP6 weights
int check_fmt_pair(int fmt, int afmt) {
  if (!valid_fmt(fmt)) return fail(MX_EINVAL, "unknown weight format %d", fmt);
  if (!valid_fmt(afmt)) return fail(MX_EINVAL, "unknown activation format %d", afmt);
  if (afmt != MX_FMT_E4M3 && fmt == MX_FMT_E4M3)
    return fail(MX_EINVAL, "FP6 activations (format %d) need FP6 weights", afmt);
  return MX_OK;
}

int check_linear_common(int64_t M, int64_t K, const void* packed, int64_t N, int fmt,
                               const void* y) {
  if (!valid_fmt(fmt)) return fail(MX_EINVAL, "unknown format %d", fmt);
  int rc = check_mk(M, K);
  if (rc) return rc;
  if ((rc = check_nk(N, K))) return rc;
  if (M > 0 && (!packed || !y)) return fail(MX_EINVAL, "null pointer (packed or y)");
  if (M > 0 && (!aligned16(packed) || !aligned16(y)))
    return fail(MX_EALIGN, "packed, y must be 16-byte aligned");
  if (M * N >= ((int64_t)1 << 31)) return fail(MX_ESHAPE, "M x N exceeds the supported size");
  return MX_OK;
}

}  // namespace

namespace mx {

int api_fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return code;
}

int api_ok() { return ok(); }

int api_check_arch() { return check_arch(); }

int linear_check(const void* x_bf16, int64_t M, int64_t K, const void* packed, int64_t N, int fmt,
                 const void* y, int64_t* need) {
  *need = 0;
  int rc = check_linear_common(M, K, packed, N, fmt, y);
  if (rc) return rc;
  if (M == 0) return MX_OK;
  if (!x_bf16) return fail(MX_EINVAL, "null pointer (x)");
  if (!aligned16(x_bf16)) return fail(MX_EALIGN, "x must be 16-byte aligned");
  *need = linear_ws_bytes(M, N, K);
  return MX_OK;
}

int linear_launch(const void* x_bf16, int64_t M, int64_t K, const void* packed, int64_t N, int fmt,
                  const void* bias, void* y, void* workspace, void* stream) {
  CallSettings settings;   // the modes of this call, read once
  hipStream_t s = (hipStream_t)stream;
  if (!mx::batch_invariant() && sk_shape(M, N, K))   // decode: K split across workgroups
    return hip_status(mx::launch_linear_decode_sk((const uint16_t*)x_bf16, M, K,
                                                  (const uint8_t*)packed, N, fmt,
                                                  (const uint16_t*)bias, (uint16_t*)y, workspace, s),
                      "linear (decode, split K) launch");
  if (mx::batch_invariant() ? mx::small_m_invariant(M, N, K, false)
                            : mx::small_m_fused(M, N, K))   // decode: quantizer fused in
    return hip_status(mx::launch_linear_small_m(x_bf16, nullptr, false, M, K,
                                                (const uint8_t*)packed, N, fmt,
                                                (const uint16_t*)bias, (uint16_t*)y, s),
                      "linear (small M) launch");
  uint8_t* xq = (uint8_t*)workspace + mx::kWorkspacePrefix;
  uint8_t* xs = xq + ((M * K + 255) / 256) * 256;
  float* part = !sk_shape(M, N, K) && !mx::small_m_fused(M, N, K) && mx::gemm_split_bytes(M, N, K)
                    ? (float*)((uint8_t*)workspace + split_offset(M, K)) : nullptr;
  hipError_t e = mx::launch_quantize_act((const uint16_t*)x_bf16, M, K, K, xq, xs, s);
  if (e != hipSuccess) return hip_status(e, "quantize_act launch");
  return hip_status(mx::launch_gemm(xq, xs, M, K, (const uint8_t*)packed, N, fmt,
                                    (const uint16_t*)bias, (uint16_t*)y, s, 1, {}, 0, part),
                    "gemm launch");
}

}  // namespace mx

extern "C" {

int mxfp8_device_supported(int device) {
  if (device < 0) return fail(MX_EINVAL, "device %d", device);
  std::lock_guard<std::mutex> lk(g_arch_mu);
  if (!g_arch_init) {
    for (int& a : g_arch) a = -1;
    g_arch_init = true;
  }
  if (device < 64 && g_arch[device] >= 0) return g_arch[device];
  hipDeviceProp_t p;
  hipError_t e = hipGetDeviceProperties(&p, device);
  if (e != hipSuccess) return fail(MX_EHIP, "hipGetDeviceProperties(%d): %s", device, hipGetErrorString(e));
  const int yes = strncmp(p.gcnArchName, "gfx950", 6) == 0 ? 1 : 0;
  if (device < 64) g_arch[device] = yes;
  return yes;
}

const char* mxfp8_last_error(void) { return g_err; }

int mxfp8_quantize_act(const void* x_bf16, int64_t M, int64_t K, int64_t ldx, void* xq, void* xs,
                       void* stream) {
  int rc = check_mk(M, K);
  if (rc) return rc;
  if (M == 0) return ok();
  if (!x_bf16 || !xq || !xs) return fail(MX_EINVAL, "null pointer (x, xq or xs)");
  if (ldx < K) return fail(MX_ESHAPE, "ldx = %lld < K = %lld", (long long)ldx, (long long)K);
  if (ldx % 8 != 0 || !aligned16(x_bf16) || !aligned16(xq))
    return fail(MX_EALIGN, "x, xq must be 16-byte aligned and ldx a multiple of 8");
  if ((rc = check_arch())) return rc;
  return hip_status(mx::launch_quantize_act((const uint16_t*)x_bf16, M, K, ldx, (uint8_t*)xq,
                                            (uint8_t*)xs, (hipStream_t)stream),
                    "quantize_act launch");
}

int mxfp8_quantize_weight(const void* w_bf16, int64_t N, int64_t K, int64_t ldw, int fmt, void* wq,
                          void* ws, void* stream) {
  if (!valid_fmt(fmt)) return fail(MX_EINVAL, "unknown format %d", fmt);
  int rc = check_nk(N, K);
  if (rc) return rc;
  if (!w_bf16 || !wq || !ws) return fail(MX_EINVAL, "null pointer (w, wq or ws)");
  if (ldw < K) return fail(MX_ESHAPE, "ldw = %lld < K = %lld", (long long)ldw, (long long)K);
  if (ldw % 8 != 0 || !aligned16(w_bf16) || !aligned16(wq))
    return fail(MX_EALIGN, "w, wq must be 16-byte aligned and ldw a multiple of 8");
  if ((rc = check_arch())) return rc;
  return hip_status(mx::launch_quantize_weight((const uint16_t*)w_bf16, N, K, ldw, fmt,
                                               (uint8_t*)wq, (uint8_t*)ws, (hipStream_t)stream),
                    "quantize_weight launch");
}

int64_t mxfp8_prepacked_bytes(int64_t N, int64_t K, int fmt) {
  if (!valid_fmt(fmt) || check_nk(N, K)) return 0;
  const mx::PackGeom p = mx::pack_geom(N, K, fmt);
  return p.wbytes + p.sbytes;
}

int mxfp8_prepack_weight(const void* wq, int64_t ldw_bytes, const void* ws, int64_t ld_ws,
                         int64_t N, int64_t K, int fmt, void* packed, void* stream) {
  if (!valid_fmt(fmt)) return fail(MX_EINVAL, "unknown format %d", fmt);
  int rc = check_nk(N, K);
  if (rc) return rc;
  if (!wq || !ws || !packed) return fail(MX_EINVAL, "null pointer (wq, ws or packed)");
  const int64_t row = fmt == MX_FMT_E4M3 ? K : K / 4 * 3;
  if (ldw_bytes < row) return fail(MX_ESHAPE, "ldw_bytes = %lld < row bytes %lld", (long long)ldw_bytes, (long long)row);
  if (ld_ws < K / 32) return fail(MX_ESHAPE, "ld_ws = %lld < K/32 = %lld", (long long)ld_ws, (long long)(K / 32));
  if (!aligned16(packed)) return fail(MX_EALIGN, "packed must be 16-byte aligned");
  if ((rc = check_arch())) return rc;
  return hip_status(mx::launch_prepack((const uint8_t*)wq, ldw_bytes, (const uint8_t*)ws, ld_ws, N,
                                       K, fmt, (uint8_t*)packed, (hipStream_t)stream),
                    "prepack launch");
}

int mxfp8_unpack_weight(const void* packed, int64_t N, int64_t K, int fmt, void* wq, void* ws,
                        void* stream) {
  if (!valid_fmt(fmt)) return fail(MX_EINVAL, "unknown format %d", fmt);
  int rc = check_nk(N, K);
  if (rc) return rc;
  if (!wq || !ws || !packed) return fail(MX_EINVAL, "null pointer (packed, wq or ws)");
  if (!aligned16(packed)) return fail(MX_EALIGN, "packed must be 16-byte aligned");
  if ((rc = check_arch())) return rc;
  return hip_status(mx::launch_unpack((const uint8_t*)packed, N, K, fmt, (uint8_t*)wq,
                                      (uint8_t*)ws, (hipStream_t)stream),
                    "unpack launch");
}

int mxfp8_prepack_weight_shuffled16(const void* w16, const void* ws, int64_t ld_ws, int64_t N,
                                    int64_t K, void* packed, void* stream) {
  int rc = check_nk(N, K);
  if (rc) return rc;
  if (!w16 || !ws || !packed) return fail(MX_EINVAL, "null pointer (w16, ws or packed)");
  if (ld_ws < K / 32) return fail(MX_ESHAPE, "ld_ws = %lld < K/32 = %lld", (long long)ld_ws, (long long)(K / 32));
  if (!aligned16(packed)) return fail(MX_EALIGN, "packed must be 16-byte aligned");
  if ((rc = check_arch())) return rc;
  return hip_status(mx::launch_prepack_shuffled16((const uint8_t*)w16, (const uint8_t*)ws, ld_ws,
                                                  N, K, (uint8_t*)packed, (hipStream_t)stream),
                    "prepack (shuffled16) launch");
}

int mxfp8_unpack_weight_shuffled16(const void* packed, int64_t N, int64_t K, void* w16, void* ws,
                                   void* stream) {
  int rc = check_nk(N, K);
  if (rc) return rc;
  if (!w16 || !ws || !packed) return fail(MX_EINVAL, "null pointer (packed, w16 or ws)");
  if (!aligned16(packed)) return fail(MX_EALIGN, "packed must be 16-byte aligned");
  if ((rc = check_arch())) return rc;
  return hip_status(mx::launch_unpack_shuffled16((const uint8_t*)packed, N, K, (uint8_t*)w16,
                                                 (uint8_t*)ws, (hipStream_t)stream),
                    "unpack (shuffled16) launch");
}

int64_t mxfp8_workspace_bytes(int64_t M, int64_t N, int64_t K, int fmt) {
  if (!valid_fmt(fmt) || check_mk(M, K) || check_nk(N, K)) return 0;
  if (M == 0) return 0;
  return linear_ws_bytes(M, N, K);
}


int mxfp8_linear(const void* x_bf16, int64_t M, int64_t K, const void* packed, int64_t N, int fmt,
                 const void* bias, void* y, void* workspace, int64_t ws_bytes, void* stream) {
  int64_t need = 0;
  int rc = mx::linear_check(x_bf16, M, K, packed, N, fmt, y, &need);
  if (rc) return rc;
  if (M == 0) return ok();
  if (!workspace || ws_bytes < need)
    return fail(MX_EWORKSPACE, "workspace of %lld bytes given, %lld needed", (long long)ws_bytes, (long long)need);
  if (!aligned16(workspace)) return fail(MX_EALIGN, "workspace must be 16-byte aligned");
  if ((rc = check_arch())) return rc;
  return mx::linear_launch(x_bf16, M, K, packed, N, fmt, bias, y, workspace, stream);
}

int mxfp8_linear_prequant(const void* xq, const void* xs, int64_t M, int64_t K, const void* packed,
                          int64_t N, int fmt, const void* bias, void* y, void* stream) {
  mx::CallSettings settings;   // the modes of this call, read once
  int rc = check_linear_common(M, K, packed, N, fmt, y);
  if (rc) return rc;
  if (M == 0) return ok();
  if (!xq || !xs) return fail(MX_EINVAL, "null pointer (xq or xs)");
  if (!aligned16(xq)) return fail(MX_EALIGN, "xq must be 16-byte aligned");
  if ((rc = check_arch())) return rc;
  return hip_status(mx::launch_gemm((const uint8_t*)xq, (const uint8_t*)xs, M, K,
                                    (const uint8_t*)packed, N, fmt, (const uint16_t*)bias,
                                    (uint16_t*)y, (hipStream_t)stream),
                    "gemm launch");
}

int mxfp8_linear_batched(const void* x_bf16, int64_t B, int64_t M, int64_t K, const void* packed,
                         int64_t N, int fmt, const void* bias, void* y, void* workspace,
                         int64_t ws_bytes, void* stream) {
  mx::CallSettings settings;   // the modes of this call, read once
  if (B < 0) return fail(MX_ESHAPE, "B = %lld is negative", (long long)B);
  if (B > 0 && M > 0 && B * M / B != M) return fail(MX_ESHAPE, "B x M overflows");
  int rc = check_linear_common(B * M, K, packed, N, fmt, y);
  if (rc) return rc;
  if (B == 0 || M == 0) return ok();
  if (!x_bf16) return fail(MX_EINVAL, "null pointer (x)");
  if (!aligned16(x_bf16)) return fail(MX_EALIGN, "x must be 16-byte aligned");
  const int64_t need = quant_ws_bytes(B * M, K);
  if (!workspace || ws_bytes < need)
    return fail(MX_EWORKSPACE, "workspace of %lld bytes given, %lld needed", (long long)ws_bytes, (long long)need);
  if (!aligned16(workspace)) return fail(MX_EALIGN, "workspace must be 16-byte aligned");
  if (B > 65535) return fail(MX_ESHAPE, "B = %lld exceeds 65535", (long long)B);
  if ((rc = check_arch())) return rc;
  hipStream_t s = (hipStream_t)stream;
  const int64_t P = mxfp8_prepacked_bytes(N, K, fmt);   // a multiple of 16
  mx::BatchStrides bs;
  bs.w = P;
  bs.y = M * N * 2;
  bs.bias = bias ? N * 2 : 0;
  if (mx::batch_invariant() ? mx::small_m_invariant(M, N, K, false)
                            : mx::small_m_fused(M, N, K)) {
    bs.x = M * K * 2;
    return hip_status(mx::launch_linear_small_m(x_bf16, nullptr, false, M, K,
                                                (const uint8_t*)packed, N, fmt,
                                                (const uint16_t*)bias, (uint16_t*)y, s, (int)B, bs),
                      "linear (batched, small M) launch");
  }
  uint8_t* xq = (uint8_t*)workspace + mx::kWorkspacePrefix;
  uint8_t* xs = xq + ((B * M * K + 255) / 256) * 256;
  hipError_t e = mx::launch_quantize_act((const uint16_t*)x_bf16, B * M, K, K, xq, xs, s);
  if (e != hipSuccess) return hip_status(e, "quantize_act launch");
  bs.x = M * K;
  bs.xs = M * (K / 32);
  return hip_status(mx::launch_gemm(xq, xs, M, K, (const uint8_t*)packed, N, fmt,
                                    (const uint16_t*)bias, (uint16_t*)y, s, (int)B, bs),
                    "gemm (batched) launch");
}

int mxfp8_linear_prequant_batched(const void* xq, const void* xs, int64_t B, int64_t M, int64_t K,
                                  const void* packed, int64_t N, int fmt, const void* bias,
                                  void* y, void* stream) {
  mx::CallSettings settings;   // the modes of this call, read once
  if (B < 0) return fail(MX_ESHAPE, "B = %lld is negative", (long long)B);
  if (B > 0 && M > 0 && B * M / B != M) return fail(MX_ESHAPE, "B x M overflows");
  int rc = check_linear_common(B * M, K, packed, N, fmt, y);
  if (rc) return rc;
  if (B == 0 || M == 0) return ok();
  if (!xq || !xs) return fail(MX_EINVAL, "null pointer (xq or xs)");
  if (!aligned16(xq)) return fail(MX_EALIGN, "xq must be 16-byte aligned");
  if (B > 65535) return fail(MX_ESHAPE, "B = %lld exceeds 65535", (long long)B);
  if ((rc = check_arch())) return rc;
  mx::BatchStrides bs;
  bs.x = M * K;
  bs.xs = M * (K / 32);
  bs.w = mxfp8_prepacked_bytes(N, K, fmt);
  bs.y = M * N * 2;
  bs.bias = bias ? N * 2 : 0;
  return hip_status(mx::launch_gemm((const uint8_t*)xq, (const uint8_t*)xs, M, K,
                                    (const uint8_t*)packed, N, fmt, (const uint16_t*)bias,
                                    (uint16_t*)y, (hipStream_t)stream, (int)B, bs),
                    "gemm (batched) launch");
}

int mxfp8_quantize_act_fmt(const void* x_bf16, int64_t M, int64_t K, int64_t ldx, int afmt,
                           void* xq, void* xs, void* stream) {
  if (!valid_fmt(afmt)) return fail(MX_EINVAL, "unknown activation format %d", afmt);
  if (afmt == MX_FMT_E4M3) return mxfp8_quantize_act(x_bf16, M, K, ldx, xq, xs, stream);
  int rc = check_mk(M, K);
  if (rc) return rc;
  if (M == 0) return ok();
  if (!x_bf16 || !xq || !xs) return fail(MX_EINVAL, "null pointer (x, xq or xs)");
  if (ldx < K) return fail(MX_ESHAPE, "ldx = %lld < K = %lld", (long long)ldx, (long long)K);
  if (ldx % 8 != 0 || !aligned16(x_bf16) || !aligned16(xq))
    return fail(MX_EALIGN, "x, xq must be 16-byte aligned and ldx a multiple of 8");
  if ((rc = check_arch())) return rc;
  return hip_status(mx::launch_quantize_act_fp6((const uint16_t*)x_bf16, M, K, ldx, afmt,
                                                (uint8_t*)xq, (uint8_t*)xs, (hipStream_t)stream),
                    "quantize_act (FP6) launch");
}

int64_t mxfp8_workspace_bytes_fmt(int64_t M, int64_t N, int64_t K, int fmt, int afmt) {
  if (!valid_fmt(fmt) || !valid_fmt(afmt) || check_mk(M, K) || check_nk(N, K)) return 0;
  if (afmt != MX_FMT_E4M3 && fmt == MX_FMT_E4M3) return 0;
  if (M == 0) return 0;
  if (afmt == MX_FMT_E4M3) return linear_ws_bytes(M, N, K);   // mxfp8_linear's
  return quant_split_ws_bytes(M, N, K, afmt);
}

int mxfp8_linear_fmt(const void* x_bf16, int64_t M, int64_t K, const void* packed, int64_t N,
                     int fmt, int afmt, const void* bias, void* y, void* workspace,
                     int64_t ws_bytes, void* stream) {
  mx::CallSettings settings;   // the modes of this call, read once
  int rc = check_fmt_pair(fmt, afmt);
  if (rc) return rc;
  if (afmt == MX_FMT_E4M3)
    return mxfp8_linear(x_bf16, M, K, packed, N, fmt, bias, y, workspace, ws_bytes, stream);
  if ((rc = check_linear_common(M, K, packed, N, fmt, y))) return rc;
  if (M == 0) return ok();
  if (!x_bf16) return fail(MX_EINVAL, "null pointer (x)");
  if (!aligned16(x_bf16)) return fail(MX_EALIGN, "x must be 16-byte aligned");
  const int64_t need = quant_split_ws_bytes(M, N, K, afmt);
  if (!workspace || ws_bytes < need)
    return fail(MX_EWORKSPACE, "workspace of %lld bytes given, %lld needed", (long long)ws_bytes, (long long)need);
  if (!aligned16(workspace)) return fail(MX_EALIGN, "workspace must be 16-byte aligned");
  if ((rc = check_arch())) return rc;
  hipStream_t s = (hipStream_t)stream;
  const int xstep = fp6_act_step(K);
  uint8_t* xq = (uint8_t*)workspace + mx::kWorkspacePrefix;
  const int64_t xrow = xstep == 128 ? K : K / 4 * 3;     // code bytes per row (as quant_ws_bytes)
  uint8_t* xs = xq + ((M * xrow + 255) / 256) * 256;
  float* part = mx::gemm_split_bytes(M, N, K) ? (float*)((uint8_t*)workspace + split_offset(M, K, afmt)) : nullptr;
  hipError_t e = mx::launch_quantize_act_fp6((const uint16_t*)x_bf16, M, K, K, afmt, xq, xs, s, xstep);
  if (e != hipSuccess) return hip_status(e, "quantize_act (FP6) launch");
  mx::BatchStrides bs;
  bs.xstep = xstep == 128 ? 128 : 0;
  return hip_status(mx::launch_gemm(xq, xs, M, K, (const uint8_t*)packed, N, fmt,
                                    (const uint16_t*)bias, (uint16_t*)y, s, 1, bs, afmt, part),
                    "gemm launch");
}

int mxfp8_linear_prequant_fmt(const void* xq, const void* xs, int64_t M, int64_t K, int afmt,
                              const void* packed, int64_t N, int fmt, const void* bias, void* y,
                              void* stream) {
  mx::CallSettings settings;   // the modes of this call, read once
  int rc = check_fmt_pair(fmt, afmt);
  if (rc) return rc;
  if (afmt == MX_FMT_E4M3)
    return mxfp8_linear_prequant(xq, xs, M, K, packed, N, fmt, bias, y, stream);
  if ((rc = check_linear_common(M, K, packed, N, fmt, y))) return rc;
  if (M == 0) return ok();
  if (!xq || !xs) return fail(MX_EINVAL, "null pointer (xq or xs)");
  if (!aligned16(xq)) return fail(MX_EALIGN, "xq must be 16-byte aligned");
  if ((rc = check_arch())) return rc;
  return hip_status(mx::launch_gemm((const uint8_t*)xq, (const uint8_t*)xs, M, K,
                                    (const uint8_t*)packed, N, fmt, (const uint16_t*)bias,
                                    (uint16_t*)y, (hipStream_t)stream, 1, {}, afmt),
                    "gemm launch");
}

int mxfp8_rmsnorm_quantize_act(const void* x_bf16, int64_t M, int64_t K, int64_t ldx,
                               const void* gamma_bf16, float eps, void* xq, void* xs,
                               void* y_bf16, void* stream) {
  int rc = check_mk(M, K);
  if (rc) return rc;
  if (!(eps >= 0.0f) || eps > 1e30f) return fail(MX_EINVAL, "eps = %g must be finite and >= 0", (double)eps);
  if (M == 0) return ok();
  if (!x_bf16 || !gamma_bf16 || !xq || !xs) return fail(MX_EINVAL, "null pointer (x, gamma, xq or xs)");
  if (ldx < K) return fail(MX_ESHAPE, "ldx = %lld < K = %lld", (long long)ldx, (long long)K);
  if (ldx % 8 != 0 || !aligned16(x_bf16) || !aligned16(gamma_bf16) || !aligned16(xq) ||
      (y_bf16 && !aligned16(y_bf16)))
    return fail(MX_EALIGN, "x, gamma, xq, y must be 16-byte aligned and ldx a multiple of 8");
  if ((rc = check_arch())) return rc;
  return hip_status(mx::launch_rmsnorm_quant((const uint16_t*)x_bf16, M, K, ldx,
                                             (const uint16_t*)gamma_bf16, eps, (uint8_t*)xq,
                                             (uint8_t*)xs, (uint16_t*)y_bf16, (hipStream_t)stream),
                    "rmsnorm_quantize_act launch");
}

int mxfp8_set_batch_invariant(int on) {
  mx::set_batch_invariant(on != 0);
  return ok();
}

int mxfp8_set_batch_invariant_thread(int mode) {
  if (mode < -1 || mode > 1) return fail(MX_EINVAL, "mode %d is not -1, 0 or 1", mode);
  mx::set_batch_invariant_thread(mode);
  return ok();
}

int mxfp8_set_tile_config(int fn, int fm) {
  static const int ok_cfg[][2] = {{0, 0}, {8, 4}, {7, 4}, {6, 4}, {4, 4}, {4, 2}, {16, 16}, {17, 16}, {18, 16}, {19, 16}, {4, 36}, {6, 36}, {7, 36}};
  for (const auto& c : ok_cfg)
    if (c[0] == fn && c[1] == fm) {
      mx::force_tile(fn, fm);
      return ok();
    }
  return fail(MX_EINVAL, "no compiled tile configuration (%d, %d)", fn, fm);
}

}  // extern "C"
