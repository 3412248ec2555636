// mx_gemm.hip — block-scaled GEMM on gfx950's scaled MFMA (v_mfma_scale_f32_16x16x128_f8f6f4).
//
// y[m, n] = sum_kb 2^(sx[m,kb]-127) 2^(sw[n,kb]-127) sum_{k in kb} xq[m,k] wq[n,k]  (+ bias[n])
// (aiter_flydsl page, apply_weights: block-scaled GEMM with row-major [M, K/32] activation
// scales and [N, K/32] weight scales, bf16 output, bias added afterwards — here fused into the
// fp32 epilogue so the output is rounded once.)
//
// The weight is the MFMA's A operand (rows = n) and the activations the B operand (columns =
// m): each lane then owns 4 consecutive n of one output row m, i.e. one 8-byte bf16 store.
#include "mx_device.h"
#include "mx_launch.h"

namespace mx {

// ---------------------------------------------------------------- generic kernel
// Any M, K % 32 == 0, N % 16 == 0.  Workgroup = 4 waves = 64 weight rows x 32 activation rows;
// each wave owns one 16-row weight fragment and two 16-row activation tiles, streaming both
// operands straight from global memory into registers (no LDS).
template <int WFMT>
__global__ __launch_bounds__(256) void k_gemm_generic(const uint8_t* __restrict__ xq,
                                                      const uint8_t* __restrict__ xs, int M, int K,
                                                      const uint8_t* __restrict__ packed, int N,
                                                      const uint16_t* __restrict__ bias,
                                                      uint16_t* __restrict__ y) {
  constexpr int FB = frag_bytes(WFMT);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int NG = N >> 4, KT = (K + 127) >> 7, KB = K >> 5;
  const int ng = blockIdx.x * 4 + w;
  if (ng >= NG) return;  // whole wave leaves; nothing below synchronizes across waves
  const int m0 = blockIdx.y * 32;
  const uint8_t* wfr = packed + (int64_t)ng * FB;
  const uint32_t* wsc = (const uint32_t*)(packed + (int64_t)KT * NG * FB) + (int64_t)ng * 64 + lane;
  // activation rows of this lane (clamped so every address is inside x; data is zeroed instead)
  int mrow[2];
  bool mok[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int m = m0 + 16 * t + r;
    mok[t] = m < M;
    mrow[t] = mok[t] ? m : M - 1;
  }
  v4f acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
  for (int kt = 0; kt < KT; ++kt) {
    const uint8_t* f = wfr + (int64_t)kt * NG * FB;
    v8i a;
    if (WFMT == 0) {
      const v4i lo = *(const v4i*)(f + lane * 16);
      const v4i hi = *(const v4i*)(f + 1024 + lane * 16);
      a = (v8i){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    } else {
      const v4i lo = *(const v4i*)(f + lane * 16);
      const v2i hi = *(const v2i*)(f + 1024 + lane * 8);
      a = (v8i){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], 0, 0};
    }
    const int sa = (int)((wsc[(int64_t)(kt >> 2) * NG * 64] >> (8 * (kt & 3))) & 0xFFu);
    const int kb = 4 * kt + g;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const uint8_t* xr = xq + (int64_t)mrow[t] * K;
      v4i b0 = {0, 0, 0, 0}, b1 = {0, 0, 0, 0};
      const int k0 = 128 * kt + 16 * g, k1 = k0 + 64;
      if (mok[t] && k0 < K) b0 = *(const v4i*)(xr + k0);
      if (mok[t] && k1 < K) b1 = *(const v4i*)(xr + k1);
      const v8i b = {b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
      const int sb = kb < KB ? (int)xs[(int64_t)mrow[t] * KB + kb] : 127;
      acc[t] = mfma16<WFMT, 0>(a, b, acc[t], sa, sb);
    }
  }
  // epilogue: lane holds n = 16 ng + 4 g + i (i < 4) of activation row m0 + 16 t + r
  const int n = 16 * ng + 4 * g;
  float bv[4] = {0.f, 0.f, 0.f, 0.f};
  if (bias) {
#pragma unroll
    for (int i = 0; i < 4; ++i) bv[i] = bf16_to_float(bias[n + i]);
  }
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    if (!mok[t]) continue;
    const v2i o = {(int)pack_bf16x2(acc[t][0] + bv[0], acc[t][1] + bv[1]),
                   (int)pack_bf16x2(acc[t][2] + bv[2], acc[t][3] + bv[3])};
    *(v2i*)(y + (int64_t)mrow[t] * N + n) = o;
  }
}

hipError_t launch_gemm(const uint8_t* xq, const uint8_t* xs, int64_t M, int64_t K,
                       const uint8_t* packed, int64_t N, int fmt, const uint16_t* bias,
                       uint16_t* y, hipStream_t s) {
  dim3 grid((unsigned)((N / 16 + 3) / 4), (unsigned)((M + 31) / 32)), block(256);
  const int m = (int)M, k = (int)K, n = (int)N;
  switch (fmt) {
    case 0: hipLaunchKernelGGL(k_gemm_generic<0>, grid, block, 0, s, xq, xs, m, k, packed, n, bias, y); break;
    case 2: hipLaunchKernelGGL(k_gemm_generic<2>, grid, block, 0, s, xq, xs, m, k, packed, n, bias, y); break;
    case 3: hipLaunchKernelGGL(k_gemm_generic<3>, grid, block, 0, s, xq, xs, m, k, packed, n, bias, y); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace mx
