// mx_small_m.hip — the MX linear layer for small M (decode shapes).
//
// y[m, n] = sum_kb 2^(sx[m,kb]-127) 2^(sw[n,kb]-127) sum_{k in kb} xq[m,k] wq[n,k]  (+ bias[n])
// (aiter_flydsl page, apply_weights: dynamic MXFP8 activation quantization followed by the
// block-scaled GEMM).  For M <= 32 the weight stream is the whole cost (N K bytes against
// 2 M N K flops), so the kernel is laid out for HBM rather than for the matrix unit:
//  * one workgroup per 16-row weight fragment column (N / 16 workgroups), 8 waves;
//  * K is split across the waves in groups of four 128-wide K steps (wave w takes groups
//    w, w + 8, ...): a wave issues the loads of a whole group (8 KiB of E4M3 weight and its
//    scale word) before using any of it, so the full weight is in flight at once;
//  * the 8 per-wave partial sums are added in LDS in wave order (a split-K whose reduction
//    order is fixed, so results do not depend on timing), then bias, one bf16 rounding, store.
//  * the weight is read with non-temporal loads: each byte is used once per call, and the hint
//    keeps it from displacing cached data (about 10 % per call at M = 1, 4096 x 4096).
// Activations come either as bf16 (M <= 16: quantized inside the kernel, bit-identical to
// k_quantize_act) or pre-quantized (E4M3 xq + row-major E8M0 xs, M <= 32).
//
// The fused quantizer works on the natural row-major layout, where it is cheapest: lane l
// quantizes elements 8 l .. 8 l + 7 of a row's 512-wide group slice (a quad of lanes is one MX
// block, reduced with DPP), writes the codes to a wave-private LDS image, and the MFMA operands
// are then read back from LDS in the operand layout.  Working directly in the operand layout
// would quantize 16 rows per wave whatever M is.
#include "mx_device.h"
#include "mx_launch.h"

namespace mx {

namespace {

// scaled MFMA, weight scale byte picked by op-select j (a constant once the K-step loop is
// unrolled), activation scale in byte 0
template <int WFMT>
__device__ __forceinline__ v4f mfma_wsel(int j, const v8i& a, const v8i& b, v4f c, uint32_t sa,
                                         uint32_t sb) {
  switch (j) {
    case 0: return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, WFMT, 0, 0, (int)sa, 0, (int)sb);
    case 1: return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, WFMT, 0, 1, (int)sa, 0, (int)sb);
    case 2: return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, WFMT, 0, 2, (int)sa, 0, (int)sb);
    default: return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, WFMT, 0, 3, (int)sa, 0, (int)sb);
  }
}

constexpr int kWaves = 8;
constexpr int kRowPitch = 512 + 16;   // LDS row of quantized codes; +16 B spreads rows over banks

}  // namespace

// MT = 16-row activation tiles (M <= 16 MT); QX = activations arrive quantized (xq, xs);
// XS16 = K % 512 == 0 and every row of xs starts 16-byte aligned (scales read 16 B at a time).
template <int WFMT, int MT, bool QX, bool XS16>
__global__ __launch_bounds__(512) void k_linear_small_m(const void* __restrict__ xin,
                                                        const uint8_t* __restrict__ xs, int M,
                                                        int K, const uint8_t* __restrict__ packed,
                                                        int N, const uint16_t* __restrict__ bias,
                                                        uint16_t* __restrict__ y, BatchStrides bs) {
  static_assert(QX || MT == 1, "the fused quantizer covers one 16-row tile");
  {  // batch blockIdx.y (byte strides; all zero when unbatched)
    const int64_t b = blockIdx.y;
    xin = (const uint8_t*)xin + b * bs.x;
    xs += b * bs.xs;
    packed += b * bs.w;
    y = (uint16_t*)((uint8_t*)y + b * bs.y);
    if (bias) bias = (const uint16_t*)((const uint8_t*)bias + b * bs.bias);
  }
  constexpr int FB = frag_bytes(WFMT);
  constexpr int XL = QX ? 16 : 16 * kRowPitch;   // wave-private codes [16 rows][kRowPitch]
  constexpr int SL = QX ? 16 : 16 * 16;          // wave-private scales [16 rows][16 blocks]
  __shared__ __attribute__((aligned(16))) uint8_t xl[kWaves][XL];
  __shared__ __attribute__((aligned(16))) uint8_t sl[kWaves][SL];
  __shared__ v4f red[kWaves][MT][64];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane & 15, g = lane >> 4;
  const int NG = N >> 4, KT = K >> 7, KT4 = (KT + 3) >> 2, KB = K >> 5;
  const int ng = blockIdx.x;
  const int n = 16 * ng + 4 * g;   // first of this lane's 4 output columns
  const uint32_t* wsc = (const uint32_t*)(packed + (int64_t)KT * NG * FB) + (int64_t)ng * 64 + lane;

  // bias of this lane's 4 output columns (the waves that finish a tile use it): one 8-byte load
  // issued behind the first weight loads, so its latency hides under theirs
  const bool want_bias = bias != nullptr && wave < MT;
  const bool bias8 = ((uintptr_t)bias & 7) == 0;
  v2i braw = {0, 0};
  bool have_bias = false;

  // activation rows of this lane's B operands; rows past M read row M - 1 instead: a B-operand
  // row only feeds its own output column, and those columns are never stored
  int mrow[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) mrow[t] = min(16 * t + r, M - 1);

  v4f acc[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) acc[t] = (v4f){0.f, 0.f, 0.f, 0.f};

  for (int kt4 = wave; kt4 < KT4; kt4 += kWaves) {
    // Loads in issue order: activations first (L2-resident after the first workgroups), then
    // the weight (HBM).  Loads retire in order, so the activation work below waits for the
    // activations only and runs while the weight is still in flight.  K steps past the end
    // re-read valid memory; their MFMAs are skipped.
    v4i xr[QX ? 4 : 16][MT][QX ? 2 : 1];
    uint32_t xsb[4][MT];
    if constexpr (QX) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int kt = min(4 * kt4 + j, KT - 1);
#pragma unroll
        for (int t = 0; t < MT; ++t) {
          const uint8_t* p = (const uint8_t*)xin + (int64_t)mrow[t] * K + 128 * kt + 16 * g;
          xr[j][t][0] = *(const v4i*)p;
          xr[j][t][1] = *(const v4i*)(p + 64);
        }
      }
      // activation scales of the group: row bytes 16 kt4 + 4 j + g; with XS16 the row's 16
      // bytes of the group come in one 16-byte load (whole groups only: K % 512 == 0)
#pragma unroll
      for (int t = 0; t < MT; ++t) {
        if constexpr (XS16) {
          const v4i w = *(const v4i*)(xs + (int64_t)mrow[t] * KB + 16 * kt4);
#pragma unroll
          for (int j = 0; j < 4; ++j) xsb[j][t] = (uint32_t)w[j];
        } else {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int kt = min(4 * kt4 + j, KT - 1);
            xsb[j][t] = xs[(int64_t)mrow[t] * KB + 4 * kt + g];
          }
        }
      }
    } else {
      // row m's elements 512 kt4 + 8 lane .. + 7 (columns past K clamped; unused)
      const int col = min(512 * kt4 + 8 * lane, K - 8);
#pragma unroll
      for (int m = 0; m < 16; ++m)
        if (m < M) xr[m][0][0] = *(const v4i*)((const uint16_t*)xin + (int64_t)m * K + col);
    }
    __builtin_amdgcn_sched_barrier(0);
    // the group's weight scale word first: loads retire in order, so it is in by the time the
    // weight is
    const uint32_t sw = wsc[(int64_t)kt4 * NG * 64];
    v8i a[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int kt = min(4 * kt4 + j, KT - 1);
      const uint8_t* f = packed + ((int64_t)kt * NG + ng) * FB;
      const v4i lo = __builtin_nontemporal_load((const v4i*)(f + lane * 16));
      if (WFMT == 0) {
        const v4i hi = __builtin_nontemporal_load((const v4i*)(f + 1024 + lane * 16));
        a[j] = (v8i){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      } else {
        const v2i hi = __builtin_nontemporal_load((const v2i*)(f + 1024 + lane * 8));
        a[j] = (v8i){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], 0, 0};
      }
    }
    if (want_bias && bias8 && !have_bias) {
      braw = *(const v2i*)(bias + n);
      have_bias = true;
    }
    __builtin_amdgcn_sched_barrier(0);

    if constexpr (!QX) {
      // quantize rows m < M into the wave's LDS image: codes at [m][8 lane], the block scale
      // (one per quad of lanes) at [m][lane / 4]
      uint8_t* xw = xl[wave];
#pragma unroll
      for (int m = 0; m < 16; ++m) {
        if (m < M) {
          const v4i v = xr[m][0][0];
          const uint32_t e = scale_byte_from_amax<0>(quad_max_u32(amax8_bf16(v)));
          v2i q;
          if (e == 0xFFu) {
            q = (v2i){0x7F7F7F7F, 0x7F7F7F7F};   // block holds Inf/NaN: NaN codes
          } else {
            const float sc = e8m0_to_float(e);
            q = (v2i){(int)cvt4_e4m3((uint32_t)v[0], (uint32_t)v[1], sc),
                      (int)cvt4_e4m3((uint32_t)v[2], (uint32_t)v[3], sc)};
          }
          *(v2i*)(xw + m * kRowPitch + 8 * lane) = q;
          if ((lane & 3) == 0) sl[wave][m * 16 + (lane >> 2)] = (uint8_t)e;
        }
      }
      // the LDS image is written and read by this wave only: LDS operations of a wave complete
      // in order, so no barrier is needed
    }

#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (4 * kt4 + j < KT) {  // wave-uniform
#pragma unroll
        for (int t = 0; t < MT; ++t) {
          v8i b;
          uint32_t sb;
          if constexpr (QX) {
            const v4i lo = xr[j][t][0], hi = xr[j][t][1];
            b = (v8i){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            sb = XS16 ? (xsb[j][t] >> (8 * g)) & 0xFFu : xsb[j][t];
          } else {
            const uint8_t* p = xl[wave] + mrow[t] * kRowPitch + 128 * j + 16 * g;
            const v4i lo = *(const v4i*)p, hi = *(const v4i*)(p + 64);
            b = (v8i){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            sb = sl[wave][mrow[t] * 16 + 4 * j + g];
          }
          acc[t] = mfma_wsel<WFMT>(j, a[j], b, acc[t], sw, sb);
        }
      }
    }
  }

  float bv[4] = {0.f, 0.f, 0.f, 0.f};
  if (want_bias) {
    if (!have_bias && bias8) braw = *(const v2i*)(bias + n);   // a wave with no K group
    if (bias8) {
      bv[0] = bf16_to_float((uint32_t)braw[0] & 0xFFFFu);
      bv[1] = bf16_to_float((uint32_t)braw[0] >> 16);
      bv[2] = bf16_to_float((uint32_t)braw[1] & 0xFFFFu);
      bv[3] = bf16_to_float((uint32_t)braw[1] >> 16);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) bv[i] = bf16_to_float(bias[n + i]);
    }
  }

  // split-K reduction: partial sums of the 8 waves added in wave order
#pragma unroll
  for (int t = 0; t < MT; ++t) red[wave][t][lane] = acc[t];
  __syncthreads();
  if (wave < MT) {
    const int t = wave;
    v4f s = red[0][t][lane];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) s += red[w][t][lane];
    const int m = 16 * t + r;
    if (m < M) {
      const v2i o = {(int)pack_bf16x2(s[0] + bv[0], s[1] + bv[1]),
                     (int)pack_bf16x2(s[2] + bv[2], s[3] + bv[3])};
      *(v2i*)(y + (int64_t)m * N + n) = o;
    }
  }
}

bool small_m_fused(int64_t M, int64_t K) { return M >= 1 && M <= 16 && K % 128 == 0; }
bool small_m_quantized(int64_t M, int64_t K) { return M >= 1 && M <= 32 && K % 128 == 0; }

template <int WFMT>
static void launch_small(const void* x, const uint8_t* xs, bool quantized, int M, int K,
                         const uint8_t* packed, int N, const uint16_t* bias, uint16_t* y,
                         hipStream_t s, int batch, const BatchStrides& bs) {
  const dim3 grid((unsigned)(N / 16), (unsigned)batch), block(512);
  const bool xs16 = ((uintptr_t)xs & 15) == 0 && K % 512 == 0;   // then K / 32 % 16 == 0 too
  if (!quantized)
    hipLaunchKernelGGL((k_linear_small_m<WFMT, 1, false, false>), grid, block, 0, s, x, xs, M, K, packed, N, bias, y, bs);
  else if (M <= 16 && xs16)
    hipLaunchKernelGGL((k_linear_small_m<WFMT, 1, true, true>), grid, block, 0, s, x, xs, M, K, packed, N, bias, y, bs);
  else if (M <= 16)
    hipLaunchKernelGGL((k_linear_small_m<WFMT, 1, true, false>), grid, block, 0, s, x, xs, M, K, packed, N, bias, y, bs);
  else if (xs16)
    hipLaunchKernelGGL((k_linear_small_m<WFMT, 2, true, true>), grid, block, 0, s, x, xs, M, K, packed, N, bias, y, bs);
  else
    hipLaunchKernelGGL((k_linear_small_m<WFMT, 2, true, false>), grid, block, 0, s, x, xs, M, K, packed, N, bias, y, bs);
}

hipError_t launch_linear_small_m(const void* x, const uint8_t* xs, bool quantized, int64_t M,
                                 int64_t K, const uint8_t* packed, int64_t N, int fmt,
                                 const uint16_t* bias, uint16_t* y, hipStream_t s, int batch,
                                 BatchStrides bs) {
  if (quantized ? !small_m_quantized(M, K) : !small_m_fused(M, K)) return hipErrorInvalidValue;
  const int m = (int)M, k = (int)K, n = (int)N;
  switch (fmt) {
    case 0: launch_small<0>(x, xs, quantized, m, k, packed, n, bias, y, s, batch, bs); break;
    case 2: launch_small<2>(x, xs, quantized, m, k, packed, n, bias, y, s, batch, bs); break;
    case 3: launch_small<3>(x, xs, quantized, m, k, packed, n, bias, y, s, batch, bs); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace mx
