// mx_quant.hip — MX quantizers for gfx950.
//
// Activations (hot path): bf16 [M, K] -> E4M3 [M, K] + E8M0 [M, K/32], both row-major, as the
// aiter_flydsl page's apply_weights produces them before the GEMM.  HBM-bound: each thread
// reads 16 bytes (8 bf16) and writes 8 code bytes, so a wavefront moves 1 KiB in and 512 B out
// in single coalesced instructions; the 32-element block maximum is a 4-lane DPP reduction
// inside a quad, and the conversion is the hardware scaled E4M3 convert with the overflow code
// mapped to the saturated one.  The bf16 input is read with non-temporal loads:
// it is read once, and left in the caches it would displace the codes and the weight that the
// GEMM reads next (the prefill step measured 5 % faster).
//
// MXFP6 activations (the mxfp6 page's activation_quant_key): one lane per block, hardware
// scaled FP6 conversion.
//
// Weights (load time): any element format, one thread per 32-element block, exact float
// arithmetic per element (speed is irrelevant there; exactness is checked against the oracle).
#include "mx_device.h"
#include "mx_launch.h"

namespace mx {

// One thread per 8 consecutive elements of a row; 4 consecutive threads form one MX block.
// groups = M * K / 8; the quad of a block never straddles two rows because K % 32 == 0.
__global__ __launch_bounds__(256) void k_quantize_act(const uint16_t* __restrict__ x, int64_t K,
                                                      int64_t ldx, int64_t groups,
                                                      uint8_t* __restrict__ xq,
                                                      uint8_t* __restrict__ xs) {
  const int64_t kg = K >> 3;  // groups of 8 per row
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  // every lane of a wave runs the same number of iterations (groups is a multiple of 4 and
  // the quad reduction only needs the 4 lanes of a block to be active together)
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t - (threadIdx.x & 63) < groups;
       t += stride) {
    const bool live = t < groups;
    const int64_t row = live ? t / kg : 0;
    const int64_t c8 = live ? t - row * kg : 0;
    v4i v = {0, 0, 0, 0};
    if (live) v = __builtin_nontemporal_load((const v4i*)(x + row * ldx + c8 * 8));
    const uint32_t m = quad_max_u32(amax8_bf16(v));
    const uint32_t byte = scale_byte_from_amax<0>(m);
    uint32_t q0, q1;
    if (byte == 0xFFu) {
      q0 = q1 = 0x7F7F7F7Fu;  // block holds Inf/NaN: NaN codes
    } else {
      const float sc = e8m0_to_float(byte);
      q0 = cvt4_e4m3((uint32_t)v[0], (uint32_t)v[1], sc);
      q1 = cvt4_e4m3((uint32_t)v[2], (uint32_t)v[3], sc);
    }
    if (live) {
      v2i o = {(int)q0, (int)q1};
      *(v2i*)(xq + row * K + c8 * 8) = o;
      if ((c8 & 3) == 0) xs[row * (K >> 5) + (c8 >> 2)] = (uint8_t)byte;
    }
  }
}

hipError_t launch_quantize_act(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, uint8_t* xq,
                               uint8_t* xs, hipStream_t s) {
  const int64_t groups = M * (K >> 3);
  int64_t blocks = (groups + 255) / 256;
  if (blocks > 256 * 16) blocks = 256 * 16;  // grid-stride beyond 16 workgroups per CU
  hipLaunchKernelGGL(k_quantize_act, dim3((unsigned)blocks), dim3(256), 0, s, x, K, ldx, groups,
                     xq, xs);
  return hipGetLastError();
}

// ---------------------------------------------------------------- activations, MXFP6
// One lane per MX block: 64 bytes of bf16 in (four 16-byte loads), 24 bytes of packed 6-bit codes
// and the scale byte out.  The scale follows the format's emax (E2M3: 2, E3M2: 4); the codes
// come from the hardware scaled conversion (v_cvt_scalef32_pk32_{fp6,bf6}_bf16), which gives
// RNE(x / scale) saturated at the format maximum, sign kept, packed little-endian in 6-bit
// fields: the same bits as the exact per-element encode for every finite bf16 and every scale
// byte.  A block holding Inf/NaN gets scale 0xFF and zero codes (FP6 has no NaN).
// xstep 96: rows of packed codes; 128: block kb's 24 bytes at 128 (kb / 4) + 24 (kb % 4) of its row
// (K % 128 == 0), so that every K step's 96 bytes start a 128-byte line for the GEMM's copies.
template <int FMT>
__global__ __launch_bounds__(256) void k_quantize_act_fp6(const uint16_t* __restrict__ x, int64_t K,
                                                          int64_t ldx, int64_t blocks,
                                                          uint8_t* __restrict__ xq,
                                                          uint8_t* __restrict__ xs, int xstep) {
  typedef __bf16 v32bf __attribute__((ext_vector_type(32)));
  const int64_t KB = K >> 5;
  const int64_t ldq = xstep == 96 ? KB * 24 : (KB >> 2) * xstep;
  for (int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; b < blocks;
       b += (int64_t)gridDim.x * blockDim.x) {
    const int64_t row = b / KB, kb = b - row * KB;
    const uint16_t* src = x + row * ldx + kb * 32;
    v4i v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = __builtin_nontemporal_load((const v4i*)(src + 8 * i));
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t a = amax8_bf16(v[i]);
      m = m > a ? m : a;
    }
    const uint32_t byte = scale_byte_from_amax<FMT>(m);
    v6i q = {0, 0, 0, 0, 0, 0};
    if (byte != 0xFFu) {
      v32bf xv;
      __builtin_memcpy(&xv, v, 64);
      const float sc = e8m0_to_float(byte);
      if constexpr (FMT == 2) q = __builtin_amdgcn_cvt_scalef32_pk32_fp6_bf16(xv, sc);
      else q = __builtin_amdgcn_cvt_scalef32_pk32_bf6_bf16(xv, sc);
    }
    uint8_t* dst = xq + row * ldq + (xstep == 96 ? kb * 24 : (kb >> 2) * xstep + (kb & 3) * 24);
    *(v2i*)dst = (v2i){q[0], q[1]};
    *(v2i*)(dst + 8) = (v2i){q[2], q[3]};
    *(v2i*)(dst + 16) = (v2i){q[4], q[5]};
    xs[row * KB + kb] = (uint8_t)byte;
  }
}

hipError_t launch_quantize_act_fp6(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, int fmt,
                                   uint8_t* xq, uint8_t* xs, hipStream_t s, int xstep) {
  if (xstep != 96 && (xstep != 128 || K % 128 != 0)) return hipErrorInvalidValue;
  const int64_t blocks = M * (K >> 5);
  int64_t grid = (blocks + 255) / 256;
  if (grid > 256 * 16) grid = 256 * 16;
  switch (fmt) {
    case 2: hipLaunchKernelGGL(k_quantize_act_fp6<2>, dim3((unsigned)grid), dim3(256), 0, s, x, K, ldx, blocks, xq, xs, xstep); break;
    case 3: hipLaunchKernelGGL(k_quantize_act_fp6<3>, dim3((unsigned)grid), dim3(256), 0, s, x, K, ldx, blocks, xq, xs, xstep); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------- fused producer: RMS norm
// The producer of a pre-quantized activation (the Mxfp8LinearKernel page's input_quant_key lets
// a layer take activations quantized outside it): r = 1 / sqrt(mean(x^2) + eps) in fp64, rounded
// once to fp32; y = bf16(bf16(fp32(x r)) gamma); then y quantized as k_quantize_act does.
// Pass 1: sum of squares in fp64 (a fixed order, every lane ending with the same bits).  Pass 2:
// the two products in fp32 (x r is one rounding; t gamma is exact), each rounded to bf16 by the
// hardware convert (RNE).

// fp64 sum of a value over the 64 lanes of a wave by DPP moves (each 64-bit step as two 32-bit
// halves): quad, half-row and row partners, then rows 0 -> 1 and 2 -> 3 and row 1 -> rows 2, 3;
// lane 63 ends with the total, which every lane reads back.  Rows left out of a step add +0.
template <int CTRL, int ROWS>
__device__ __forceinline__ double dpp_add_f64(double x) {
  const uint64_t u = __builtin_bit_cast(uint64_t, x);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)u, CTRL, ROWS, 0xF, false);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(u >> 32), CTRL, ROWS, 0xF, false);
  return x + __builtin_bit_cast(double, (uint64_t)hi << 32 | lo);
}
__device__ __forceinline__ double wave_sum_f64(double v) {
  v = dpp_add_f64<0xB1, 0xF>(v);    // quad_perm [1, 0, 3, 2]
  v = dpp_add_f64<0x4E, 0xF>(v);    // quad_perm [2, 3, 0, 1]
  v = dpp_add_f64<0x141, 0xF>(v);   // row_half_mirror: the other quad of the half-row
  v = dpp_add_f64<0x140, 0xF>(v);   // row_mirror: the other half of the row
  v = dpp_add_f64<0x142, 0xA>(v);   // row_bcast15: row 0's sum into row 1, row 2's into row 3
  v = dpp_add_f64<0x143, 0xC>(v);   // row_bcast31: rows 0 + 1 into rows 2 and 3
  const uint64_t u = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)u, 63);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), 63);
  return __builtin_bit_cast(double, (uint64_t)hi << 32 | lo);
}

// One row per workgroup of WPR waves; lane L = 64 h + lane of wave h takes columns
// 512 WPR c + 8 L .. + 7 of pass c.  CH > 0: the row (K <= 512 WPR CH) is loaded once, all
// chunks in flight together, and kept in registers for the second pass; CH == 0: any K, chunk
// by chunk, re-read in the second pass.  The sum of squares: four fp64 partial sums per lane,
// a fixed DPP tree per wave (wave_sum_f64), then the waves' sums added in wave order.  The sum
// of bf16 squares in fp64 is exact for rows whose squares span under 2^25 of magnitude (16-bit
// significands, at most 2^12 terms in 53 bits), so there the order gives the oracle's bits.
template <int CH, int WPR>
__global__ __launch_bounds__(64 * WPR) void k_rmsnorm_quant(const uint16_t* __restrict__ x, int M,
                                                            int K, int64_t ldx,
                                                            const uint16_t* __restrict__ gamma,
                                                            double eps, uint8_t* __restrict__ xq,
                                                            uint8_t* __restrict__ xs,
                                                            uint16_t* __restrict__ yout) {
  __shared__ double part[WPR];
  const int lane = threadIdx.x & 63, h = threadIdx.x >> 6;
  const int L = 64 * h + lane;
  constexpr int SPAN = 512 * WPR;
  const int row = blockIdx.x;
  const uint16_t* xr = x + (int64_t)row * ldx;
  const int chunks = CH > 0 ? CH : (K + SPAN - 1) / SPAN;
  constexpr int RC = CH > 0 ? CH : 1;
  v4i xv[RC];
  if constexpr (CH > 0) {
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int col = SPAN * c + 8 * L;
      xv[c] = col < K ? __builtin_nontemporal_load((const v4i*)(xr + col)) : (v4i){0, 0, 0, 0};
    }
  }
  double s4[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll RC
  for (int c = 0; c < chunks; ++c) {
    const int col = SPAN * c + 8 * L;
    v4i v = {0, 0, 0, 0};
    if constexpr (CH > 0) v = xv[c];
    else if (col < K) v = __builtin_nontemporal_load((const v4i*)(xr + col));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const double lo = (double)bf16_to_float((uint32_t)v[i] & 0xFFFFu);
      const double hi = (double)bf16_to_float((uint32_t)v[i] >> 16);
      s4[i] = __builtin_fma(lo, lo, s4[i]);
      s4[i] = __builtin_fma(hi, hi, s4[i]);
    }
  }
  double ss = (s4[0] + s4[1]) + (s4[2] + s4[3]);
  ss = wave_sum_f64(ss);
  if constexpr (WPR > 1) {
    if (lane == 0) part[h] = ss;
    __syncthreads();
    ss = part[0];
#pragma unroll
    for (int w = 1; w < WPR; ++w) ss += part[w];
  }
  const double r = 1.0 / __builtin_sqrt(ss / (double)K + eps);
  const float r32 = (float)r;
  const int KB = K >> 5;
#pragma unroll RC
  for (int c = 0; c < chunks; ++c) {
    // every lane runs every chunk (the quad reduction needs whole quads); lanes past K work on
    // a clamped column and store nothing
    const int col = SPAN * c + 8 * L;
    const bool live = col < K;
    const int cc = live ? col : K - 8;
    v4i v;
    if constexpr (CH > 0) v = xv[c];
    else v = *(const v4i*)(xr + cc);
    const v4i gw = *(const v4i*)(gamma + cc);
    v4i y8;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t w = (uint32_t)v[i], gq = (uint32_t)gw[i];
      const uint32_t t = pack_bf16x2(__uint_as_float(w << 16) * r32,
                                     __uint_as_float(w & 0xFFFF0000u) * r32);
      y8[i] = (int)pack_bf16x2(__uint_as_float(t << 16) * __uint_as_float(gq << 16),
                               __uint_as_float(t & 0xFFFF0000u) * __uint_as_float(gq & 0xFFFF0000u));
    }
    // the MX quantization of y: packed 16-bit amax, the scale as one ldexp, converted whatever
    // the scale (branch-free), an Inf/NaN block's codes replaced by NaN codes
    const uint32_t byte = scale_byte_from_amax<0>(quad_max_u32(amax8_bf16_pk(y8)));
    v2i q = cvt8_e4m3(y8, e8m0_to_float_ldexp(byte));
    if (byte == 0xFFu) q = (v2i){0x7F7F7F7F, 0x7F7F7F7F};
    if (live) {
      *(v2i*)(xq + (int64_t)row * K + col) = q;
      if ((lane & 3) == 0) xs[(int64_t)row * KB + (col >> 5)] = (uint8_t)byte;
      if (yout) *(v4i*)(yout + (int64_t)row * K + col) = y8;
    }
  }
}

template <int WPR>
static void launch_rms(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, const uint16_t* gamma,
                       float eps, uint8_t* xq, uint8_t* xs, uint16_t* y, hipStream_t s) {
  const dim3 grid((unsigned)M), block(64 * WPR);
  if (K <= 4096)
    hipLaunchKernelGGL((k_rmsnorm_quant<8 / WPR, WPR>), grid, block, 0, s, x, (int)M, (int)K, ldx, gamma, (double)eps, xq, xs, y);
  else if (K <= 8192)
    hipLaunchKernelGGL((k_rmsnorm_quant<16 / WPR, WPR>), grid, block, 0, s, x, (int)M, (int)K, ldx, gamma, (double)eps, xq, xs, y);
  else
    hipLaunchKernelGGL((k_rmsnorm_quant<0, WPR>), grid, block, 0, s, x, (int)M, (int)K, ldx, gamma, (double)eps, xq, xs, y);
}

hipError_t launch_rmsnorm_quant(const uint16_t* x, int64_t M, int64_t K, int64_t ldx,
                                const uint16_t* gamma, float eps, uint8_t* xq, uint8_t* xs,
                                uint16_t* y, hipStream_t s) {
  if (M == 0) return hipSuccess;
  // about 16 elements per lane: more waves in flight hide the load latency and the serial
  // per-row work (measured on 4096 x 4096: 15.3 us with 4 waves per row, 18.6 us with one)
  if (K <= 4096) launch_rms<4>(x, M, K, ldx, gamma, eps, xq, xs, y, s);
  else launch_rms<8>(x, M, K, ldx, gamma, eps, xq, xs, y, s);
  return hipGetLastError();
}

// ---------------------------------------------------------------- weights, any format

template <int FMT>
__global__ __launch_bounds__(256) void k_quantize_weight(const uint16_t* __restrict__ w, int64_t N,
                                                         int64_t K, int64_t ldw,
                                                         uint8_t* __restrict__ wq,
                                                         uint8_t* __restrict__ ws) {
  const int64_t KB = K >> 5;
  const int64_t nblk = N * KB;
  for (int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; b < nblk;
       b += (int64_t)gridDim.x * blockDim.x) {
    const int64_t row = b / KB, kb = b - row * KB;
    const uint16_t* src = w + row * ldw + kb * 32;
    uint32_t m = 0;
    for (int j = 0; j < 32; ++j) {
      const uint32_t u = src[j] & 0x7FFFu;
      m = m > u ? m : u;
    }
    const uint32_t byte = scale_byte_from_amax<FMT>(m);
    ws[row * KB + kb] = (uint8_t)byte;
    uint32_t codes[32];
    for (int j = 0; j < 32; ++j) {
      if (byte == 0xFFu) {
        codes[j] = FMT == 0 ? 0x7Fu : 0u;
      } else {
        // x / 2^(byte - 127), exact for every result that can round to a nonzero code
        const float v = __builtin_ldexpf(bf16_to_float(src[j]), 127 - (int)byte);
        codes[j] = encode_elem<FMT>(v);
      }
    }
    if (FMT == 0) {
      uint8_t* dst = wq + row * K + kb * 32;
      for (int j = 0; j < 32; ++j) dst[j] = (uint8_t)codes[j];
    } else {
      uint8_t* dst = wq + row * (K / 4 * 3) + kb * 24;
      for (int g = 0; g < 8; ++g) {
        const uint32_t w24 = codes[4 * g] | codes[4 * g + 1] << 6 | codes[4 * g + 2] << 12 |
                             codes[4 * g + 3] << 18;
        dst[3 * g] = (uint8_t)(w24 & 0xFF);
        dst[3 * g + 1] = (uint8_t)((w24 >> 8) & 0xFF);
        dst[3 * g + 2] = (uint8_t)(w24 >> 16);
      }
    }
  }
}

hipError_t launch_quantize_weight(const uint16_t* w, int64_t N, int64_t K, int64_t ldw, int fmt,
                                  uint8_t* wq, uint8_t* ws, hipStream_t s) {
  const int64_t nblk = N * (K >> 5);
  int64_t blocks = (nblk + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  dim3 grid((unsigned)blocks), block(256);
  switch (fmt) {
    case 0: hipLaunchKernelGGL(k_quantize_weight<0>, grid, block, 0, s, w, N, K, ldw, wq, ws); break;
    case 2: hipLaunchKernelGGL(k_quantize_weight<2>, grid, block, 0, s, w, N, K, ldw, wq, ws); break;
    case 3: hipLaunchKernelGGL(k_quantize_weight<3>, grid, block, 0, s, w, N, K, ldw, wq, ws); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace mx
