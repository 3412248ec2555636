// mx_device.h — device-side building blocks shared by the gfx950 kernels of this library.
//
// Hardware facts used here were measured on gfx950 with one-hot probes:
//  * v_mfma_scale_f32_16x16x128_f8f6f4, FP8 operand: lane l (row r = l % 16, group g = l / 16)
//    holds 32 bytes; byte t is K index 64 * (t / 16) + 16 * g + t % 16.  FP6 operand: lane l holds
//    the 32 values of K range [32 g, 32 g + 32) as 6-bit fields packed little-endian in 24 bytes.
//    The scale of MX block b (K range [32 b, 32 b + 32)) of row r is taken from lane r + 16 b;
//    the op-select argument picks which byte of that lane's 32-bit scale register is used.
//    The accumulator of lane l, element i, is C[4 * (l / 16) + i][l % 16].
//  * v_cvt_scalef32_pk_fp8_bf16 computes RNE(x / scale) into OCP E4M3 but does not saturate:
//    magnitudes that round above 448 become the NaN code S.1111.111.  Replacing that code by
//    S.1111.110 gives exactly the saturating conversion (checked over every finite bf16 and
//    every power-of-two scale).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mx {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v6i __attribute__((ext_vector_type(6)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v2i __attribute__((ext_vector_type(2)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef short v2s __attribute__((ext_vector_type(2)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));

// OCP MX element-format parameters (emax = exponent of the largest normal).
template <int FMT> struct Fmt;
template <> struct Fmt<0> { static constexpr int mbits = 3, emin = -6, emax = 8, maxcode = 0x7E, signbit = 7; static constexpr float maxval = 448.f; };
template <> struct Fmt<2> { static constexpr int mbits = 3, emin = 0, emax = 2, maxcode = 0x1F, signbit = 5; static constexpr float maxval = 7.5f; };
template <> struct Fmt<3> { static constexpr int mbits = 2, emin = -2, emax = 4, maxcode = 0x1F, signbit = 5; static constexpr float maxval = 28.f; };

// Bytes of one prepacked weight fragment (16 rows x 128 K) per element format.
__host__ __device__ constexpr int frag_bytes(int fmt) { return fmt == 0 ? 2048 : 1536; }

// E8M0 byte from the largest |bf16| bit pattern of a block (sign bit already cleared):
// floor(log2(amax)) = E - 127 for a normal amax with exponent field E, so the byte is
// max(E - emax, 0); zero and bf16-subnormal amax give 0 (scale 2^-127); Inf/NaN give 0xFF.
template <int FMT>
__device__ __forceinline__ uint32_t scale_byte_from_amax(uint32_t amax_bits) {
  if (amax_bits >= 0x7F80u) return 0xFFu;
  int e = (int)(amax_bits >> 7) - Fmt<FMT>::emax;
  return (uint32_t)(e > 0 ? e : 0);
}

// 2^(byte - 127) as an fp32 bit pattern (byte 0 is the subnormal 2^-127).
__device__ __forceinline__ float e8m0_to_float(uint32_t byte) {
  return __uint_as_float(byte ? (byte << 23) : 0x00400000u);
}

// The same value as e8m0_to_float for bytes 0 .. 254 in one instruction: 2^-127 (an fp32
// subnormal, kept since the kernels run with fp32 subnormals on) times 2^byte.
__device__ __forceinline__ float e8m0_to_float_ldexp(uint32_t byte) {
  return __builtin_ldexpf(__uint_as_float(0x00400000u), (int)byte);
}

// Four E4M3 codes (bytes of the result) from four bf16 values packed in two dwords, divided
// by `scale` (a power of two), round-to-nearest-even, saturated at +-448.
__device__ __forceinline__ uint32_t cvt4_e4m3(uint32_t bf_lo, uint32_t bf_hi, float scale) {
  v2bf a, b;
  __builtin_memcpy(&a, &bf_lo, 4);
  __builtin_memcpy(&b, &bf_hi, 4);
  v2s r = {0, 0};
  r = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(r, a, scale, false);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(r, b, scale, true);
  uint32_t u;
  __builtin_memcpy(&u, &r, 4);
  // bytes equal to 0x7F / 0xFF (overflow) -> 0x7E / 0xFE: add one to the low 7 bits, the
  // carry into bit 7 appears only for 0x7F; subtract it back as a 1 in that byte.
  uint32_t t = ((u & 0x7F7F7F7Fu) + 0x01010101u) & 0x80808080u;
  return u - (t >> 7);
}

// Exact element encode of an fp32 value (already divided by the block scale) for any format,
// nearest-even with saturation, sign kept.  Used by the load-time weight quantizer.
template <int FMT>
__device__ __forceinline__ uint32_t encode_elem(float v) {
  using F = Fmt<FMT>;
  const uint32_t s = __float_as_uint(v) >> 31;
  const float a = __builtin_fabsf(v);
  uint32_t mag;
  if (!(a < F::maxval)) {
    mag = F::maxcode;
  } else {
    int e = (int)(__float_as_uint(a) >> 23) - 127;      // floor(log2 a) for normal a
    if (e < F::emin) e = F::emin;                        // subnormal range of the format
    const float q = __builtin_rintf(__builtin_ldexpf(a, F::mbits - e));   // exact scaling
    mag = (uint32_t)((e - F::emin) << F::mbits) + (uint32_t)q;
  }
  return (s << F::signbit) | mag;
}

__device__ __forceinline__ float bf16_to_float(uint32_t b16) { return __uint_as_float(b16 << 16); }

// fp32 -> bf16 bits, round to nearest even (hardware conversion).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef float v2f __attribute__((ext_vector_type(2)));
  const v2bf b = __builtin_convertvector((v2f){lo, hi}, v2bf);   // one v_cvt_pk_bf16_f32
  uint32_t u;
  __builtin_memcpy(&u, &b, 4);
  return u;
}

// max over the 4 lanes of a quad (lanes 4j..4j+3), unsigned.
__device__ __forceinline__ uint32_t quad_max_u32(uint32_t v) {
  // quad_perm [1,0,3,2] then [2,3,0,1]
  uint32_t t = (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, true);
  v = v > t ? v : t;
  t = (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, true);
  return v > t ? v : t;
}

// largest |bf16| bit pattern (sign cleared) among the 8 values of a 16-byte piece
__device__ __forceinline__ uint32_t amax8_bf16(const v4i& v) {
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t u = (uint32_t)v[i] & 0x7FFF7FFFu;
    const uint32_t lo = u & 0xFFFFu, hi = u >> 16;
    m = m > lo ? m : lo;
    m = m > hi ? m : hi;
  }
  return m;
}

// The same as amax8_bf16 with the maxima taken two 16-bit fields at a time (v_pk_max_u16):
// |bf16| bit patterns compare as unsigned integers in the order of the magnitudes.
__device__ __forceinline__ uint32_t amax8_bf16_pk(const v4i& v) {
  typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
  u16x2 h[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t u = (uint32_t)v[i] & 0x7FFF7FFFu;
    __builtin_memcpy(&h[i], &u, 4);
  }
  const u16x2 m = __builtin_elementwise_max(__builtin_elementwise_max(h[0], h[1]),
                                            __builtin_elementwise_max(h[2], h[3]));
  return m[0] > m[1] ? (uint32_t)m[0] : (uint32_t)m[1];
}

// Eight E4M3 codes (two dwords) of the bf16 values of a 16-byte piece, divided by `scale`,
// RNE, saturated: cvt4_e4m3 twice.  The first convert of each dword writes its low half and
// the second its high half, so the register's previous contents never reach the result.
__device__ __forceinline__ v2i cvt8_e4m3(const v4i& v, float scale) {
  uint32_t u[2];
#pragma unroll
  for (int d = 0; d < 2; ++d) {
    const uint32_t lo = (uint32_t)v[2 * d], hi = (uint32_t)v[2 * d + 1];
    v2bf a, b;
    __builtin_memcpy(&a, &lo, 4);
    __builtin_memcpy(&b, &hi, 4);
    v2s r = __builtin_nondeterministic_value(r);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(r, a, scale, false);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(r, b, scale, true);
    __builtin_memcpy(&u[d], &r, 4);
    const uint32_t t = ((u[d] & 0x7F7F7F7Fu) + 0x01010101u) & 0x80808080u;
    u[d] -= t >> 7;
  }
  return (v2i){(int)u[0], (int)u[1]};
}

// ds_swizzle, bit-mask mode: lane i of each 32-lane half reads lane i ^ 16
__device__ __forceinline__ uint32_t lane_xor16(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, 0x401F);
}

// One 16-row activation tile of a 128-wide K step, quantized to E4M3 (OCP MX rule: the same
// codes and scales as k_quantize_act) straight in the scaled MFMA's B-operand layout.  Lane
// (r, g) = (lane % 16, lane / 16) brings row r's bf16 elements 16 g .. 16 g + 15 (xv[0], xv[1])
// and 64 + 16 g .. 64 + 16 g + 15 (xv[2], xv[3]): halves of MX blocks g / 2 and 2 + g / 2,
// whose other halves are in lane ^ 16.  Out: the lane's 32 operand bytes and the scale byte
// the MFMA reads from this lane, that of block g.
__device__ __forceinline__ void quantize_tile_operand_e4m3(const v4i (&xv)[4], int lane, v8i& b,
                                                           uint32_t& sb) {
  const int g = lane >> 4;
  uint32_t m0 = amax8_bf16(xv[0]), m1 = amax8_bf16(xv[2]);
  const uint32_t m0b = amax8_bf16(xv[1]), m1b = amax8_bf16(xv[3]);
  m0 = m0 > m0b ? m0 : m0b;
  m1 = m1 > m1b ? m1 : m1b;
  const uint32_t o0 = lane_xor16(m0), o1 = lane_xor16(m1);
  m0 = m0 > o0 ? m0 : o0;    // block g / 2
  m1 = m1 > o1 ? m1 : o1;    // block 2 + g / 2
  const uint32_t e0 = scale_byte_from_amax<0>(m0), e1 = scale_byte_from_amax<0>(m1);
  uint32_t q[8];
  if (e0 == 0xFFu) {
    q[0] = q[1] = q[2] = q[3] = 0x7F7F7F7Fu;   // block holds Inf/NaN: NaN codes
  } else {
    const float sc = e8m0_to_float(e0);
    q[0] = cvt4_e4m3((uint32_t)xv[0][0], (uint32_t)xv[0][1], sc);
    q[1] = cvt4_e4m3((uint32_t)xv[0][2], (uint32_t)xv[0][3], sc);
    q[2] = cvt4_e4m3((uint32_t)xv[1][0], (uint32_t)xv[1][1], sc);
    q[3] = cvt4_e4m3((uint32_t)xv[1][2], (uint32_t)xv[1][3], sc);
  }
  if (e1 == 0xFFu) {
    q[4] = q[5] = q[6] = q[7] = 0x7F7F7F7Fu;
  } else {
    const float sc = e8m0_to_float(e1);
    q[4] = cvt4_e4m3((uint32_t)xv[2][0], (uint32_t)xv[2][1], sc);
    q[5] = cvt4_e4m3((uint32_t)xv[2][2], (uint32_t)xv[2][3], sc);
    q[6] = cvt4_e4m3((uint32_t)xv[3][0], (uint32_t)xv[3][1], sc);
    q[7] = cvt4_e4m3((uint32_t)xv[3][2], (uint32_t)xv[3][3], sc);
  }
  b = (v8i){(int)q[0], (int)q[1], (int)q[2], (int)q[3], (int)q[4], (int)q[5], (int)q[6], (int)q[7]};
  // the MFMA takes block g's scale from this lane: g = 0 and 3 computed it (e0 of block 0, e1
  // of block 3); block 1 sits in e0 of g = 2 and block 2 in e1 of g = 1 (lane ^ 48)
  const uint32_t give = g == 1 ? e1 : e0;
  const uint32_t got = (uint32_t)__builtin_amdgcn_ds_bpermute((lane ^ 48) << 2, (int)give);
  sb = g == 0 ? e0 : (g == 3 ? e1 : got);
}

template <int AFMT, int BFMT>
__device__ __forceinline__ v4f mfma16(const v8i& a, const v8i& b, v4f c, int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, AFMT, BFMT, 0, sa, 0, sb);
}

}  // namespace mx
