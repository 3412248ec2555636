// mx_prepack.hip — load-time weight rearrangement into MFMA register order, and its inverse.
//
// The aiter_flydsl page rearranges weights once at load (process_weights_after_loading) and
// gives the inverse for readers of row-major weights (row_major_weight).  The layout below is
// this library's own, chosen for gfx950's scaled MFMA (16x16x128, weight as the A operand):
//
//   weight region: fragment f(kt, ng) = 16 rows (16 ng .. 16 ng + 15) x 128 K (128 kt ..),
//     at byte offset (kt * NG + ng) * frag, K zero-padded to a multiple of 128.
//     E4M3 (frag = 2048): [half h][lane l][16 B], lane l = (row r = l % 16, group g = l / 16)
//       holds W[r][128 kt + 64 h + 16 g + j], j < 16 — the two 16-byte halves of the MFMA's
//       A-register of lane l, so one 16-byte load per lane per half, 1 KiB contiguous per wave.
//     FP6 (frag = 1536): [lane][16 B] then [lane][8 B]: lane l holds the 24 packed bytes of
//       MX block 4 kt + g of row r, split 16 + 8 (the register image of the FP6 A operand).
//   scale region (after the weights): 32-bit word per (kt / 4, ng, lane), byte kt % 4 =
//     E8M0 scale of (row 16 ng + l % 16, block 4 kt + l / 16) — the scale each lane feeds the
//     MFMA; padded blocks get 127 (1.0), never the NaN byte.
#include "mx_device.h"
#include "mx_launch.h"

namespace mx {

PackGeom pack_geom(int64_t N, int64_t K, int fmt) {
  PackGeom p;
  p.N = N;
  p.K = K;
  p.NG = N / 16;
  p.KT = (K + 127) / 128;
  p.KT4 = (p.KT + 3) / 4;
  p.frag = frag_bytes(fmt);
  p.wbytes = p.KT * p.NG * p.frag;
  p.sbytes = p.KT4 * p.NG * 256;
  return p;
}

// Byte offset of W[row][k] in the source (PACK) or destination (unpack) weight:
//   row-major with row stride ldw, or (SHUF) the aiter_flydsl page's (16, 16) preshuffled E4M3
//   layout, which stores the logical [N/16, 16, K/32, 2, 16] array as [N/16, K/32, 2, 16, 16]
//   (aiter_flydsl page, row_major_weight).
template <bool SHUF>
__device__ __forceinline__ int64_t w_offset(int64_t row, int64_t k, int64_t ldw, int64_t KB) {
  if (!SHUF) return row * ldw + k;
  return ((((row >> 4) * KB + (k >> 5)) * 2 + ((k >> 4) & 1)) * 16 + (row & 15)) * 16 + (k & 15);
}

// one thread per (fragment, lane); byte-granular copies (load-time only, any stride)
template <int FMT, bool PACK, bool SHUF = false>
__global__ __launch_bounds__(256) void k_pack(uint8_t* __restrict__ wq, int64_t ldw,
                                              uint8_t* __restrict__ ws, int64_t ld_ws, int64_t N,
                                              int64_t K, uint8_t* __restrict__ packed) {
  const int64_t NG = N / 16, KT = (K + 127) / 128, KB = K / 32;
  const int64_t frag = frag_bytes(FMT);
  const int64_t total = KT * NG * 64;
  uint8_t* sreg = packed + KT * NG * frag;
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < total;
       t += (int64_t)gridDim.x * blockDim.x) {
    const int64_t f = t >> 6;
    const int l = (int)(t & 63), r = l & 15, g = l >> 4;
    const int64_t kt = f / NG, ng = f - kt * NG;
    const int64_t row = 16 * ng + r;
    uint8_t* fr = packed + f * frag;
    if (FMT == 0) {
      for (int h = 0; h < 2; ++h) {
        const int64_t k = 128 * kt + 64 * h + 16 * g;
        uint8_t* d = fr + h * 1024 + l * 16;
        for (int j = 0; j < 16; ++j) {
          if (PACK) d[j] = (k + j < K) ? wq[w_offset<SHUF>(row, k + j, ldw, KB)] : 0;
          else if (k + j < K) wq[w_offset<SHUF>(row, k + j, ldw, KB)] = d[j];
        }
      }
    } else {
      const int64_t kb = 4 * kt + g;
      for (int j = 0; j < 24; ++j) {
        uint8_t* d = j < 16 ? fr + l * 16 + j : fr + 1024 + l * 8 + (j - 16);
        if (PACK) d[0] = (kb < KB) ? wq[row * ldw + kb * 24 + j] : 0;
        else if (kb < KB) wq[row * ldw + kb * 24 + j] = d[0];
      }
    }
    // scale byte of this lane
    const int64_t kb = 4 * kt + g;
    uint8_t* sd = sreg + ((kt >> 2) * NG + ng) * 256 + l * 4 + (kt & 3);
    if (PACK) sd[0] = (kb < KB) ? ws[row * ld_ws + kb] : 127;
    else if (kb < KB) ws[row * ld_ws + kb] = sd[0];
  }
}

// the unused bytes of a partially filled last scale word (KT % 4 != 0) are set to 127 too
__global__ void k_pack_scale_tail(uint8_t* __restrict__ sreg, int64_t NG, int64_t KT) {
  const int64_t KT4 = (KT + 3) / 4;
  const int64_t total = NG * 256;
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < total;
       t += (int64_t)gridDim.x * blockDim.x) {
    if ((int64_t)((t & 3)) >= KT - 4 * (KT4 - 1)) sreg[(KT4 - 1) * NG * 256 + t] = 127;
  }
}

template <bool PACK, bool SHUF = false>
static hipError_t launch_pack(const uint8_t* wq, int64_t ldw, const uint8_t* ws, int64_t ld_ws,
                              int64_t N, int64_t K, int fmt, uint8_t* packed, hipStream_t s) {
  const PackGeom p = pack_geom(N, K, fmt);
  const int64_t total = p.KT * p.NG * 64;
  int64_t blocks = (total + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  dim3 grid((unsigned)blocks), block(256);
  uint8_t* w = const_cast<uint8_t*>(wq);
  uint8_t* sc = const_cast<uint8_t*>(ws);
  if (SHUF) {   // the preshuffled layout is defined for 1-byte (E4M3) elements only
    if (fmt != 0) return hipErrorInvalidValue;
    hipLaunchKernelGGL((k_pack<0, PACK, true>), grid, block, 0, s, w, ldw, sc, ld_ws, N, K, packed);
  } else {
    switch (fmt) {
      case 0: hipLaunchKernelGGL((k_pack<0, PACK>), grid, block, 0, s, w, ldw, sc, ld_ws, N, K, packed); break;
      case 2: hipLaunchKernelGGL((k_pack<2, PACK>), grid, block, 0, s, w, ldw, sc, ld_ws, N, K, packed); break;
      case 3: hipLaunchKernelGGL((k_pack<3, PACK>), grid, block, 0, s, w, ldw, sc, ld_ws, N, K, packed); break;
      default: return hipErrorInvalidValue;
    }
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (PACK && (p.KT & 3)) {
    int64_t b2 = (p.NG * 256 + 255) / 256;
    if (b2 > 4096) b2 = 4096;
    hipLaunchKernelGGL(k_pack_scale_tail, dim3((unsigned)b2), dim3(256), 0, s, packed + p.wbytes,
                       p.NG, p.KT);
    e = hipGetLastError();
  }
  return e;
}

hipError_t launch_prepack(const uint8_t* wq, int64_t ldw, const uint8_t* ws, int64_t ld_ws,
                          int64_t N, int64_t K, int fmt, uint8_t* packed, hipStream_t s) {
  return launch_pack<true>(wq, ldw, ws, ld_ws, N, K, fmt, packed, s);
}

hipError_t launch_unpack(const uint8_t* packed, int64_t N, int64_t K, int fmt, uint8_t* wq,
                         uint8_t* ws, hipStream_t s) {
  const int64_t ldw = fmt == 0 ? K : K / 4 * 3;
  return launch_pack<false>(wq, ldw, ws, K / 32, N, K, fmt, const_cast<uint8_t*>(packed), s);
}

hipError_t launch_prepack_shuffled16(const uint8_t* w16, const uint8_t* ws, int64_t ld_ws,
                                     int64_t N, int64_t K, uint8_t* packed, hipStream_t s) {
  return launch_pack<true, true>(w16, K, ws, ld_ws, N, K, 0, packed, s);
}

hipError_t launch_unpack_shuffled16(const uint8_t* packed, int64_t N, int64_t K, uint8_t* w16,
                                    uint8_t* ws, hipStream_t s) {
  return launch_pack<false, true>(w16, K, ws, K / 32, N, K, 0, const_cast<uint8_t*>(packed), s);
}

}  // namespace mx
