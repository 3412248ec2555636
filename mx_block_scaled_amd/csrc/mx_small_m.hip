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
// Activations come either as bf16 (quantized inside the kernel, bit-identical to
// k_quantize_act) or pre-quantized (E4M3 xq + row-major E8M0 xs, M <= 32).  For the bf16 entry
// k_linear_small_m_rs below (up to 16 rows with K <= 8192, 32 with K <= 4096) puts the
// quantizer and the weight stream in different waves; this kernel keeps the other bf16 shapes
// (M <= 16 with a larger K) and the pre-quantized entry.
//
// The fused quantizer works on the natural row-major layout, where it is cheapest: lane l
// quantizes elements 8 l .. 8 l + 7 of a row's 512-wide group slice (a quad of lanes is one MX
// block, reduced with DPP), writes the codes to a wave-private LDS image, and the MFMA operands
// are then read back from LDS in the operand layout.  Working directly in the operand layout
// would quantize 16 rows per wave whatever M is.
//
// Above the role-split kernel's rows (bf16 entry), k_linear_decode_sk below also splits K
// across workgroups, so that each workgroup reads and quantizes only a part of the
// activations; there the operand layout is the cheaper place to quantize.
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
          const uint32_t e = scale_byte_from_amax<0>(quad_max_u32(amax8_bf16_pk(v)));
          // converted whatever e is (branch-free); a block holding Inf/NaN gets NaN codes
          v2i q = cvt8_e4m3(v, e8m0_to_float_ldexp(e));
          if (e == 0xFFu) q = (v2i){0x7F7F7F7F, 0x7F7F7F7F};
          *(v2i*)(xw + m * kRowPitch + 8 * lane) = q;
          // the four lanes of the block store the same byte
          sl[wave][m * 16 + (lane >> 2)] = (uint8_t)e;
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

// ---------------------------------------------------------------------------------------------
// Small M, bf16 entry, with the waves of a workgroup in two roles (up to 32 rows, K <= KMAX).
// A wave that issues a long run of loads stalls once the CU's memory pipeline is full, and a
// wave issues in order: in k_linear_small_m each wave's quantizer therefore starts only after
// its last weight load has gone out, 1-3 us into the call at M = 8 (per-wave clock stamps),
// and the quantizer's VALU time then adds to the call instead of hiding under the weight
// stream.  Here:
//  * waves 0-7 load the activation rows and quantize them (row-major, as k_linear_small_m)
//    into an LDS image of the whole [rows, K] block of codes and scales (K groups q, q + 8, ..);
//  * the next NW = 4 (8 with four fragments per workgroup) waves issue the weight stream of all
//    their K groups (w, w + NW, ..; up to 16 fragments of 2 KiB each, all in registers) and
//    wait at one barrier for the image;
//  * then those waves run the MFMAs, B operands and scales read from the image;
//  * their NW partials are added in wave order, then bias, one bf16 rounding, store.
// A workgroup computes F weight fragments (16 F output columns).  With F > 1 the rows are split
// into tiles of RT rows, one workgroup per (column group, row tile): each workgroup then quantizes
// only its own rows, so the quantizer's VALU time per workgroup stays that of one tile while
// the row tiles of a column group read the same weight bytes (placed on one XCD, so the second
// read comes from its L2).  Every output is the same sum in the same order whatever the tiling.
// Same codes and scales as k_quantize_act, so the same operands as every other path; the sum
// over K runs in a different order than k_linear_small_m's (within the tolerance of any split).
// NQ quantizer waves (4 or 8), MT 16-row activation tiles, F weight fragments, code image for
// K <= KMAX
// The weight waves come in sets of four; set s takes fragments s FPW .. s FPW + FPW - 1, and its
// wave l the K groups l, l + 4, .. of them, so every output is the same 4-way split of K, added
// in wave order, whatever F is (one set for F <= 2, two for F = 4).
template <int NQ, int MT, int F, int KMAX>
struct RsCfg {
  static constexpr int NW = F >= 4 ? 8 : 4;                // weight (MFMA) waves
  static constexpr int SETS = NW / 4;                      // sets of four weight waves
  static constexpr int FPW = F / SETS;                     // fragments per weight wave
  static constexpr int ROWS = 16 * MT;
  static constexpr int PITCH = KMAX + 16;                  // code row pitch (max); +16 B: banks
  static constexpr int GMAX = KMAX / 512 / 4;              // weight groups per weight wave
  static constexpr int QMAX = KMAX / 512 / NQ;             // K groups per quantizer wave
  static constexpr int PAIRS = MT * F;                     // (row tile, fragment) outputs
  static constexpr int LDS = ROWS * PITCH + ROWS * (KMAX / 32) + NW * MT * FPW * 64 * 16;
  static_assert(LDS <= 160 * 1024, "must fit the 160 KiB LDS");
  static_assert(FPW * SETS == F && GMAX >= 1 && GMAX * 4 * FPW <= 16,
                "weight fragments held in registers per wave");
  static_assert(PAIRS <= NW, "one weight wave finishes each output pair");
};

// s_waitcnt lgkmcnt(0), then the workgroup barrier; the empty assembly statements keep the
// compiler from moving LDS accesses across it
__device__ __forceinline__ void rs_lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0), vmcnt / expcnt not waited for
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Workgroup blockIdx.x -> (column group c, row tile t) for R row tiles of G column groups.
// Workgroups are dealt to the 8 XCDs in turn (workgroup i to XCD i mod 8), so with G a
// multiple of 8 the R tiles of a column group are given indices of one residue mod 8, and
// their shared weight bytes meet in one L2.  Any order computes the same outputs.
__device__ __forceinline__ void rs_tile_of(int i, int G, int R, int& c, int& t) {
  if (R == 1) {
    c = i;
    t = 0;
  } else if ((G & 7) == 0) {
    const int j = i >> 3;
    c = 8 * (j / R) + (i & 7);
    t = j % R;
  } else {
    c = i / R;
    t = i % R;
  }
}

// QR: rows quantized per workgroup, >= the rows of its tile (rows past the tile repeat its
// last row; they are never read), so that the row loops have no branches.  RT: rows per row
// tile (used with F > 1; with F == 1 the workgroup takes all M rows).
// SEQ (batch-invariant mode): weight wave w holds the contiguous K groups [w GPW, w GPW + GPW)
// instead of w, w + NW, .., and the waves extend one accumulator chain in turn (wave w starts
// from wave w - 1's sums, passed through LDS) instead of adding partials: every output then
// takes its K steps in order, one MFMA each, from a zero start, exactly as the tiled and
// generic GEMM kernels do, so its bits do not depend on M or on the kernel.
template <int WFMT, int NQ, int MT, int F, int KMAX, int QR, bool SEQ>
__global__ __launch_bounds__(64 * (NQ + RsCfg<NQ, MT, F, KMAX>::NW)) void k_linear_small_m_rs(const uint16_t* __restrict__ x, int M,
                                                           int K, const uint8_t* __restrict__ packed,
                                                           int N, const uint16_t* __restrict__ bias,
                                                           uint16_t* __restrict__ y, BatchStrides bs,
                                                           int RT) {
  using R = RsCfg<NQ, MT, F, KMAX>;
  static_assert(QR >= 1 && QR <= R::ROWS, "quantized rows");
  {  // batch blockIdx.y (byte strides; all zero when unbatched)
    const int64_t b = blockIdx.y;
    x = (const uint16_t*)((const uint8_t*)x + b * bs.x);
    packed += b * bs.w;
    y = (uint16_t*)((uint8_t*)y + b * bs.y);
    if (bias) bias = (const uint16_t*)((const uint8_t*)bias + b * bs.bias);
  }
  constexpr int FB = frag_bytes(WFMT);
  __shared__ __attribute__((aligned(16))) uint8_t lds[R::LDS];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane & 15, g = lane >> 4;
  const int NG = N >> 4, KT = K >> 7, KT4 = (KT + 3) >> 2, KB = K >> 5;
  const int GPW = (KT4 + 3) / 4;                          // K groups per weight wave (SEQ)
  const int P = K + 16;                                   // code row pitch
  uint8_t* const codes = lds;                             // [ROWS][P]
  uint8_t* const scl = lds + R::ROWS * P;                 // [ROWS][KB]
  v4f* const red = (v4f*)(lds + R::ROWS * R::PITCH + R::ROWS * (KMAX / 32));   // [NW][PAIRS][64]
  int ng = blockIdx.x;                                    // first weight fragment
  if constexpr (F > 1) {                                  // row tiles (one with F == 1)
    const int RTn = (M + RT - 1) / RT;
    int c, t;
    rs_tile_of(blockIdx.x, gridDim.x / RTn, RTn, c, t);
    ng = F * c;
    const int m0 = RT * t;
    M = min(RT, M - m0);                                  // rows of this tile
    x += (int64_t)m0 * K;
    y += (int64_t)m0 * N;
  }

  v8i a[R::GMAX][4][R::FPW];
  uint32_t sw[R::GMAX][R::FPW];
  v2i braw = {0, 0};
  const bool bias8 = bias != nullptr && ((uintptr_t)bias & 7) == 0;
  if (wave < NQ) {
    // quantizer waves: K groups q, q + NQ, ..; lane l takes row m's elements 512 kt4 + 8 l .. + 7
    // (a quad of lanes is one MX block).  Every row load of every group goes out before any is
    // used; columns past K (a last group of fewer than 4 steps) and groups past the end re-read
    // valid elements, whose codes are not stored (whole quads: K % 128 == 0).
    typedef const __attribute__((address_space(1))) v4i* gv4i_t;
    const __attribute__((address_space(1))) uint8_t* xg = (const __attribute__((address_space(1))) uint8_t*)x;
    v4i xr[R::QMAX][QR];
#pragma unroll
    for (int i = 0; i < R::QMAX; ++i) {
      const int colc = min(512 * (wave + NQ * i) + 8 * lane, K - 8);
#pragma unroll
      for (int m = 0; m < QR; ++m) xr[i][m] = *(gv4i_t)(xg + (uint32_t)(2 * (min(m, M - 1) * K + colc)));
    }
#pragma unroll
    for (int i = 0; i < R::QMAX; ++i) {
      const int col = 512 * (wave + NQ * i) + 8 * lane;
      const bool on = col < K;
#pragma unroll
      for (int m = 0; m < QR; ++m) {
        const v4i v = xr[i][m];
        const uint32_t e = scale_byte_from_amax<0>(quad_max_u32(amax8_bf16_pk(v)));
        v2i q = cvt8_e4m3(v, e8m0_to_float_ldexp(e));
        if (e == 0xFFu) q = (v2i){0x7F7F7F7F, 0x7F7F7F7F};   // Inf/NaN block: NaN codes
        if (on) {
          *(v2i*)(codes + m * P + col) = q;
          scl[m * KB + (col >> 5)] = (uint8_t)e;          // the quad's four lanes, one byte
        }
      }
    }
  } else {
    // weight waves: the scale words and fragments of every K group of this wave, non-temporal
    // (read once per call); steps past the end re-read the last one, unused
    const int w = wave - NQ, wl = w & 3;
    const int f0 = ng + (w >> 2) * R::FPW;                // this wave's first fragment
    const uint32_t* wsc = (const uint32_t*)(packed + (int64_t)KT * NG * FB) + (int64_t)f0 * 64 + lane;
#pragma unroll
    for (int i = 0; i < R::GMAX; ++i) {
      const int kt4 = SEQ ? wl * GPW + i : wl + 4 * i;
      if (kt4 < KT4 && (!SEQ || i < GPW)) {               // wave-uniform
#pragma unroll
        for (int f = 0; f < R::FPW; ++f) sw[i][f] = wsc[(int64_t)kt4 * NG * 64 + 64 * f];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int kt = min(4 * kt4 + j, KT - 1);
#pragma unroll
          for (int f = 0; f < R::FPW; ++f) {
            const uint8_t* fr = packed + ((int64_t)kt * NG + f0 + f) * FB;
            const v4i lo = __builtin_nontemporal_load((const v4i*)(fr + lane * 16));
            if (WFMT == 0) {
              const v4i hi = __builtin_nontemporal_load((const v4i*)(fr + 1024 + lane * 16));
              a[i][j][f] = (v8i){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            } else {
              const v2i hi = __builtin_nontemporal_load((const v2i*)(fr + 1024 + lane * 8));
              a[i][j][f] = (v8i){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], 0, 0};
            }
          }
        }
      }
    }
    // weight wave w finishes output pair w = (row tile w / F, fragment w % F): its bias
    if (w < R::PAIRS && bias8) braw = *(const v2i*)(bias + 16 * (ng + w % F) + 4 * g);
  }
  rs_lds_barrier();   // the code image is complete

  // the K groups of weight wave l of its set onto the accumulators, in K order
  auto mfma_groups = [&](v4f (&acc)[MT][R::FPW], int wl) __attribute__((always_inline)) {
    int mrow[MT];     // rows past the tile read its last row: their outputs are not stored
#pragma unroll
    for (int t = 0; t < MT; ++t) mrow[t] = min(16 * t + r, M - 1);
#pragma unroll
    for (int i = 0; i < R::GMAX; ++i) {
      const int kt4 = SEQ ? wl * GPW + i : wl + 4 * i;
      if (kt4 < KT4 && (!SEQ || i < GPW)) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int kt = 4 * kt4 + j;
          if (kt < KT) {                                  // wave-uniform
#pragma unroll
            for (int t = 0; t < MT; ++t) {
              const uint8_t* p = codes + mrow[t] * P + 128 * kt + 16 * g;
              const v4i lo = *(const v4i*)p, hi = *(const v4i*)(p + 64);
              const v8i b = (v8i){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
              const uint32_t sb = scl[mrow[t] * KB + 4 * kt + g];
#pragma unroll
              for (int f = 0; f < R::FPW; ++f)
                acc[t][f] = mfma_wsel<WFMT>(j, a[i][j][f], b, acc[t][f], sw[i][f], sb);
            }
          }
        }
      }
    }
  };
  if constexpr (SEQ) {
    // one chain per output pair, red[pair][64]: wave l of each set extends its set's chains in
    // segment l (a wave with no K group leaves them alone); every wave passes the 4 barriers
#pragma unroll
    for (int seg = 0; seg < 4; ++seg) {
      if (wave >= NQ && ((wave - NQ) & 3) == seg && seg * GPW < KT4) {   // wave-uniform
        const int fs = ((wave - NQ) >> 2) * R::FPW;       // the set's first fragment
        v4f acc[MT][R::FPW];
#pragma unroll
        for (int t = 0; t < MT; ++t)
#pragma unroll
          for (int f = 0; f < R::FPW; ++f)
            acc[t][f] = seg == 0 ? (v4f){0.f, 0.f, 0.f, 0.f} : red[(t * F + fs + f) * 64 + lane];
        mfma_groups(acc, seg);
#pragma unroll
        for (int t = 0; t < MT; ++t)
#pragma unroll
          for (int f = 0; f < R::FPW; ++f) red[(t * F + fs + f) * 64 + lane] = acc[t][f];
      }
      rs_lds_barrier();
    }
  } else {
    if (wave >= NQ) {
      const int w = wave - NQ;
      v4f acc[MT][R::FPW];
#pragma unroll
      for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int f = 0; f < R::FPW; ++f) acc[t][f] = (v4f){0.f, 0.f, 0.f, 0.f};
      mfma_groups(acc, w & 3);
#pragma unroll
      for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int f = 0; f < R::FPW; ++f) red[((w * MT + t) * R::FPW + f) * 64 + lane] = acc[t][f];
    }
    rs_lds_barrier();   // the partials are in
  }
  if (wave >= NQ && wave - NQ < R::PAIRS) {
    const int pr = wave - NQ, t = pr / F, f = pr % F;
    v4f s4;
    if constexpr (SEQ) {
      s4 = red[pr * 64 + lane];
    } else {
      // the four partials of the fragment's set, in wave order
      const int w0 = 4 * (f / R::FPW), fl = f % R::FPW;
      s4 = red[((w0 * MT + t) * R::FPW + fl) * 64 + lane];
#pragma unroll
      for (int l = 1; l < 4; ++l) s4 += red[(((w0 + l) * MT + t) * R::FPW + fl) * 64 + lane];
    }
    const int n = 16 * (ng + f) + 4 * g;                  // this lane's 4 output columns
    float bv[4] = {0.f, 0.f, 0.f, 0.f};
    if (bias8) {
      bv[0] = bf16_to_float((uint32_t)braw[0] & 0xFFFFu);
      bv[1] = bf16_to_float((uint32_t)braw[0] >> 16);
      bv[2] = bf16_to_float((uint32_t)braw[1] & 0xFFFFu);
      bv[3] = bf16_to_float((uint32_t)braw[1] >> 16);
    } else if (bias) {
#pragma unroll
      for (int i = 0; i < 4; ++i) bv[i] = bf16_to_float(bias[n + i]);
    }
    const int m = 16 * t + r;
    if (m < M) {
      const v2i o = {(int)pack_bf16x2(s4[0] + bv[0], s4[1] + bv[1]),
                     (int)pack_bf16x2(s4[2] + bv[2], s4[3] + bv[3])};
      *(v2i*)(y + (int64_t)m * N + n) = o;
    }
  }
}

// ---------------------------------------------------------------------------------------------
// Decode with the K dimension also split across workgroups (M <= 64 in up to four 16-row
// activation tiles, bf16 activations; used from M = 16 on).
// Workgroup (b, p) computes 64 output columns (weight fragments 4 b .. 4 b + 3) over K part p
// of P; its 8 waves take that part's K steps in turn.  Per K step a wave loads its activation
// rows straight in the MFMA operand layout and quantizes them there: lane (r, g) holds row r's
// K bytes [16 g, 16 g + 16) and [64 + 16 g, ...), i.e. halves of MX blocks g / 2 and 2 + g / 2,
// whose maxima are completed with the lane 16 apart; the block scale the MFMA reads from lane
// r + 16 b is then fetched from the lane that computed it.  The codes and scales are those of
// k_quantize_act, bit for bit.  Each workgroup reads only its K part of x, and no second
// launch quantizes x first.
// Reduction: the 8 wave partials in wave order (LDS), then, with P > 1, the P workgroup
// partials of a column group in part order by the last of them to arrive (a counter per
// column group in the workspace, left at zero by that workgroup; no workgroup ever waits).

constexpr int kSkMaxParts = 8;
constexpr int kSkMaxM = 64;     // up to four 16-row activation tiles

// The workgroup's sums of its (fragment, activation tile) pairs, pair pr = wave + NW u in s[u],
// to the output: with P > 1 through the workspace, the P parts of a column group added in
// part order by the last workgroup of the group to finish; then bias, one bf16 rounding,
// store.  Every thread of the workgroup calls it (it holds workgroup barriers); `last` is a
// workgroup-shared int.
template <int MT, int NW, int PPW>
__device__ __forceinline__ void sk_parts_to_output(v4f (&s)[PPW], int wave, int lane, int M,
                                                   int N, int P, int p, int bx, int NG4,
                                                   uint32_t* __restrict__ cnt,
                                                   v4f* __restrict__ part,
                                                   const uint16_t* __restrict__ bias,
                                                   uint16_t* __restrict__ y, int& last) {
  constexpr int CT = 4 * MT;
  const int r = lane & 15, g = lane >> 4;
  const int ng0 = 4 * bx;
  if (P > 1) {
    // The partials go through device-coherent accesses (agent-scope atomic stores and loads,
    // which bypass the non-coherent caches), so the exchange needs no cache write-back or
    // invalidation: a workgroup's stores have completed (vmcnt 0) before its thread 0 counts it
    // in, and the last one reads the others' partials after its count.
#pragma unroll
    for (int u = 0; u < PPW; ++u) {
      const int pr = wave + NW * u;
      if (pr < CT) {
        uint64_t* dst = (uint64_t*)(part + ((int64_t)(p * NG4 + bx) * CT + pr) * 64 + lane);
        uint64_t v[2];
        __builtin_memcpy(v, &s[u], 16);
        __hip_atomic_store(dst, v[0], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(dst + 1, v[1], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    __builtin_amdgcn_s_waitcnt(0x0070);   // vmcnt(0) lgkmcnt(0): the stores are done
    __syncthreads();
    if (threadIdx.x == 0)
      last = __hip_atomic_fetch_add(&cnt[bx], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
             (uint32_t)(P - 1);
    __syncthreads();
    if (!last) return;
#pragma unroll
    for (int u = 0; u < PPW; ++u) {
      const int pr = wave + NW * u;
      if (pr < CT) {
        // all parts' loads in flight together, then the sum in part order, whichever
        // workgroup finished last
        uint64_t v[kSkMaxParts][2];
#pragma unroll
        for (int q = 0; q < kSkMaxParts; ++q) {
          if (q < P) {
            const uint64_t* src = (const uint64_t*)(part + ((int64_t)(q * NG4 + bx) * CT + pr) * 64 + lane);
            v[q][0] = __hip_atomic_load(src, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            v[q][1] = __hip_atomic_load(src + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          }
        }
#pragma unroll
        for (int q = 0; q < kSkMaxParts; ++q) {
          if (q < P) {
            v4f t;
            __builtin_memcpy(&t, v[q], 16);
            s[u] = q == 0 ? t : s[u] + t;
          }
        }
      }
    }
    if (threadIdx.x == 0) __hip_atomic_store(&cnt[bx], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
#pragma unroll
  for (int u = 0; u < PPW; ++u) {
    const int pr = wave + NW * u;
    if (pr < CT) {
      const int c = pr / MT, t = pr % MT;
      const int m = 16 * t + r, n = 16 * (ng0 + c) + 4 * g;
      if (m < M) {
        float bv[4] = {0.f, 0.f, 0.f, 0.f};
        if (bias) {
#pragma unroll
          for (int i = 0; i < 4; ++i) bv[i] = bf16_to_float(bias[n + i]);
        }
        const v2i o = {(int)pack_bf16x2(s[u][0] + bv[0], s[u][1] + bv[1]),
                       (int)pack_bf16x2(s[u][2] + bv[2], s[u][3] + bv[3])};
        *(v2i*)(y + (int64_t)m * N + n) = o;
      }
    }
  }
}

template <int WFMT, int MT>
__global__ __launch_bounds__(512) void k_linear_decode_sk(const uint16_t* __restrict__ x, int M,
                                                          int K, const uint8_t* __restrict__ packed,
                                                          int N, const uint16_t* __restrict__ bias,
                                                          uint16_t* __restrict__ y, int P,
                                                          uint32_t* __restrict__ cnt,
                                                          v4f* __restrict__ part) {
  constexpr int FB = frag_bytes(WFMT);
  constexpr int CT = 4 * MT;                    // (fragment, activation tile) pairs
  __shared__ v4f red[kWaves][CT][64];
  __shared__ int last;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane & 15, g = lane >> 4;
  const int NG = N >> 4, KT = K >> 7;
  const int bx = blockIdx.x, p = blockIdx.y, NG4 = gridDim.x;
  const int ng0 = 4 * bx;
  const int kt_lo = (int)((int64_t)p * KT / P), kt_hi = (int)((int64_t)(p + 1) * KT / P);
  const uint32_t* wsc = (const uint32_t*)(packed + (int64_t)KT * NG * FB) + (int64_t)ng0 * 64 + lane;

  // activation rows of this lane; rows past M repeat row M - 1 (their outputs are not stored)
  int mrow[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) mrow[t] = min(16 * t + r, M - 1);
  v4f acc[4][MT];
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int t = 0; t < MT; ++t) acc[c][t] = (v4f){0.f, 0.f, 0.f, 0.f};

  for (int kt = kt_lo + wave; kt < kt_hi; kt += kWaves) {
    // activations first (L2-resident after the first workgroups), then the weight (HBM, read
    // once: non-temporal)
    v4i xv[MT][4];
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      const uint16_t* xr = x + (int64_t)mrow[t] * K + 128 * kt + 16 * g;
      xv[t][0] = *(const v4i*)xr;
      xv[t][1] = *(const v4i*)(xr + 8);
      xv[t][2] = *(const v4i*)(xr + 64);
      xv[t][3] = *(const v4i*)(xr + 72);
    }
    __builtin_amdgcn_sched_barrier(0);
    uint32_t sw[4];
    v8i a[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) sw[c] = wsc[(int64_t)(kt >> 2) * NG * 64 + c * 64];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const uint8_t* f = packed + ((int64_t)kt * NG + ng0 + c) * FB;
      const v4i lo = __builtin_nontemporal_load((const v4i*)(f + lane * 16));
      if (WFMT == 0) {
        const v4i hi = __builtin_nontemporal_load((const v4i*)(f + 1024 + lane * 16));
        a[c] = (v8i){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      } else {
        const v2i hi = __builtin_nontemporal_load((const v2i*)(f + 1024 + lane * 8));
        a[c] = (v8i){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], 0, 0};
      }
    }
    __builtin_amdgcn_sched_barrier(0);

    // quantize in the operand layout
    v8i b[MT];
    uint32_t sb[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) quantize_tile_operand_e4m3(xv[t], lane, b[t], sb[t]);
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int t = 0; t < MT; ++t)
        acc[c][t] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
            a[c], b[t], acc[c][t], WFMT, 0, 0, (int)(sw[c] >> (8 * (kt & 3))), 0, (int)sb[t]);
  }

  // wave partials, summed in wave order: wave w finishes pairs w, w + 8, ... of the CT pairs
  // (c, t), pair index c MT + t
  constexpr int PPW = (CT + kWaves - 1) / kWaves;
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int t = 0; t < MT; ++t) red[wave][c * MT + t][lane] = acc[c][t];
  __syncthreads();
  v4f s[PPW];
#pragma unroll
  for (int u = 0; u < PPW; ++u) {
    const int pr = wave + kWaves * u;
    s[u] = (v4f){0.f, 0.f, 0.f, 0.f};
    if (pr < CT) {
      s[u] = red[0][pr][lane];
#pragma unroll
      for (int w = 1; w < kWaves; ++w) s[u] += red[w][pr][lane];
    }
  }
  sk_parts_to_output<MT, kWaves, PPW>(s, wave, lane, M, N, P, p, bx, NG4, cnt, part, bias, y, last);
}

// The split-K decode kernel with the waves in two roles, for K parts of at most 8 steps: eight
// waves load the part's activation rows and quantize them row-major (as k_linear_small_m_rs)
// into an LDS image of codes and scales, while four waves issue the part's weight stream (two
// steps of the 4 fragments each, in registers); one barrier, then the four run the MFMAs from
// the image.  Their partials are added in wave order per (fragment, tile) pair, then the parts
// as in k_linear_decode_sk.  Same codes and scales as k_quantize_act.
constexpr int kSkRsSteps = 8;                        // K steps per part, at most
constexpr int kSkRsPitch = 128 * kSkRsSteps + 16;    // code row pitch; +16 B: banks
constexpr int kSkRsQ = 8;                            // quantizer waves
constexpr int kSkRsW = 4;                            // weight (MFMA) waves

template <int WFMT, int MT>
__global__ __launch_bounds__(64 * (kSkRsQ + kSkRsW)) void k_linear_decode_sk_rs(
    const uint16_t* __restrict__ x, int M, int K, const uint8_t* __restrict__ packed, int N,
    const uint16_t* __restrict__ bias, uint16_t* __restrict__ y, int P, uint32_t* __restrict__ cnt,
    v4f* __restrict__ part) {
  constexpr int NW = kSkRsQ + kSkRsW;
  constexpr int FB = frag_bytes(WFMT);
  constexpr int CT = 4 * MT;                         // (fragment, activation tile) pairs
  constexpr int ROWS = 16 * MT;
  constexpr int CODES = ROWS * kSkRsPitch;
  constexpr int SCL = ROWS * 4 * kSkRsSteps;         // [ROWS][32 blocks]
  constexpr int RED = kSkRsW * CT * 64 * 16;         // the weight waves' partials (after the MFMAs)
  constexpr int LDS = CODES + SCL > RED ? CODES + SCL : RED;
  constexpr int UMAX = (ROWS * 2 + kSkRsQ - 1) / kSkRsQ;   // (row, 4-step group) units per wave
  __shared__ __attribute__((aligned(16))) uint8_t lds[LDS];
  __shared__ int last;
  uint8_t* const codes = lds;                        // [ROWS][kSkRsPitch]
  uint8_t* const scl = lds + CODES;                  // [ROWS][4 kSkRsSteps]
  v4f* const red = (v4f*)lds;                        // [kSkRsW][CT][64], over the image
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane & 15, g = lane >> 4;
  const int NG = N >> 4, KT = K >> 7;
  const int bx = blockIdx.x, p = blockIdx.y, NG4 = gridDim.x;
  const int ng0 = 4 * bx;
  const int kt_lo = (int)((int64_t)p * KT / P), kt_hi = (int)((int64_t)(p + 1) * KT / P);
  const int KS = kt_hi - kt_lo, GP = (KS + 3) >> 2;  // steps, 4-step groups of the part

  v8i a[2][4];
  uint32_t sw[2][4];
  if (wave < kSkRsQ) {
    // quantizer waves: units u = wave + 8 i, row u / GP, group u % GP; lane l takes the row's
    // elements 512 group + 8 l .. + 7 of the part.  All loads first; units past the last row
    // and columns past the part re-read valid elements, whose codes are not stored.
    typedef const __attribute__((address_space(1))) v4i* gv4i_t;
    const __attribute__((address_space(1))) uint8_t* xg = (const __attribute__((address_space(1))) uint8_t*)x;
    const uint32_t kbase = (uint32_t)kt_lo * 128;
    v4i xr[UMAX];
#pragma unroll
    for (int i = 0; i < UMAX; ++i) {
      const int u = wave + kSkRsQ * i;
      const int row = min(u / GP, M - 1);
      const int colc = min(512 * (u % GP) + 8 * lane, 128 * KS - 8);
      xr[i] = *(gv4i_t)(xg + 2 * ((uint32_t)row * (uint32_t)K + kbase + (uint32_t)colc));
    }
#pragma unroll
    for (int i = 0; i < UMAX; ++i) {
      const int u = wave + kSkRsQ * i;
      const int row = u / GP, col = 512 * (u % GP) + 8 * lane;
      const v4i v = xr[i];
      const uint32_t e = scale_byte_from_amax<0>(quad_max_u32(amax8_bf16_pk(v)));
      v2i q = cvt8_e4m3(v, e8m0_to_float_ldexp(e));
      if (e == 0xFFu) q = (v2i){0x7F7F7F7F, 0x7F7F7F7F};   // Inf/NaN block: NaN codes
      if (row < M && col < 128 * KS) {
        *(v2i*)(codes + row * kSkRsPitch + col) = q;
        scl[row * (4 * kSkRsSteps) + (col >> 5)] = (uint8_t)e;   // the quad's lanes, one byte
      }
    }
  } else {
    // weight waves: steps kt_lo + w and kt_lo + w + 4 of the part, the 4 fragments of each and
    // their scale words (non-temporal: read once per call)
    const int w = wave - kSkRsQ;
    const uint32_t* wsc = (const uint32_t*)(packed + (int64_t)KT * NG * FB) + (int64_t)ng0 * 64 + lane;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int kt = kt_lo + w + 4 * h;
      if (kt < kt_hi) {                              // wave-uniform
#pragma unroll
        for (int c = 0; c < 4; ++c) sw[h][c] = wsc[(int64_t)(kt >> 2) * NG * 64 + c * 64];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const uint8_t* f = packed + ((int64_t)kt * NG + ng0 + c) * FB;
          const v4i lo = __builtin_nontemporal_load((const v4i*)(f + lane * 16));
          if (WFMT == 0) {
            const v4i hi = __builtin_nontemporal_load((const v4i*)(f + 1024 + lane * 16));
            a[h][c] = (v8i){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          } else {
            const v2i hi = __builtin_nontemporal_load((const v2i*)(f + 1024 + lane * 8));
            a[h][c] = (v8i){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], 0, 0};
          }
        }
      }
    }
  }
  rs_lds_barrier();   // the code image is complete

  v4f acc[4][MT];
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int t = 0; t < MT; ++t) acc[c][t] = (v4f){0.f, 0.f, 0.f, 0.f};
  if (wave >= kSkRsQ) {
    const int w = wave - kSkRsQ;
    int mrow[MT];     // rows past M read row M - 1: their outputs are not stored
#pragma unroll
    for (int t = 0; t < MT; ++t) mrow[t] = min(16 * t + r, M - 1);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int kt = kt_lo + w + 4 * h;
      if (kt < kt_hi) {
        const int ks = kt - kt_lo;
#pragma unroll
        for (int t = 0; t < MT; ++t) {
          const uint8_t* pb = codes + mrow[t] * kSkRsPitch + 128 * ks + 16 * g;
          const v4i lo = *(const v4i*)pb, hi = *(const v4i*)(pb + 64);
          const v8i b = (v8i){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          const uint32_t sb = scl[mrow[t] * (4 * kSkRsSteps) + 4 * ks + g];
#pragma unroll
          for (int c = 0; c < 4; ++c)
            acc[c][t] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                a[h][c], b, acc[c][t], WFMT, 0, 0, (int)(sw[h][c] >> (8 * (kt & 3))), 0, (int)sb);
        }
      }
    }
  }
  rs_lds_barrier();   // every MFMA has read the image: the partials may go over it
  if (wave >= kSkRsQ) {
    const int w = wave - kSkRsQ;
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int t = 0; t < MT; ++t) red[(w * CT + c * MT + t) * 64 + lane] = acc[c][t];
  }
  rs_lds_barrier();
  // the four weight waves' partials of pair pr, added in wave order, by wave pr % 12
  constexpr int PPW = (CT + NW - 1) / NW;
  v4f s4[PPW];
#pragma unroll
  for (int u = 0; u < PPW; ++u) {
    const int pr = wave + NW * u;
    s4[u] = (v4f){0.f, 0.f, 0.f, 0.f};
    if (pr < CT) {
      s4[u] = red[pr * 64 + lane];
#pragma unroll
      for (int w = 1; w < kSkRsW; ++w) s4[u] += red[(w * CT + pr) * 64 + lane];
    }
  }
  sk_parts_to_output<MT, NW, PPW>(s4, wave, lane, M, N, P, p, bx, NG4, cnt, part, bias, y, last);
}

// the role-split variant holds parts of at most 8 K steps
static bool decode_sk_rs_ok(int64_t KT, int P) { return (KT + P - 1) / P <= kSkRsSteps; }

// K parts: about 256 workgroups, at least 8 K steps (one per wave) in each part, at most 8
int decode_sk_parts(int64_t N, int64_t K) {
  const int64_t ng4 = N / 64, kt = K / 128;
  int64_t p = (256 + ng4 - 1) / ng4;
  int64_t pmax = kt / 8 > 1 ? kt / 8 : 1;
  if (pmax > kSkMaxParts) pmax = kSkMaxParts;
  if (p > pmax) p = pmax;
  return (int)(p < 1 ? 1 : p);
}

bool decode_sk_ok(int64_t M, int64_t N, int64_t K) {
  return M >= 1 && M <= kSkMaxM && K % 128 == 0 && N % 64 == 0 && N / 64 * 4 <= kWorkspacePrefix;
}

int64_t decode_sk_workspace(int64_t M, int64_t N, int64_t K) {
  const int64_t mt = (M + 15) / 16;
  return decode_sk_parts(N, K) * (N / 64) * 4 * mt * 64 * 16;
}

hipError_t launch_linear_decode_sk(const uint16_t* x, int64_t M, int64_t K, const uint8_t* packed,
                                   int64_t N, int fmt, const uint16_t* bias, uint16_t* y,
                                   void* workspace, hipStream_t s) {
  if (!decode_sk_ok(M, N, K)) return hipErrorInvalidValue;
  const int P = decode_sk_parts(N, K);
  uint32_t* cnt = (uint32_t*)workspace;
  v4f* part = (v4f*)((uint8_t*)workspace + kWorkspacePrefix);
  const dim3 grid((unsigned)(N / 64), (unsigned)P), block(512);
  const int m = (int)M, k = (int)K, n = (int)N;
  if (decode_sk_rs_ok(K / 128, P)) {
    const dim3 block_rs(64 * (kSkRsQ + kSkRsW));
#define MX_SKRS(W)                                                                                    \
  do {                                                                                                \
    if (M <= 16)                                                                                      \
      hipLaunchKernelGGL((k_linear_decode_sk_rs<W, 1>), grid, block_rs, 0, s, x, m, k, packed, n, bias, y, P, cnt, part); \
    else if (M <= 32)                                                                                 \
      hipLaunchKernelGGL((k_linear_decode_sk_rs<W, 2>), grid, block_rs, 0, s, x, m, k, packed, n, bias, y, P, cnt, part); \
    else if (M <= 48)                                                                                 \
      hipLaunchKernelGGL((k_linear_decode_sk_rs<W, 3>), grid, block_rs, 0, s, x, m, k, packed, n, bias, y, P, cnt, part); \
    else                                                                                              \
      hipLaunchKernelGGL((k_linear_decode_sk_rs<W, 4>), grid, block_rs, 0, s, x, m, k, packed, n, bias, y, P, cnt, part); \
  } while (0)
    switch (fmt) {
      case 0: MX_SKRS(0); break;
      case 2: MX_SKRS(2); break;
      case 3: MX_SKRS(3); break;
      default: return hipErrorInvalidValue;
    }
#undef MX_SKRS
    return hipGetLastError();
  }
#define MX_SK(W)                                                                                      \
  do {                                                                                                \
    if (M <= 16)                                                                                      \
      hipLaunchKernelGGL((k_linear_decode_sk<W, 1>), grid, block, 0, s, x, m, k, packed, n, bias, y, P, cnt, part); \
    else if (M <= 32)                                                                                 \
      hipLaunchKernelGGL((k_linear_decode_sk<W, 2>), grid, block, 0, s, x, m, k, packed, n, bias, y, P, cnt, part); \
    else if (M <= 48)                                                                                 \
      hipLaunchKernelGGL((k_linear_decode_sk<W, 3>), grid, block, 0, s, x, m, k, packed, n, bias, y, P, cnt, part); \
    else                                                                                              \
      hipLaunchKernelGGL((k_linear_decode_sk<W, 4>), grid, block, 0, s, x, m, k, packed, n, bias, y, P, cnt, part); \
  } while (0)
  switch (fmt) {
    case 0: MX_SK(0); break;
    case 2: MX_SK(2); break;
    case 3: MX_SK(3); break;
    default: return hipErrorInvalidValue;
  }
#undef MX_SK
  return hipGetLastError();
}

// Up to 16 rows with K <= 8192 in one row tile; with K <= 4096, 17 to 32 rows in two row tiles
// of at most 16 rows (two weight fragments per workgroup, N % 32 == 0) and 33 to 64 rows in
// three or four (four fragments per workgroup, N % 64 == 0), or, for other N, up to 24 rows in
// one tile.  A workgroup quantizes its whole row tile, so the quantizer's VALU time grows with
// the tile's rows (4096 x 4096 in one tile: 6.2 us at M = 16, 8.6 at 24, 10.3 at 32).
constexpr int kRsRowSplitMinM = 17;   // from this many rows on: row tiles
// fragments per workgroup of the row-split form, 0 where it is not used
static int rs_row_split(int64_t M, int64_t N, int64_t K) {
  if (K > 4096 || M < kRsRowSplitMinM || M > 64) return 0;
  if (M <= 32) return N % 32 == 0 ? 2 : 0;
  return N % 64 == 0 ? 4 : 0;
}
bool small_m_rs(int64_t M, int64_t N, int64_t K) {
  return M >= 1 && K % 128 == 0 &&
         ((M <= 16 && K <= 8192) || (M <= 24 && K <= 4096) || rs_row_split(M, N, K) > 0);
}
bool small_m_fused(int64_t M, int64_t N, int64_t K) {
  return M >= 1 && K % 128 == 0 && (M <= 16 || small_m_rs(M, N, K));
}
bool small_m_quantized(int64_t M, int64_t K) { return M >= 1 && M <= 32 && K % 128 == 0; }
bool small_m_invariant(int64_t M, int64_t N, int64_t K, bool quantized) {
  return !quantized && small_m_rs(M, N, K);
}

// the role-split kernel with the smallest code image and row count that hold a row tile of RT
// rows; four quantizer waves for one or two rows (fewer waves in the workgroup) and beside the
// eight weight waves of four fragments per workgroup, eight otherwise
template <int WFMT, int MT, int F, int KMAX, bool SEQ>
static void launch_rs_k(const uint16_t* x, int M, int K, const uint8_t* packed, int N,
                        const uint16_t* bias, uint16_t* y, hipStream_t s, dim3 grid,
                        const BatchStrides& bs, int RT) {
#define MX_RS(NQ, QR) hipLaunchKernelGGL((k_linear_small_m_rs<WFMT, NQ, MT, F, KMAX, QR, SEQ>), grid, dim3(64 * (NQ + RsCfg<NQ, MT, F, KMAX>::NW)), 0, s, x, M, K, packed, N, bias, y, bs, RT)
  if constexpr (F == 4) {
    if (RT <= 1) MX_RS(4, 1);
    else if (RT <= 2) MX_RS(4, 2);
    else if (RT <= 4) MX_RS(4, 4);
    else if (RT <= 8) MX_RS(4, 8);
    else if (RT <= 12) MX_RS(4, 12);
    else MX_RS(4, 16);
  } else if constexpr (MT == 1) {
    if (RT <= 1) MX_RS(4, 1);
    else if (RT <= 2) MX_RS(4, 2);
    else if (RT <= 4) MX_RS(8, 4);
    else if (RT <= 8) MX_RS(8, 8);
    else if (RT <= 12) MX_RS(8, 12);
    else MX_RS(8, 16);
  } else {
    MX_RS(8, 24);
  }
#undef MX_RS
}
// Weight fragments per workgroup, widened (from 4 rows on) while the grid still holds at least
// 256 workgroups: a workgroup then loads and quantizes its activation rows once for more output
// columns, so each CU pulls fewer bytes per output (calls of several layers, wide N).  Eight
// 4096 x 4096 layers per call: M = 8 3.94 -> 3.22 us per layer, M = 32 5.79 -> 4.81 us; at
// M = 1 the activation rows are too few to pay (2.96 against 3.08 us with four fragments).
// Every tiling adds each output's K steps in the same order, so the choice never changes bits.
constexpr int kRsWidenMax = 4, kRsWidenMinM = 4;
template <int WFMT, bool SEQ>
static void launch_rs(const uint16_t* x, int M, int K, const uint8_t* packed, int N,
                      const uint16_t* bias, uint16_t* y, hipStream_t s, int batch,
                      const BatchStrides& bs) {
  int F = rs_row_split(M, N, K), R = 1;                 // row tiles from 17 rows (K <= 4096)
  if (F > 0) R = (M + 15) / 16;
  else if (M > 16) {                                    // up to 24 rows in one tile, N % 32 != 0
    launch_rs_k<WFMT, 2, 1, 4096, SEQ>(x, M, K, packed, N, bias, y, s,
                                       dim3((unsigned)(N / 16), (unsigned)batch), bs, M);
    return;
  } else {
    F = 1;
  }
  if (K <= 4096 && M >= kRsWidenMinM) {
    for (int f = kRsWidenMax; f > F; f >>= 1)
      if (N % (16 * f) == 0 && (int64_t)batch * (N / (16 * f)) * R >= 256) {
        F = f;
        break;
      }
  }
  const int RT = (M + R - 1) / R;                       // rows per tile
  R = (M + RT - 1) / RT;
  const dim3 grid((unsigned)(N / (16 * F) * R), (unsigned)batch);
  if (F == 4) {
    launch_rs_k<WFMT, 1, 4, 4096, SEQ>(x, M, K, packed, N, bias, y, s, grid, bs, RT);
  } else if (F == 2) {
    launch_rs_k<WFMT, 1, 2, 4096, SEQ>(x, M, K, packed, N, bias, y, s, grid, bs, RT);
  } else if (K <= 4096) {
    launch_rs_k<WFMT, 1, 1, 4096, SEQ>(x, M, K, packed, N, bias, y, s, grid, bs, M);
  } else {
    launch_rs_k<WFMT, 1, 1, 8192, SEQ>(x, M, K, packed, N, bias, y, s, grid, bs, M);
  }
}

template <int WFMT>
static void launch_small(const void* x, const uint8_t* xs, bool quantized, int M, int K,
                         const uint8_t* packed, int N, const uint16_t* bias, uint16_t* y,
                         hipStream_t s, int batch, const BatchStrides& bs) {
  const dim3 grid((unsigned)(N / 16), (unsigned)batch), block(512);
  const bool xs16 = ((uintptr_t)xs & 15) == 0 && K % 512 == 0;   // then K / 32 % 16 == 0 too
  if (!quantized && small_m_rs(M, N, K) && batch_invariant())
    launch_rs<WFMT, true>((const uint16_t*)x, M, K, packed, N, bias, y, s, batch, bs);
  else if (!quantized && small_m_rs(M, N, K))
    launch_rs<WFMT, false>((const uint16_t*)x, M, K, packed, N, bias, y, s, batch, bs);
  else if (!quantized)
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
  if (quantized ? !small_m_quantized(M, K) : !small_m_fused(M, N, K)) return hipErrorInvalidValue;
  if (batch_invariant() && !small_m_invariant(M, N, K, quantized)) return hipErrorInvalidValue;
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
