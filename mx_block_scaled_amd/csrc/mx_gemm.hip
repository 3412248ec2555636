// mx_gemm.hip — block-scaled GEMM on gfx950's scaled MFMA (v_mfma_scale_f32_16x16x128_f8f6f4).
//
// y[m, n] = sum_kb 2^(sx[m,kb]-127) 2^(sw[n,kb]-127) sum_{k in kb} xq[m,k] wq[n,k]  (+ bias[n])
// (aiter_flydsl page, apply_weights: block-scaled GEMM with row-major [M, K/32] activation
// scales and [N, K/32] weight scales, bf16 output, bias added afterwards — here fused into the
// fp32 epilogue so the output is rounded once.)
//
// The weight is the MFMA's A operand (rows = n) and the activations the B operand (columns =
// m): each lane then owns 4 consecutive n of one output row m, i.e. one 8-byte bf16 store.
#include <atomic>
#include <type_traits>

#include "mx_device.h"
#include "mx_launch.h"

namespace mx {

// Offsets the operand pointers (kernel parameters) to batch b (byte strides; all zero when
// unbatched).
#define MX_BATCH_OFFSET(b)                                                   \
  do {                                                                       \
    const int64_t b_ = (b);                                                  \
    xq += b_ * bs.x;                                                         \
    xs += b_ * bs.xs;                                                        \
    packed += b_ * bs.w;                                                     \
    y = (uint16_t*)((uint8_t*)y + b_ * bs.y);                                \
    if (bias) bias = (const uint16_t*)((const uint8_t*)bias + b_ * bs.bias); \
  } while (0)

// ---------------------------------------------------------------- generic kernel
// Any M, K % 32 == 0, N % 16 == 0.  One wave per workgroup: a 16-row weight fragment and MT
// 16-row activation tiles, both operands streamed straight from global memory into registers
// (no LDS).  The loads of U K steps go out together before their MFMAs, which then run in K
// order (each output's sum is the same MFMA chain as in the tiled kernel, so rows do not depend
// on M).  With one fragment per workgroup the weight stream spreads over N / 16 CUs; U = 16
// with one activation tile (M <= 16), 8 with two, keeps the registers under 256.
template <int WFMT, int XFMT, int MT>
__global__ __launch_bounds__(64) void k_gemm_generic(const uint8_t* __restrict__ xq,
                                                     const uint8_t* __restrict__ xs, int M, int K,
                                                     const uint8_t* __restrict__ packed, int N,
                                                     const uint16_t* __restrict__ bias,
                                                     uint16_t* __restrict__ y, BatchStrides bs) {
  constexpr int FB = frag_bytes(WFMT);
  constexpr int U = MT == 1 ? 16 : 8;
  MX_BATCH_OFFSET(blockIdx.z);
  const int lane = threadIdx.x;
  const int r = lane & 15, g = lane >> 4;
  const int NG = N >> 4, KT = (K + 127) >> 7, KB = K >> 5;
  // activation row bytes; an FP6 block kb's 24 bytes at XS (kb / 4) + 24 (kb % 4) of its row
  const int XS = XFMT == 0 ? 128 : (bs.xstep ? bs.xstep : 96);
  const int LDX = XFMT == 0 ? K : (bs.xstep ? K / 128 * bs.xstep : K / 4 * 3);
  const int ng = blockIdx.x;
  const int m0 = blockIdx.y * 16 * MT;
  const uint8_t* wfr = packed + (int64_t)ng * FB;
  const uint32_t* wsc = (const uint32_t*)(packed + (int64_t)KT * NG * FB) + (int64_t)ng * 64 + lane;
  // activation rows of this lane (clamped so every address is inside x; data is zeroed instead)
  int mrow[MT];
  bool mok[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    const int m = m0 + 16 * t + r;
    mok[t] = m < M;
    mrow[t] = mok[t] ? m : M - 1;
  }
  v4f acc[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) acc[t] = (v4f){0.f, 0.f, 0.f, 0.f};
  for (int kt0 = 0; kt0 < KT; kt0 += U) {
    // loads of steps kt0 .. kt0 + U - 1 (steps past the end re-read the last one, unused); the
    // weight, used once per call, with non-temporal loads
    v8i a[U], b[U][MT];
    int sa[U], sb[U][MT];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int kt = min(kt0 + u, KT - 1);
      const uint8_t* f = wfr + (int64_t)kt * NG * FB;
      if (WFMT == 0) {
        const v4i lo = __builtin_nontemporal_load((const v4i*)(f + lane * 16));
        const v4i hi = __builtin_nontemporal_load((const v4i*)(f + 1024 + lane * 16));
        a[u] = (v8i){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      } else {
        const v4i lo = __builtin_nontemporal_load((const v4i*)(f + lane * 16));
        const v2i hi = __builtin_nontemporal_load((const v2i*)(f + 1024 + lane * 8));
        a[u] = (v8i){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], 0, 0};
      }
      sa[u] = (int)((wsc[(int64_t)(kt >> 2) * NG * 64] >> (8 * (kt & 3))) & 0xFFu);
      const int kb = 4 * kt + g;
#pragma unroll
      for (int t = 0; t < MT; ++t) {
        const uint8_t* xr = xq + (int64_t)mrow[t] * LDX;
        if constexpr (XFMT == 0) {
          v4i b0 = {0, 0, 0, 0}, b1 = {0, 0, 0, 0};
          const int k0 = 128 * kt + 16 * g, k1 = k0 + 64;
          if (mok[t] && k0 < K) b0 = *(const v4i*)(xr + k0);
          if (mok[t] && k1 < K) b1 = *(const v4i*)(xr + k1);
          b[u][t] = (v8i){b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
        } else {
          // FP6 operand: block kb's 24 bytes (8-byte aligned: rows are 24 K/32 or XS K/128 bytes)
          v2i d0 = {0, 0}, d1 = {0, 0}, d2 = {0, 0};
          if (mok[t] && kb < KB) {
            const uint8_t* p = xr + XS * (kb >> 2) + 24 * (kb & 3);
            d0 = *(const v2i*)p;
            d1 = *(const v2i*)(p + 8);
            d2 = *(const v2i*)(p + 16);
          }
          b[u][t] = (v8i){d0[0], d0[1], d1[0], d1[1], d2[0], d2[1], 0, 0};
        }
        sb[u][t] = kb < KB ? (int)xs[(int64_t)mrow[t] * KB + kb] : 127;
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (kt0 + u < KT) {   // wave-uniform
#pragma unroll
        for (int t = 0; t < MT; ++t) acc[t] = mfma16<WFMT, XFMT>(a[u], b[u][t], acc[t], sa[u], sb[u][t]);
      }
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
  for (int t = 0; t < MT; ++t) {
    if (!mok[t]) continue;
    const v2i o = {(int)pack_bf16x2(acc[t][0] + bv[0], acc[t][1] + bv[1]),
                   (int)pack_bf16x2(acc[t][2] + bv[2], acc[t][3] + bv[3])};
    *(v2i*)(y + (int64_t)mrow[t] * N + n) = o;
  }
}

// ---------------------------------------------------------------- LDS-tiled kernel (large M)
// Workgroup tile: 32 FN weight rows (n) x 64 FM activation rows (m), K step 128, 8 waves in a
// 2 (n) x 4 (m) grid, each wave FN x FM MFMA tiles of 16 x 16 (TileCfg below).  Both operand
// tiles are copied global -> LDS with the 16-byte direct-to-LDS load (lane i of an instruction
// lands at LDS base + 16 i), in S stages:
//   A (weight): the prepacked fragments of one K step are contiguous in global memory, so the
//     LDS image is a plain copy and each lane's MFMA operand is one (or two) lane-contiguous
//     16-byte LDS reads — conflict-free.
//   B (activations, row-major [M, K]): 128-byte row slices; the 16-byte chunk c of row r is kept
//     in slot c ^ swz(r), so one DMA instruction covers 8 whole rows (coalesced global reads) and
//     the MFMA-order reads (16 rows, same chunk) hit 16 distinct bank groups.
// Scales: the weight's come prepacked per lane (one 32-bit word per 4 K steps); the
// activations' are gathered per lane from row-major [M, K/32] into the same form; the MFMA's
// op-select picks the byte of the current K step.
// Requires K % 128 == 0 (no K tail) and a 4-byte aligned xs; rows/columns past M/N are clamped
// on load and skipped on store.
__device__ __forceinline__ int swz(int row) { return ((row >> 1) ^ ((row & 1) << 2)) & 7; }

__device__ __forceinline__ void dma16(const void* src, void* lds_dst) {
  __builtin_amdgcn_global_load_lds((const void __attribute__((address_space(1)))*)src,
                                   (void __attribute__((address_space(3)))*)lds_dst, 16, 0, 0);
}

// scaled MFMA with the scale byte chosen by op-select; q is a constant after loop unrolling
__device__ __forceinline__ void dma4(const void* src, void* lds_dst) {
  __builtin_amdgcn_global_load_lds((const void __attribute__((address_space(1)))*)src,
                                   (void __attribute__((address_space(3)))*)lds_dst, 4, 0, 0);
}

template <int WFMT>
__device__ __forceinline__ v4f mfma_opsel(int q, const v8i& a, const v8i& b, v4f c, uint32_t sa,
                                          uint32_t sb) {
  switch (q) {
    case 0: return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, WFMT, 0, 0, (int)sa, 0, (int)sb);
    case 1: return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, WFMT, 0, 1, (int)sa, 1, (int)sb);
    case 2: return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, WFMT, 0, 2, (int)sa, 2, (int)sb);
    default: return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, WFMT, 0, 3, (int)sa, 3, (int)sb);
  }
}

// In-place scaled MFMA (D == C) as inline assembly: the builtin often gets a separate
// destination from the register allocator, which costs a spare accumulator quad per MFMA in
// flight.  Q = op-select byte of both scale registers; CBSZ = A-operand format (weight).
#define MX_MFMA_OPSEL_0 "op_sel_hi:[0,0,0]"
#define MX_MFMA_OPSEL_1 "op_sel:[1,1,0] op_sel_hi:[0,0,0]"
#define MX_MFMA_OPSEL_2 "op_sel_hi:[1,1,0]"
#define MX_MFMA_OPSEL_3 "op_sel:[1,1,0] op_sel_hi:[1,1,0]"
// PRE: instructions in the same statement ahead of the MFMA (the guard's wait states)
#define MX_MFMA_ASM(PRE, OPSEL, FMT)                                                            \
  asm volatile(PRE "v_mfma_scale_f32_16x16x128_f8f6f4 %0, %1, %2, %0, %3, %4 " OPSEL FMT       \
               : "+v"(acc) : "v"(a), "v"(b), "v"(sa), "v"(sb))
#define MX_MFMA_Q(PRE, FMT)                                            \
  do {                                                                 \
    if constexpr (Q == 0) MX_MFMA_ASM(PRE, MX_MFMA_OPSEL_0, FMT);      \
    else if constexpr (Q == 1) MX_MFMA_ASM(PRE, MX_MFMA_OPSEL_1, FMT); \
    else if constexpr (Q == 2) MX_MFMA_ASM(PRE, MX_MFMA_OPSEL_2, FMT); \
    else MX_MFMA_ASM(PRE, MX_MFMA_OPSEL_3, FMT);                       \
  } while (0)
#define MX_MFMA_FMT(PRE)                                                      \
  do {                                                                        \
    if constexpr (WFMT == 0) MX_MFMA_Q(PRE, "");                              \
    else if constexpr (WFMT == 2 && XFMT == 0) MX_MFMA_Q(PRE, " cbsz:2");     \
    else if constexpr (WFMT == 3 && XFMT == 0) MX_MFMA_Q(PRE, " cbsz:3");     \
    else if constexpr (WFMT == 2 && XFMT == 2) MX_MFMA_Q(PRE, " cbsz:2 blgp:2"); \
    else if constexpr (WFMT == 2 && XFMT == 3) MX_MFMA_Q(PRE, " cbsz:2 blgp:3"); \
    else if constexpr (WFMT == 3 && XFMT == 2) MX_MFMA_Q(PRE, " cbsz:3 blgp:2"); \
    else MX_MFMA_Q(PRE, " cbsz:3 blgp:3");                                    \
  } while (0)
// operand register image of one 16-row x 128-K fragment: 32 bytes for E4M3, 24 for FP6
template <int F> struct AReg { typedef v8i type; };
template <> struct AReg<2> { typedef v6i type; };
template <> struct AReg<3> { typedef v6i type; };

// WFMT = A (weight) format, XFMT = B (activation) format: the cbsz / blgp fields.
// GUARD: three wait states inside the statement, ahead of the MFMA.  The compiler takes the
// statement for opaque code, so it inserts no wait after its own vector writes of the operand
// registers (copies into the registers the statement asks for, shifted scale words); a VALU
// write needs two wait states before an MFMA reads the register.  Kernels whose assembly has
// such writes within two instructions of the MFMA take the guard.
template <int WFMT, int XFMT, int Q, bool GUARD = false, class TA, class TB>
__device__ __forceinline__ void mfma_inplace(v4f& acc, const TA& a, const TB& b, uint32_t sa,
                                             uint32_t sb) {
  static_assert(Q >= 0 && Q < 4, "op-select byte");
  static_assert(std::is_same<TA, typename AReg<WFMT>::type>::value &&
                    std::is_same<TB, typename AReg<XFMT>::type>::value,
                "operand register images: 8 registers for E4M3, 6 for FP6");
  static_assert(XFMT == 0 || WFMT != 0, "FP6 activations go with FP6 weights");
#if defined(__HIP_DEVICE_COMPILE__)   // the VGPR operand constraints exist for gfx950 only
  if constexpr (GUARD) MX_MFMA_FMT("s_nop 2\n\t");
  else MX_MFMA_FMT("");
#endif
}

// Activation (B) operand of one 16-row group from the LDS tile.  E4M3: two 16-byte pieces (K
// bytes 16 g.. and 64 + 16 g.. of the row).  FP6: block g's 24 bytes, a whole 16-byte chunk `p`
// and the 8-byte half `q` of its neighbour, which comes first for odd g.
template <int XFMT>
__device__ __forceinline__ typename AReg<XFMT>::type lds_b_operand(const uint8_t* p,
                                                                  const uint8_t* q, bool godd) {
  if constexpr (XFMT == 0) {
    const v4i lo = *(const v4i*)p, hi = *(const v4i*)q;
    return (v8i){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  } else {
    const v4i x = *(const v4i*)p;
    const v2i h = *(const v2i*)q;
    return godd ? (v6i){h[0], h[1], x[0], x[1], x[2], x[3]} : (v6i){x[0], x[1], x[2], x[3], h[0], h[1]};
  }
}

// Tile geometry: 8 waves (2 per SIMD) in a 2 (n) x 4 (m) grid; each wave owns FN weight
// fragments (16 rows each) and FM activation groups (16 rows each).  Workgroup tile =
// 32 FN weight rows x 64 FM activation rows; S LDS stages (the K step being computed plus
// S - 1 prefetched).  Two waves per SIMD: while one waits on LDS or the barrier, the other
// keeps the matrix pipe busy, and together they draw about twice the LDS read bandwidth of one.
// XFMT is the activations' format: E4M3 (128 bytes per row and K step) or, with FP6 weights,
// E2M3 / E3M2 (96 bytes: four 24-byte blocks); the LDS row slot stays 128 bytes either way.
template <int WFMT, int XFMT, int FN, int FM, int S>
struct TileCfg {
  static constexpr int NW = 8, WGN = 2, WGM = 4;
  // The copies are issued by waves 0-3 only, one per SIMD (waves w and w + 4 share a SIMD):
  // a wave stalls while it issues a copy, and the SIMD's other wave keeps the matrix pipe busy
  // meanwhile (all eight waves issuing their share measured 5-6 % slower, two or one slower
  // still).
  static constexpr int NDW = 4;
  static constexpr int FB = frag_bytes(WFMT);
  static constexpr int XB = XFMT == 0 ? 128 : 96;  // activation bytes per row per K step
  static constexpr int BN = 16 * FN * WGN, BM = 16 * FM * WGM;
  static constexpr int A_BYTES = (BN / 16) * FB;   // BN weight rows x one K step
  static constexpr int B_BYTES = BM * 128;         // BM activation rows x 128 bytes
  static constexpr int STAGE = A_BYTES + B_BYTES;
  static constexpr int A_CHUNKS = A_BYTES / 1024;  // 1 KiB DMA instructions
  static constexpr int A_PER_WAVE = (A_CHUNKS + NDW - 1) / NDW;   // surplus slots -> scratch
  static constexpr int B_PER_WAVE = B_BYTES / 1024 / NDW;
  static constexpr int D = A_PER_WAVE + B_PER_WAVE;   // vector-memory ops per copy wave per step
  // scales of 4 K steps ("group") staged in LDS: the weight's BN/16 fragments x 64 lane words,
  // moved 4 fragments (1 KiB) per 16-byte DMA; the activations' BM rows x 16 B, moved 16 rows
  // (256 B) per 4-byte DMA, since a row's 16 bytes need not be 16-byte aligned
  static constexpr int SA_PIECES = (BN / 16 + 3) / 4, SB_PIECES = BM / 16;
  static constexpr int SA_PER_WAVE = (SA_PIECES + NDW - 1) / NDW;
  static constexpr int SB_PER_WAVE = (SB_PIECES + NDW - 1) / NDW;
  static constexpr int SA_BYTES = SA_PIECES * 1024, SB_BYTES = SB_PIECES * 256;
  static constexpr int SCALE_BYTES = SA_BYTES + SB_BYTES;
  static constexpr int SL = SA_PER_WAVE + SB_PER_WAVE;  // scale DMAs per copy wave per group
  static constexpr int SCRATCH = 1024;                  // target of surplus DMA slots
  // epilogue: bf16 tile [BM][BN]; a row pitch of 16 (mod 256) bytes puts the 8-byte writes of
  // a wave (16 rows x 4 column groups) on distinct bank pairs
  static constexpr int OUT_PITCH = (BN * 2 - 16 + 255) / 256 * 256 + 16;
  static constexpr int LDS_MAIN = S * STAGE + 2 * SCALE_BYTES + SCRATCH;
  static constexpr int LDS_BYTES = LDS_MAIN > BM * OUT_PITCH ? LDS_MAIN : BM * OUT_PITCH;
  static_assert(A_BYTES % 1024 == 0 && B_BYTES % (1024 * NDW) == 0, "1 KiB DMA chunks");
  static_assert(S >= 2 && LDS_BYTES <= 160 * 1024, "must fit the 160 KiB LDS");
  // vector-memory ops issued after the DMA of step kt when step kt starts (q = kt % 4): the
  // DMAs of the next S - 2 steps, plus one group of scale DMAs if one was issued in between
  // (scale DMAs go out right after the DMA of each group's first step).
  static constexpr int vm_after(int q) { return (S - 2) * D + ((q >= 1 && q <= S - 1) ? SL : 0); }
  static_assert(vm_after(1) <= 63, "vmcnt is a 6-bit counter");
  static_assert(S <= 4, "the scale DMAs of a group must retire before the group's first step");
};

// s_waitcnt vmcnt(N) lgkmcnt(0) (expcnt not waited), then the workgroup barrier.  A plain
// barrier is used instead of __syncthreads(), whose fence would wait for every DMA in flight.
template <int N>
__device__ __forceinline__ void wait_vm_barrier() {
  static_assert(N >= 0 && N <= 63, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (0 << 8) | ((N >> 4) << 14));
  __builtin_amdgcn_s_barrier();
}

// Epilogue of the eight-wave kernels: bias, bf16 rounding, through LDS as a row-major [BM][BN]
// tile (rows padded by 16 B so the 8-byte writes of a wave hit distinct banks), then 16-byte
// coalesced stores.  Lane holds n = 16 (wn FN + i) + 4 g + (0..3) of activation row
// wm 16 FM + 16 j + r.  The caller has finished with the LDS stages (all copies landed, all
// waves past a barrier) and given the last MFMAs their result latency.
template <class C, int FN, int FM>
__device__ __forceinline__ void store_tile(uint8_t* lds, const v4f (&acc)[FN][FM],
                                           const uint16_t* __restrict__ bias,
                                           uint16_t* __restrict__ y, int M, int N, int m0, int n0,
                                           int wn, int wm, int r, int g, int tid) {
#pragma unroll
  for (int i = 0; i < FN; ++i) {
    const int nl = wn * 16 * FN + 16 * i + 4 * g;
    float bv[4] = {0.f, 0.f, 0.f, 0.f};
    if (bias && n0 + nl < N) {
#pragma unroll
      for (int e = 0; e < 4; ++e) bv[e] = bf16_to_float(bias[n0 + nl + e]);
    }
#pragma unroll
    for (int j = 0; j < FM; ++j) {
      const int ml = wm * 16 * FM + 16 * j + r;
      const v2i o = {(int)pack_bf16x2(acc[i][j][0] + bv[0], acc[i][j][1] + bv[1]),
                     (int)pack_bf16x2(acc[i][j][2] + bv[2], acc[i][j][3] + bv[3])};
      *(v2i*)(lds + ml * C::OUT_PITCH + nl * 2) = o;
    }
  }
  __syncthreads();
  // non-temporal stores: the output streams out instead of displacing the operand panels that
  // the running tiles still read from the caches (about 8 % on the prefill GEMM with operands
  // and outputs rotated over more memory than the Infinity Cache holds)
  constexpr int ROW_PIECES = C::BN * 2 / 16;          // 16-byte pieces per tile row
#pragma unroll 4
  for (int p = tid; p < C::BM * ROW_PIECES; p += C::NW * 64) {
    const int ml = p / ROW_PIECES, cp = p - ml * ROW_PIECES;
    const int m = m0 + ml, n = n0 + cp * 8;
    if (m < M && n < N)
      __builtin_nontemporal_store(*(const v4i*)(lds + ml * C::OUT_PITCH + cp * 16), (v4i*)(y + (int64_t)m * N + n));
  }
}

template <int WFMT, int XFMT, int FN, int FM, int S>
__global__ __launch_bounds__(512, 2) void k_gemm_tile(const uint8_t* __restrict__ xq,
                                                      const uint8_t* __restrict__ xs, int M, int K,
                                                      const uint8_t* __restrict__ packed, int N,
                                                      const uint16_t* __restrict__ bias,
                                                      uint16_t* __restrict__ y, int tiles_m,
                                                      int tiles_n, int group_m, BatchStrides bs,
                                                      float* __restrict__ part) {
  using C = TileCfg<WFMT, XFMT, FN, FM, S>;
  MX_BATCH_OFFSET(blockIdx.y);
  __shared__ __attribute__((aligned(1024))) uint8_t lds[C::LDS_BYTES];
  uint8_t* const slds = lds + S * C::STAGE;                  // two group-scale buffers
  uint8_t* const scratch = slds + 2 * C::SCALE_BYTES;        // surplus DMA slots land here

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wn = wave & 1, wm = wave >> 1;
  const int r = lane & 15, g = lane >> 4;

  // ---- tile of this workgroup: workgroups go round-robin to the 8 XCDs; give each XCD a
  // contiguous range of tiles, ordered in groups of group_m activation-row tiles so the tiles
  // running together on one XCD share operand panels in its L2.
  const int T = tiles_m * tiles_n;
  const int bid = blockIdx.x, xcd = bid & 7, slot = bid >> 3;
  const int t = xcd * (T >> 3) + (xcd < (T & 7) ? xcd : (T & 7)) + slot;
  const int gsz = group_m * tiles_n;
  const int first_m = (t / gsz) * group_m;
  const int gm = min(tiles_m - first_m, group_m);
  const int tm = first_m + (t % gsz) % gm;
  const int tn = (t % gsz) / gm;
  const int n0 = tn * C::BN, m0 = tm * C::BM;

  const int NG = N >> 4, KB = K >> 5;
  // bytes per K step of an activation row in global memory (FP6: packed 96, or 128-byte slices)
  const int XS = XFMT != 0 && bs.xstep ? bs.xstep : C::XB;
  const int LDX = K / 128 * XS;      // activation row bytes
  const uint32_t* wsc = (const uint32_t*)(packed + (int64_t)(K >> 7) * NG * C::FB);
  // K part of this workgroup (split K: grid z, whole groups of four K steps; one part unless
  // `part` is given): the operand and scale bases move to the part's first step
  const int pz = blockIdx.z, NP = gridDim.z;
  const int G = ((K >> 7) + 3) >> 2;
  const int g_lo = (int)((int64_t)pz * G / NP), g_hi = (int)((int64_t)(pz + 1) * G / NP);
  const int kt_lo = 4 * g_lo;
  const int KT = min(K >> 7, 4 * g_hi) - kt_lo;   // K steps of this part
  const int KBr = KB - 4 * kt_lo;                 // scale bytes of a row from this part on
  packed += (int64_t)kt_lo * NG * C::FB;
  wsc += (int64_t)g_lo * NG * 64;
  xq += (int64_t)kt_lo * XS;
  xs += 4 * kt_lo;

  // ---- per-lane DMA sources, as 32-bit offsets from uniform bases (every operand < 2^31 B):
  // each DMA address is then a 64-bit scalar base plus a 32-bit lane offset, the instruction's
  // own base + offset form, and no 64-bit per-lane address stays live
  // A: copy wave w copies 1 KiB chunks w, w + 4, ... of the stage's A block (fragments clamped to
  // NG); chunk indices past the block are surplus slots aimed at the scratch area
  // (E4M3 fragments are 2 KiB, so a chunk lies in one fragment and the offset is uniform +
  // lane * 16; FP6 fragments are 1.5 KiB and a chunk may straddle two, so the offset is per lane)
  uint32_t a_off[C::A_PER_WAVE];
#pragma unroll
  for (int i = 0; i < C::A_PER_WAVE; ++i) {
    const int c = min(wave + C::NDW * i, C::A_CHUNKS - 1);
    if (C::FB % 1024 == 0) {
      const int f = c * 1024 / C::FB;
      a_off[i] = (uint32_t)(min((n0 >> 4) + f, NG - 1) * C::FB + (c * 1024 - f * C::FB));
    } else {
      const int off = c * 1024 + lane * 16;
      const int f = off / C::FB;
      a_off[i] = (uint32_t)(min((n0 >> 4) + f, NG - 1) * C::FB + (off - f * C::FB));
    }
  }
  const uint32_t a_lane = C::FB % 1024 == 0 ? (uint32_t)lane * 16 : 0u;
  // B: copy wave w copies rows 8 c .. 8 c + 7 for c = w, w + 4, ..., lane -> (row, slot); an FP6
  // row has 6 chunks, so the lanes of slots holding chunks 6 and 7 stay idle
  uint32_t b_off[C::B_PER_WAVE];
  bool b_on[C::B_PER_WAVE];
#pragma unroll
  for (int i = 0; i < C::B_PER_WAVE; ++i) {
    const int row = 8 * (wave + C::NDW * i) + (lane >> 3);
    const int chunk = (lane & 7) ^ swz(row);
    b_on[i] = chunk < C::XB / 16;
    b_off[i] = (uint32_t)(min(m0 + row, M - 1) * LDX + min(chunk, C::XB / 16 - 1) * 16);
  }
  // the p-th tile DMA of a step (p < D: weight chunks first, then activation rows)
  auto issue_one = [&](int kt, int stage, int p) __attribute__((always_inline)) {
    uint8_t* base = lds + stage * C::STAGE;
    if (p < C::A_PER_WAVE) {
      const int c = wave + C::NDW * p;     // wave-uniform
      dma16(packed + (uint32_t)(kt * NG * C::FB + a_off[p] + a_lane),
            c < C::A_CHUNKS ? base + c * 1024 : scratch);
    } else {
      const int i = p - C::A_PER_WAVE;
      if (XFMT == 0 || b_on[i])
        dma16(xq + (uint32_t)(kt * XS + b_off[i]), base + C::A_BYTES + (wave + C::NDW * i) * 1024);
    }
  };
  auto issue = [&](int kt, int stage) __attribute__((always_inline)) {
    if (wave < C::NDW) {
#pragma unroll
      for (int p = 0; p < C::D; ++p) issue_one(kt, stage, p);
    }
  };

  // ---- per-lane scale DMA sources
  // weight (16-byte DMA): chunk c moves fragments n0/16 + 4 c .. + 3, the 64 lane words of each
  // (fragments past N are clamped; their words land beyond the tile's and are never read)
  uint32_t sa_src[C::SA_PER_WAVE];
#pragma unroll
  for (int i = 0; i < C::SA_PER_WAVE; ++i) {
    const int c = min(wave + C::NDW * i, C::SA_PIECES - 1);
    sa_src[i] = (uint32_t)(min((n0 >> 4) + 4 * c + (lane >> 4), NG - 1) * 256 + (lane & 15) * 16);
  }
  // activations: piece c moves rows 16 c .. 16 c + 15, 4 words (16 B) each; lane l takes row
  // 16 c + l / 4, word l % 4 (columns clamped inside the row at issue time)
  uint32_t sb_src[C::SB_PER_WAVE];
#pragma unroll
  for (int i = 0; i < C::SB_PER_WAVE; ++i) {
    const int c = min(wave + C::NDW * i, C::SB_PIECES - 1);
    sb_src[i] = (uint32_t)(min(m0 + 16 * c + (lane >> 2), M - 1) * KB);
  }
  const int q4 = (lane & 3) * 4;
  auto issue_scales = [&](int kt4, int sbuf) __attribute__((always_inline)) {
    uint8_t* base = slds + sbuf * C::SCALE_BYTES;
    if (wave >= C::NDW) return;
#pragma unroll
    for (int i = 0; i < C::SA_PER_WAVE; ++i) {
      const int c = wave + C::NDW * i;
      dma16((const uint8_t*)wsc + (uint32_t)(kt4 * NG * 256 + sa_src[i]),
            c < C::SA_PIECES ? base + c * 1024 : scratch);
    }
    const int col = min(16 * kt4 + q4, KBr - 4);
#pragma unroll
    for (int i = 0; i < C::SB_PER_WAVE; ++i) {
      const int c = wave + C::NDW * i;
      dma4(xs + (uint32_t)(sb_src[i] + col), c < C::SB_PIECES ? base + C::SA_BYTES + c * 256 : scratch);
    }
  };
  const uint32_t psel = (uint32_t)g | ((uint32_t)(4 + g) << 8) | ((uint32_t)g << 16) | ((uint32_t)(4 + g) << 24);
  // this lane's op-select scale words of group kt4 from buffer sbuf
  auto read_scales = [&](int kt4, int sbuf, uint32_t* sa, uint32_t* sb) __attribute__((always_inline)) {
    const uint8_t* base = slds + sbuf * C::SCALE_BYTES;
#pragma unroll
    for (int i = 0; i < FN; ++i) sa[i] = *(const uint32_t*)(base + (wn * FN + i) * 256 + lane * 4);
    const int left = KBr - 16 * kt4;   // scale bytes of a row from this group on
#pragma unroll
    for (int j = 0; j < FM; ++j) {
      const v4i w = *(const v4i*)(base + C::SA_BYTES + (wm * 16 * FM + 16 * j + r) * 16);
      uint32_t d[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) d[q] = (4 * q < left) ? (uint32_t)w[q] : 0x7F7F7F7Fu;
      const uint32_t t01 = __builtin_amdgcn_perm(d[1], d[0], psel);
      const uint32_t t23 = __builtin_amdgcn_perm(d[3], d[2], psel);
      sb[j] = __builtin_amdgcn_perm(t23, t01, 0x05040100u);
    }
    // two wait states between these VALU-written scale words and the (assembly) MFMAs that
    // read them; the scheduling barrier keeps the writes above the nops
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_nop 2" ::: "memory");
  };

  v4f acc[FN][FM];
#pragma unroll
  for (int i = 0; i < FN; ++i)
#pragma unroll
    for (int j = 0; j < FM; ++j) acc[i][j] = (v4f){0.f, 0.f, 0.f, 0.f};

  typedef typename AReg<WFMT>::type AR;
  typedef typename AReg<XFMT>::type BR;
  auto load_a = [&](const uint8_t* base, int i) __attribute__((always_inline)) {
    const uint8_t* fa = base + (wn * FN + i) * C::FB;
    const v4i lo = *(const v4i*)(fa + lane * 16);
    if constexpr (WFMT == 0) {
      const v4i hi = *(const v4i*)(fa + 1024 + lane * 16);
      return (AR){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    } else {
      const v2i hi = *(const v2i*)(fa + 1024 + lane * 8);
      return (AR){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1]};
    }
  };
  // One K step's MFMAs from LDS stage `stage`.  LDS reads run one weight fragment ahead of the
  // MFMAs (fragment 0 first, then the activation fragments, then fragment i + 1 before the
  // MFMAs of fragment i), pinned with scheduling-group barriers.
  // activation rows of this lane are wm 16 FM + 16 j + r: all share row & 15 == r and so the
  // swizzle, leaving one address per half and a constant 2 KiB step per j
  const uint32_t b_lo = (uint32_t)((wm * 16 * FM + r) * 128 + ((g ^ swz(r)) << 4));
  const uint32_t b_hi = (uint32_t)((wm * 16 * FM + r) * 128 + (((4 + g) ^ swz(r)) << 4));
  // FP6: block g is bytes [24 g, 24 g + 24) of the row slice, i.e. chunk 3g/2 in full plus
  // half of its neighbour (after it for even g, before it for odd g)
  const bool godd = (g & 1) != 0;
  const int c_full = (3 * g + 1) >> 1, c_half = godd ? c_full - 1 : c_full + 1;
  const uint32_t bx_off = (uint32_t)((wm * 16 * FM + r) * 128 + ((c_full ^ swz(r)) << 4));
  const uint32_t by_off = (uint32_t)((wm * 16 * FM + r) * 128 + ((c_half ^ swz(r)) << 4) + (godd ? 8 : 0));
  // `mid` runs once the first operand reads are issued and before the first MFMA: the step's
  // DMAs go out there, so their issue overlaps the LDS read latency instead of delaying it.
  // operands of the previous step's last weight fragment: its MFMAs run after the next
  // barrier, covering the latency of that step's first LDS reads (same order per accumulator)
  // The last TN MFMAs of a step (last weight fragment x last TN activation tiles) run at the
  // top of the next step, after its barrier and first LDS reads, so that the two waves of a SIMD
  // do not both stall on those reads with an empty matrix pipe; each accumulator still sees
  // the K steps in order, so results do not change.  The 8 x 4 tile has no registers to spare.
  constexpr int TN = FN >= 8 ? 0 : (FM < 2 ? FM : 2);
  AR a_tail;
  BR b_tail[TN > 0 ? TN : 1];
  uint32_t sa_tail = 0, sb_tail[TN > 0 ? TN : 1];
  auto run_tail = [&](bool have) __attribute__((always_inline)) {
    if (TN > 0 && have) {
      asm volatile("s_nop 2" ::: "memory");   // the tail scale words are VALU-written
#pragma unroll
      for (int j = 0; j < TN; ++j) mfma_inplace<WFMT, XFMT, 0, true>(acc[FN - 1][FM - TN + j], a_tail, b_tail[j], sa_tail, sb_tail[j]);
    }
  };
  auto compute = [&](int stage, auto qc, const uint32_t* sa_in, const uint32_t* sb_in, int sh, bool have_tail, auto&& mid) __attribute__((always_inline)) {
    constexpr int Q = decltype(qc)::value;
    // remainder steps: the step's scale byte shifted into byte 0 (op-select 0); the nops keep
    // two wait states between these VALU writes and the MFMAs that read them
    uint32_t sa[FN], sb[FM];
#pragma unroll
    for (int i = 0; i < FN; ++i) sa[i] = Q >= 0 ? sa_in[i] : sa_in[i] >> sh;
#pragma unroll
    for (int j = 0; j < FM; ++j) sb[j] = Q >= 0 ? sb_in[j] : sb_in[j] >> sh;
    if constexpr (Q < 0) {
      __builtin_amdgcn_sched_barrier(0);
      asm volatile("s_nop 2" ::: "memory");
    }
    const uint8_t* base = lds + stage * C::STAGE;
    const uint8_t* bl = base + C::A_BYTES;
    AR a = load_a(base, 0);
    BR b[FM];
#pragma unroll
    for (int j = 0; j < FM; ++j)
      b[j] = lds_b_operand<XFMT>(bl + (XFMT == 0 ? b_lo : bx_off) + j * 2048,
                                 bl + (XFMT == 0 ? b_hi : by_off) + j * 2048, godd);
    AR an = FN > 1 ? load_a(base, 1) : a;
    __builtin_amdgcn_sched_barrier(0);
    run_tail(have_tail);
    __builtin_amdgcn_sched_barrier(0);
    mid();
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < FN; ++i) {
      AR an2 = an;
      if (i + 2 < FN) {
        an2 = load_a(base, i + 2);
      }
#pragma unroll
      for (int j = 0; j < (i == FN - 1 ? FM - TN : FM); ++j) {
        mfma_inplace<WFMT, XFMT, (Q >= 0 ? Q : 0), true>(acc[i][j], a, b[j], sa[i], sb[j]);
      }
      __builtin_amdgcn_sched_barrier(0);
      if (i < FN - 1) {
        a = an;
        an = an2;
      }
    }
    // the last TN MFMAs wait for the next step (their scale words shifted to byte 0)
    constexpr int QS = Q >= 0 ? 8 * Q : 0;
    a_tail = a;
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      b_tail[j] = b[FM - TN + j];
      sb_tail[j] = sb[FM - TN + j] >> QS;
    }
    sa_tail = sa[FN - 1] >> QS;
    __builtin_amdgcn_sched_barrier(0);
  };

  uint32_t sa[FN], sb[FM];
  const int KT4 = (KT + 3) >> 2;
  const int KT4f = KT >> 2;               // groups of four whole K steps
  // prologue: scales of group 0 and the DMAs of steps 0 .. S-2 go out together; the scales
  // are waited for (the tile DMAs of steps 1 .. S-2 may still be in flight) and read
  issue_scales(0, 0);
#pragma unroll
  for (int st = 0; st < S - 1; ++st) issue(min(st, KT - 1), st);
  wait_vm_barrier<(S - 1) * C::D>();
  read_scales(0, 0, sa, sb);

  // One K step of a full group.  At the top, the tiles of step kt have landed once at most
  // vm_after(q) later memory operations are outstanding (vmcnt retires in issue order); the
  // DMA of step kt + S - 1 then goes to the stage freed by step kt - 1 (past the last step the
  // last step is fetched again, unused: the operation count per step never changes).  The
  // first step of a group reads the group's scales and sends the next group's scale DMAs.
  auto step = [&](int kt, auto qc) __attribute__((always_inline)) {
    constexpr int Q = decltype(qc)::value;
    __builtin_amdgcn_sched_barrier(0);
    wait_vm_barrier<C::vm_after(Q)>();
    if (Q == 0 && kt > 0) read_scales(kt >> 2, (kt >> 2) & 1, sa, sb);
    // this step's DMAs: tile DMAs first, then (first step of a group) the scale DMAs
    compute(kt % S, qc, sa, sb, 0, kt > 0, [&]() __attribute__((always_inline)) {
      issue(min(kt + S - 1, KT - 1), (kt + S - 1) % S);
      if (Q == 0) issue_scales(min((kt >> 2) + 1, KT4 - 1), ((kt >> 2) + 1) & 1);
    });
  };
  for (int kt4 = 0; kt4 < KT4f; ++kt4) {
    step(4 * kt4 + 0, std::integral_constant<int, 0>());
    step(4 * kt4 + 1, std::integral_constant<int, 1>());
    step(4 * kt4 + 2, std::integral_constant<int, 2>());
    step(4 * kt4 + 3, std::integral_constant<int, 3>());
  }
  // remainder steps (K / 128 not a multiple of 4): everything waited for, no prefetch
  for (int kt = 4 * KT4f; kt < KT; ++kt) {
    wait_vm_barrier<0>();
    if (kt == 4 * KT4f && KT4f > 0) read_scales(KT4f, KT4f & 1, sa, sb);
    compute(kt % S, std::integral_constant<int, -1>(), sa, sb, 8 * (kt & 3), kt > 0, [&]() __attribute__((always_inline)) {
      if (kt + S - 1 < KT) issue(kt + S - 1, (kt + S - 1) % S);
    });
  }
  run_tail(KT > 0);
  // all DMAs landed and all waves done with the stages before LDS is reused for the output;
  // the nops give the last MFMAs (issued as assembly, so untracked by the compiler's hazard
  // checks) their result latency before VALU code reads the accumulators
  wait_vm_barrier<0>();
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_nop 15\n s_nop 15\n s_nop 15" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);

  if (part) {
    // split K: this part's fp32 sums, row-major [part][M][N], for k_splitk_reduce to add in part
    // order (bias and rounding there); written once, read once: non-temporal
    float* pp = part + (int64_t)pz * M * N;
#pragma unroll
    for (int i = 0; i < FN; ++i) {
      const int n = n0 + wn * 16 * FN + 16 * i + 4 * g;
#pragma unroll
      for (int j = 0; j < FM; ++j) {
        const int m = m0 + wm * 16 * FM + 16 * j + r;
        if (m < M && n < N) __builtin_nontemporal_store(acc[i][j], (v4f*)(pp + (int64_t)m * N + n));
      }
    }
    return;
  }

  store_tile<C, FN, FM>(lds, acc, bias, y, M, N, m0, n0, wn, wm, r, g, tid);
}

// ---------------------------------------------------------------- ping-pong kernel
// The eight waves of k_gemm_tile's geometry as two groups of four, one wave of each group per
// SIMD (waves w and w + 4 share a SIMD): group 0 (waves 0-3) owns the tile's activation rows
// 0 .. BM/2 - 1, group 1 the rest, each group's four waves splitting its rows 2 (n) x 2 (m).  The
// groups run half a K step apart: in each phase one group issues all MFMAs of a K step from
// registers while the other reads its next step's operands from LDS into registers and issues
// copies; a workgroup barrier ends each phase.  A SIMD's matrix pipe is then fed by one wave at
// a time and never waits on LDS latency, and each wave's memory work runs under its partner's
// MFMAs (the all-waves-in-step kernel spends a fifth of its wave time waiting at the barrier and
// on the first operand reads of each step).
//
// Phases, for K step k: in phase 2k group 0 computes step k and group 1 reads it; in phase
// 2k + 1 group 1 computes step k and group 0 reads step k + 1.  LDS holds three weight stages
// and two activation stages (step k in weight stage k % 3, activation stage k % 2) and one
// buffer of group scales.  The copies go out from the computing waves, one after every few
// MFMAs, so that the L1 (64 B/clk per CU, about 18 clocks per 1 KiB copy) never backs up and
// a read phase is LDS reads alone: in phase 2k group 0 copies its activation rows and its
// share of the weight tile of step k + 2, in phase 2k + 1 group 1 its activation rows of step
// k + 2 and its weight share of step k + 3, each into a stage whose readers are done, each
// with at least two and a half phases to land.  A wave waits for its copies of a phase by the
// end of its next phase but one; the barriers then publish them.  Past the last step the last
// step is copied again, unused, so that every wait count is a constant.  Group 0 copies the
// scales of the next four-step group in a read phase once both groups have read the current
// one.  K % 512 == 0 (whole scale groups); results equal k_gemm_tile's bit for bit (the same
// MFMAs, each accumulator taking the K steps in order).
template <int WFMT, int XFMT, int FN, int FM>
struct PPCfg {
  using C = TileCfg<WFMT, XFMT, FN, FM, 2>;
  static constexpr int GW = 4;                                           // waves per group
  static constexpr int A_PW0 = (C::A_CHUNKS + 2 * GW - 1) / (2 * GW);    // weight chunks per wave
  static constexpr int A_PW1 = (C::A_CHUNKS - GW * A_PW0 + GW - 1) / GW; // (surplus -> scratch)
  static constexpr int A_PWM = A_PW0 > A_PW1 ? A_PW0 : A_PW1;
  static constexpr int B_PW = C::B_BYTES / 1024 / (2 * GW);              // activation chunks per wave
  static constexpr int SA_PW = (C::SA_PIECES + GW - 1) / GW, SB_PW = (C::SB_PIECES + GW - 1) / GW;
  static constexpr int OFF_B = 3 * C::A_BYTES;
  static constexpr int OFF_S = OFF_B + 2 * C::B_BYTES;
  static constexpr int OFF_SCR = OFF_S + C::SCALE_BYTES;
  static constexpr int LDS_MAIN = OFF_SCR + 1024;
  static constexpr int LDS_BYTES = LDS_MAIN > C::BM * C::OUT_PITCH ? LDS_MAIN : C::BM * C::OUT_PITCH;
  static_assert(LDS_BYTES <= 160 * 1024, "must fit the 160 KiB LDS");
  static_assert(C::B_BYTES % (2048 * GW) == 0, "each group copies its own activation rows");
  static_assert(GW * (A_PW0 + A_PW1) >= C::A_CHUNKS, "weight chunk split");
  static_assert(B_PW + A_PWM + SA_PW + SB_PW <= 63, "vmcnt is a 6-bit counter");
};

// s_waitcnt vmcnt(VM) lgkmcnt(0) (VM = 63: no vector-memory wait), then the workgroup barrier;
// the empty assembly statements keep the compiler from moving LDS accesses across it
template <int VM>
__device__ __forceinline__ void pp_wait_barrier() {
  static_assert(VM >= 0 && VM <= 63, "vmcnt range");
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt((VM & 15) | (7 << 4) | (0 << 8) | ((VM >> 4) << 14));
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

template <int WFMT, int XFMT, int FN, int FM>
__global__ __launch_bounds__(512, 2) void k_gemm_pp(const uint8_t* __restrict__ xq,
                                                    const uint8_t* __restrict__ xs, int M, int K,
                                                    const uint8_t* __restrict__ packed, int N,
                                                    const uint16_t* __restrict__ bias,
                                                    uint16_t* __restrict__ y, int tiles_m,
                                                    int tiles_n, int group_m, BatchStrides bs) {
  using C = TileCfg<WFMT, XFMT, FN, FM, 2>;
  using P = PPCfg<WFMT, XFMT, FN, FM>;
  constexpr int GW = P::GW;
  MX_BATCH_OFFSET(blockIdx.y);
  __shared__ __attribute__((aligned(1024))) uint8_t lds[P::LDS_BYTES];
  uint8_t* const lds_b = lds + P::OFF_B;
  uint8_t* const slds = lds + P::OFF_S;
  uint8_t* const scratch = lds + P::OFF_SCR;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wn = wave & 1, wm = wave >> 1;
  const int r = lane & 15, g = lane >> 4;
  const bool g1 = wave >= GW;                             // wave-uniform
  const int w4 = wave & (GW - 1);

  // tile of this workgroup: as k_gemm_tile (XCD-contiguous ranges, group_m row tiles per group)
  const int T = tiles_m * tiles_n;
  const int bid = blockIdx.x, xcd = bid & 7, slot = bid >> 3;
  const int t = xcd * (T >> 3) + (xcd < (T & 7) ? xcd : (T & 7)) + slot;
  const int gsz = group_m * tiles_n;
  const int first_m = (t / gsz) * group_m;
  const int gm = min(tiles_m - first_m, group_m);
  const int tm = first_m + (t % gsz) % gm;
  const int tn = (t % gsz) / gm;
  const int n0 = tn * C::BN, m0 = tm * C::BM;

  const int NG = N >> 4, KB = K >> 5, KT = K >> 7, G = KT >> 2;
  const int LDX = KT * C::XB;
  const uint32_t* wsc = (const uint32_t*)(packed + (int64_t)KT * NG * C::FB);

  // copy sources (32-bit offsets from uniform bases, as in k_gemm_tile).  Weight chunks: group 0
  // wave w takes chunks w, w + 4, .. below 4 A_PW0, group 1 wave 4 + w the chunks 4 A_PW0 + w, ..
  // (surplus slots to the scratch area).  Activation chunks (8 rows each): each group its rows.
  const int a_c0 = g1 ? GW * P::A_PW0 : 0;
  const int a_cend = g1 ? C::A_CHUNKS : GW * P::A_PW0;
  uint32_t a_off[P::A_PWM];
#pragma unroll
  for (int i = 0; i < P::A_PWM; ++i) {
    const int c = min(a_c0 + w4 + GW * i, C::A_CHUNKS - 1);
    if (C::FB % 1024 == 0) {
      const int f = c * 1024 / C::FB;
      a_off[i] = (uint32_t)(min((n0 >> 4) + f, NG - 1) * C::FB + (c * 1024 - f * C::FB));
    } else {
      const int off = c * 1024 + lane * 16;
      const int f = off / C::FB;
      a_off[i] = (uint32_t)(min((n0 >> 4) + f, NG - 1) * C::FB + (off - f * C::FB));
    }
  }
  const uint32_t a_lane = C::FB % 1024 == 0 ? (uint32_t)lane * 16 : 0u;
  const int cb0 = g1 ? C::B_BYTES / 2048 : 0;             // first activation chunk of the group
  uint32_t b_off[P::B_PW];
  bool b_on[P::B_PW];
#pragma unroll
  for (int i = 0; i < P::B_PW; ++i) {
    const int row = 8 * (cb0 + w4 + GW * i) + (lane >> 3);
    const int chunk = (lane & 7) ^ swz(row);
    b_on[i] = chunk < C::XB / 16;
    b_off[i] = (uint32_t)(min(m0 + row, M - 1) * LDX + min(chunk, C::XB / 16 - 1) * 16);
  }
  // copy i of this wave's weight share of step kt into weight stage `stage`
  auto copy_a = [&](int i, int kt, int stage) __attribute__((always_inline)) {
    const int c = a_c0 + w4 + GW * i;   // wave-uniform
    dma16(packed + (uint32_t)(kt * NG * C::FB + a_off[i] + a_lane),
          c < a_cend ? lds + stage * C::A_BYTES + c * 1024 : scratch);
  };
  // copy i of this wave's activation rows of step kt into activation stage `stage`
  auto copy_b = [&](int i, int kt, int stage) __attribute__((always_inline)) {
    if (XFMT == 0 || b_on[i])
      dma16(xq + (uint32_t)(kt * C::XB + b_off[i]), lds_b + stage * C::B_BYTES + (cb0 + w4 + GW * i) * 1024);
  };
  // scale copies (group 0): weight words 4 fragments per 16-byte copy, activation rows 16 per
  // 4-byte copy, as k_gemm_tile
  uint32_t sa_src[P::SA_PW], sb_src[P::SB_PW];
#pragma unroll
  for (int i = 0; i < P::SA_PW; ++i) {
    const int c = min(w4 + GW * i, C::SA_PIECES - 1);
    sa_src[i] = (uint32_t)(min((n0 >> 4) + 4 * c + (lane >> 4), NG - 1) * 256 + (lane & 15) * 16);
  }
#pragma unroll
  for (int i = 0; i < P::SB_PW; ++i) {
    const int c = min(w4 + GW * i, C::SB_PIECES - 1);
    sb_src[i] = (uint32_t)(min(m0 + 16 * c + (lane >> 2), M - 1) * KB);
  }
  const int q4 = (lane & 3) * 4;
  auto issue_scales = [&](int kt4) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < P::SA_PW; ++i) {
      const int c = w4 + GW * i;
      dma16((const uint8_t*)wsc + (uint32_t)(kt4 * NG * 256 + sa_src[i]),
            c < C::SA_PIECES ? slds + c * 1024 : scratch);
    }
#pragma unroll
    for (int i = 0; i < P::SB_PW; ++i) {
      const int c = w4 + GW * i;
      dma4(xs + (uint32_t)(sb_src[i] + 16 * kt4 + q4), c < C::SB_PIECES ? slds + C::SA_BYTES + c * 256 : scratch);
    }
  };

  typedef typename AReg<WFMT>::type AR;
  typedef typename AReg<XFMT>::type BR;
  AR a[FN];
  BR b[FM];
  uint32_t sa[FN], sb[FM];
  const uint32_t psel = (uint32_t)g | ((uint32_t)(4 + g) << 8) | ((uint32_t)g << 16) | ((uint32_t)(4 + g) << 24);
  auto read_scales = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < FN; ++i) sa[i] = *(const uint32_t*)(slds + (wn * FN + i) * 256 + lane * 4);
#pragma unroll
    for (int j = 0; j < FM; ++j) {
      const v4i w = *(const v4i*)(slds + C::SA_BYTES + (wm * 16 * FM + 16 * j + r) * 16);
      const uint32_t t01 = __builtin_amdgcn_perm((uint32_t)w[1], (uint32_t)w[0], psel);
      const uint32_t t23 = __builtin_amdgcn_perm((uint32_t)w[3], (uint32_t)w[2], psel);
      sb[j] = __builtin_amdgcn_perm(t23, t01, 0x05040100u);
    }
  };
  const uint32_t b_lo = (uint32_t)((wm * 16 * FM + r) * 128 + ((g ^ swz(r)) << 4));
  const uint32_t b_hi = (uint32_t)((wm * 16 * FM + r) * 128 + (((4 + g) ^ swz(r)) << 4));
  const bool godd = (g & 1) != 0;
  const int c_full = (3 * g + 1) >> 1, c_half = godd ? c_full - 1 : c_full + 1;
  const uint32_t bx_off = (uint32_t)((wm * 16 * FM + r) * 128 + ((c_full ^ swz(r)) << 4));
  const uint32_t by_off = (uint32_t)((wm * 16 * FM + r) * 128 + ((c_half ^ swz(r)) << 4) + (godd ? 8 : 0));
  // all operands of one K step into registers
  auto read_ops = [&](int astage, int bstage) __attribute__((always_inline)) {
    const uint8_t* base = lds + astage * C::A_BYTES;
    const uint8_t* bl = lds_b + bstage * C::B_BYTES;
#pragma unroll
    for (int j = 0; j < FM; ++j)
      b[j] = lds_b_operand<XFMT>(bl + (XFMT == 0 ? b_lo : bx_off) + j * 2048,
                                 bl + (XFMT == 0 ? b_hi : by_off) + j * 2048, godd);
#pragma unroll
    for (int i = 0; i < FN; ++i) {
      const uint8_t* fa = base + (wn * FN + i) * C::FB;
      const v4i lo = *(const v4i*)(fa + lane * 16);
      if constexpr (WFMT == 0) {
        const v4i hi = *(const v4i*)(fa + 1024 + lane * 16);
        a[i] = (AR){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      } else {
        const v2i hi = *(const v2i*)(fa + 1024 + lane * 8);
        a[i] = (AR){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1]};
      }
    }
  };

  v4f acc[FN][FM];
#pragma unroll
  for (int i = 0; i < FN; ++i)
#pragma unroll
    for (int j = 0; j < FM; ++j) acc[i][j] = (v4f){0.f, 0.f, 0.f, 0.f};
  // one K step's MFMAs with ND copies interleaved: copy c (copy(c) issues it) after MFMA
  // number 1 + c * SPACE, spread over the step
  auto compute = [&](auto qc, auto nd, auto&& copy) __attribute__((always_inline)) {
    constexpr int Q = decltype(qc)::value;
    constexpr int ND = decltype(nd)::value;
    constexpr int SPACE = (FN * FM - 1) / (ND > 1 ? ND : 1) > 0 ? (FN * FM - 1) / (ND > 1 ? ND : 1) : 1;
    // the scale words were written by VALU code before the last barrier; two wait states
    asm volatile("s_nop 1" ::: "memory");
#pragma unroll
    for (int i = 0; i < FN; ++i)
#pragma unroll
      for (int j = 0; j < FM; ++j) {
        mfma_inplace<WFMT, XFMT, Q>(acc[i][j], a[i], b[j], sa[i], sb[j]);
        const int mm = i * FM + j;   // a constant once unrolled
        if ((mm - 1) % SPACE == 0 && (mm - 1) / SPACE < ND && mm >= 1) {
          __builtin_amdgcn_sched_barrier(0);
          copy((mm - 1) / SPACE);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
  };
  const std::integral_constant<int, P::B_PW + P::A_PW0> nd0;
  const std::integral_constant<int, P::B_PW + P::A_PW1> nd1;
  const int KL = KT - 1;

  // prologue: steps 0 and 1, group 1's weight share of step 2 and scale group 0
  if (!g1) {
    issue_scales(0);
#pragma unroll
    for (int st = 0; st < 2; ++st) {
#pragma unroll
      for (int i = 0; i < P::B_PW; ++i) copy_b(i, min(st, KL), st);
#pragma unroll
      for (int i = 0; i < P::A_PW0; ++i) copy_a(i, min(st, KL), st);
    }
  } else {
#pragma unroll
    for (int st = 0; st < 2; ++st) {
#pragma unroll
      for (int i = 0; i < P::B_PW; ++i) copy_b(i, min(st, KL), st);
    }
#pragma unroll
    for (int st = 0; st < 3; ++st) {
#pragma unroll
      for (int i = 0; i < P::A_PW1; ++i) copy_a(i, min(st, KL), st);
    }
  }
  pp_wait_barrier<0>();
  // Each group runs its own loop (the branch is wave-uniform); both pass the same barriers, two
  // per K step, so the phases line up across the groups.
  if (!g1) {
    read_ops(0, 0);                       // phase -1: read step 0
    read_scales();
    pp_wait_barrier<63>();
    // phase 2 kt: compute step kt, copying group 0's activation rows and weight share of step
    // kt + 2; phase 2 kt + 1: read step kt + 1 (at a group's last step with the next group's
    // scales) and, at a group's first step, copy the next group's scales
    auto step = [&](int kt, auto qc) __attribute__((always_inline)) {
      constexpr int Q = decltype(qc)::value;
      const int k2 = min(kt + 2, KL);
      compute(qc, nd0, [&](int c) __attribute__((always_inline)) {
        if (c < P::B_PW) copy_b(c, k2, kt & 1);
        else copy_a(c - P::B_PW, k2, (kt + 2) % 3);
      });
      pp_wait_barrier<P::B_PW + P::A_PW0>();   // copies of two phases ago (step kt + 1)
      if (kt + 1 < KT) {
        read_ops((kt + 1) % 3, (kt + 1) & 1);
        if (Q == 3) read_scales();
      }
      if (Q == 0 && (kt >> 2) + 1 < G) issue_scales((kt >> 2) + 1);
      pp_wait_barrier<63>();
    };
    for (int kt = 0; kt < KT; kt += 4) {
      step(kt + 0, std::integral_constant<int, 0>());
      step(kt + 1, std::integral_constant<int, 1>());
      step(kt + 2, std::integral_constant<int, 2>());
      step(kt + 3, std::integral_constant<int, 3>());
    }
  } else {
    pp_wait_barrier<63>();                // phase -1: nothing to read yet
    // phase 2 kt: read step kt (at a group's first step with its scales); phase 2 kt + 1:
    // compute step kt, copying group 1's activation rows of step kt + 2 and its weight share of
    // step kt + 3
    auto step = [&](int kt, auto qc) __attribute__((always_inline)) {
      constexpr int Q = decltype(qc)::value;
      read_ops(kt % 3, kt & 1);
      if (Q == 0) read_scales();
      pp_wait_barrier<P::B_PW + P::A_PW1>();   // copies of three phases ago (weight of kt + 1)
      const int k2 = min(kt + 2, KL), k3 = min(kt + 3, KL);
      compute(qc, nd1, [&](int c) __attribute__((always_inline)) {
        if (c < P::B_PW) copy_b(c, k2, kt & 1);
        else copy_a(c - P::B_PW, k3, kt % 3);
      });
      pp_wait_barrier<P::B_PW + P::A_PW1>();   // copies of two phases ago (activations of kt + 1)
    };
    for (int kt = 0; kt < KT; kt += 4) {
      step(kt + 0, std::integral_constant<int, 0>());
      step(kt + 1, std::integral_constant<int, 1>());
      step(kt + 2, std::integral_constant<int, 2>());
      step(kt + 3, std::integral_constant<int, 3>());
    }
  }
  // every copy landed and every wave done with the stages before LDS takes the output tile; the
  // nops give the last MFMAs (assembly, so untracked by the compiler's hazard checks) their
  // result latency before VALU code reads the accumulators
  pp_wait_barrier<0>();
  asm volatile("s_nop 15\n s_nop 15\n s_nop 15" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
  store_tile<C, FN, FM>(lds, acc, bias, y, M, N, m0, n0, wn, wm, r, g, tid);
}

// ---------------------------------------------------------------- 4-wave kernel (large tiles)
// One wave per SIMD, 2 (n) x 2 (m) waves, each owning a 32 FNB x 32 FMB block of the output
// as FNB x FMB tiles of the 32x32x64 scaled MFMA, accumulators held in the AGPRs (256 of them
// for the 128 x 128 wave tile of the 256 x 256 workgroup tile).  Per 128-wide K step a wave
// reads (32 FNB + 32 FMB) x 128 operand bytes from LDS for 2 FNB FMB MFMAs: half the LDS reads
// per MFMA of the eight-wave kernel's 112 x 64 wave tiles, and 7 % fewer copied bytes per
// output (workgroup tile 256 x 256 against 224 x 256).
//
// 32x32x64 operand layout (measured on gfx950 with one-hot inputs): lane l = (R = l % 32,
// g = l / 32) holds row R's K bytes 32 h + 16 g + t (piece h = 0, 1, byte t < 16); the scale of
// row R, 32-block b comes from lane R + 32 b (op-select picks its byte); accumulator element e
// of lane l is C[8 (e / 4) + 4 (l / 32) + e % 4][l % 32].  A prepacked 16 x 128 fragment keeps
// K bytes 64 h' + 16 g' + t of row r in lane (r, g') of half h', so the operand of K half s is
// the 16-byte pieces (h' = s, g' = g) and (h' = s, g' = 2 + g): two LDS reads, 512 bytes apart.
//
// Pipeline: both stages of a step are copied global -> LDS one step ahead (direct-to-LDS, every
// wave issuing a share, interleaved one copy per MFMA).  Within a step the second K half's
// MFMAs are deferred past the next barrier: after it, a wave first issues the next step's
// first-half operand reads, then runs the deferred MFMAs (their operands are already in
// registers), so the matrix pipe is busy while the barrier resolves and the reads land.
// Results equal the other kernels' within the usual fp32 reordering; every accumulator takes
// its K steps in order.
template <int WFMT, int WGN, int FNB, int FMB>
struct W4Cfg {
  static constexpr int NW = 4, WGM = NW / WGN;            // wave grid WGN (n) x WGM (m)
  static constexpr int FB = frag_bytes(WFMT);
  static constexpr int BN = 32 * FNB * WGN, BM = 32 * FMB * WGM;
  static constexpr int A_BYTES = (BN / 16) * FB;
  static constexpr int B_BYTES = BM * 128;
  static constexpr int STAGE = A_BYTES + B_BYTES;
  static constexpr int A_CHUNKS = A_BYTES / 1024;
  static constexpr int A_PW = (A_CHUNKS + NW - 1) / NW;   // surplus slots -> scratch
  static constexpr int B_PW = B_BYTES / 1024 / NW;
  static constexpr int D = A_PW + B_PW;                   // tile copies per wave per step
  static constexpr int SA_PIECES = (BN / 16 + 3) / 4, SB_PIECES = BM / 16;
  static constexpr int SA_PW = (SA_PIECES + NW - 1) / NW, SB_PW = (SB_PIECES + NW - 1) / NW;
  static constexpr int SA_BYTES = SA_PIECES * 1024, SB_BYTES = SB_PIECES * 256;
  static constexpr int SCALE_BYTES = SA_BYTES + SB_BYTES;
  static constexpr int SCRATCH = 1024;
  static constexpr int OUT_PITCH = (BN * 2 - 16 + 255) / 256 * 256 + 16;
  static constexpr int LDS_MAIN = 2 * STAGE + 2 * SCALE_BYTES + SCRATCH;
  static constexpr int LDS_BYTES = LDS_MAIN > BM * OUT_PITCH ? LDS_MAIN : BM * OUT_PITCH;
  static_assert(WGN == 1 || WGN == 2 || WGN == 4, "wave grid");
  static_assert(A_BYTES % 1024 == 0 && B_BYTES % (1024 * NW) == 0, "1 KiB copy chunks");
  static_assert(LDS_BYTES <= 160 * 1024, "must fit the 160 KiB LDS");
  static_assert(FNB * FMB * 16 <= 256, "accumulators must fit the AGPRs");
};

#define MX_MFMA32_ASM(OPSEL, FMT)                                                               \
  asm volatile("v_mfma_scale_f32_32x32x64_f8f6f4 %0, %1, %2, %0, %3, %4 " OPSEL FMT          \
               : "+a"(acc) : "v"(a), "v"(b), "v"(sa), "v"(sb))
#define MX_MFMA32_Q(FMT)                                            \
  do {                                                              \
    if constexpr (Q == 0) MX_MFMA32_ASM(MX_MFMA_OPSEL_0, FMT);      \
    else if constexpr (Q == 1) MX_MFMA32_ASM(MX_MFMA_OPSEL_1, FMT); \
    else if constexpr (Q == 2) MX_MFMA32_ASM(MX_MFMA_OPSEL_2, FMT); \
    else MX_MFMA32_ASM(MX_MFMA_OPSEL_3, FMT);                       \
  } while (0)

// 32x32x64 scaled MFMA, accumulating in place in AGPRs (A = weight format, B = E4M3)
template <int WFMT, int Q, class TA>
__device__ __forceinline__ void mfma32_inplace(v16f& acc, const TA& a, const v8i& b, uint32_t sa,
                                               uint32_t sb) {
  static_assert(Q >= 0 && Q < 4, "op-select byte");
  static_assert(std::is_same<TA, typename AReg<WFMT>::type>::value, "operand register image");
#if defined(__HIP_DEVICE_COMPILE__)
  if constexpr (WFMT == 0) MX_MFMA32_Q("");
  else if constexpr (WFMT == 2) MX_MFMA32_Q(" cbsz:2");
  else MX_MFMA32_Q(" cbsz:3");
#endif
}

template <int WFMT, int WGN, int FNB, int FMB>
__global__ __launch_bounds__(256, 1) void k_gemm_w4(const uint8_t* __restrict__ xq,
                                                    const uint8_t* __restrict__ xs, int M, int K,
                                                    const uint8_t* __restrict__ packed, int N,
                                                    const uint16_t* __restrict__ bias,
                                                    uint16_t* __restrict__ y, int tiles_m,
                                                    int tiles_n, int group_m, BatchStrides bs) {
  using C = W4Cfg<WFMT, WGN, FNB, FMB>;
  typedef typename AReg<WFMT>::type AR;
  MX_BATCH_OFFSET(blockIdx.y);
  __shared__ __attribute__((aligned(1024))) uint8_t lds[C::LDS_BYTES];
  uint8_t* const slds = lds + 2 * C::STAGE;                  // two group-scale buffers
  uint8_t* const scratch = slds + 2 * C::SCALE_BYTES;        // surplus copy slots land here

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wn = wave % WGN, wm = wave / WGN;
  const int R = lane & 31, gq = lane >> 5, r = lane & 15;

  // ---- tile of this workgroup: each XCD a contiguous range, in groups of group_m m-tiles
  const int T = tiles_m * tiles_n;
  const int bid = blockIdx.x, xcd = bid & 7, slot = bid >> 3;
  const int t = xcd * (T >> 3) + (xcd < (T & 7) ? xcd : (T & 7)) + slot;
  const int gsz = group_m * tiles_n;
  const int first_m = (t / gsz) * group_m;
  const int gm = min(tiles_m - first_m, group_m);
  const int tm = first_m + (t % gsz) % gm;
  const int tn = (t % gsz) / gm;
  const int n0 = tn * C::BN, m0 = tm * C::BM;

  const int NG = N >> 4, KB = K >> 5, KT = K >> 7;
  const uint32_t* wsc = (const uint32_t*)(packed + (int64_t)KT * NG * C::FB);

  // ---- copy sources: 32-bit lane offsets from uniform bases (as in k_gemm_tile)
  uint32_t a_off[C::A_PW];
#pragma unroll
  for (int i = 0; i < C::A_PW; ++i) {
    const int c = min(wave + C::NW * i, C::A_CHUNKS - 1);
    if (C::FB % 1024 == 0) {
      const int f = c * 1024 / C::FB;
      a_off[i] = (uint32_t)(min((n0 >> 4) + f, NG - 1) * C::FB + (c * 1024 - f * C::FB));
    } else {
      const int off = c * 1024 + lane * 16;
      const int f = off / C::FB;
      a_off[i] = (uint32_t)(min((n0 >> 4) + f, NG - 1) * C::FB + (off - f * C::FB));
    }
  }
  const uint32_t a_lane = C::FB % 1024 == 0 ? (uint32_t)lane * 16 : 0u;
  uint32_t b_off[C::B_PW];
#pragma unroll
  for (int i = 0; i < C::B_PW; ++i) {
    const int row = 8 * (wave + C::NW * i) + (lane >> 3);
    const int chunk = (lane & 7) ^ swz(row);
    b_off[i] = (uint32_t)(min(m0 + row, M - 1) * K + chunk * 16);
  }
  // the p-th tile copy of step kt into stage `stage` (p < D: weight chunks, then activations)
  auto copy_one = [&](int kt, int stage, int p) __attribute__((always_inline)) {
    uint8_t* base = lds + stage * C::STAGE;
    if (p < C::A_PW) {
      const int c = wave + C::NW * p;
      dma16(packed + (uint32_t)(kt * NG * C::FB + a_off[p] + a_lane),
            c < C::A_CHUNKS ? base + c * 1024 : scratch);
    } else {
      const int i = p - C::A_PW;
      dma16(xq + (uint32_t)(kt * 128 + b_off[i]), base + C::A_BYTES + (wave + C::NW * i) * 1024);
    }
  };
  // scale copies of group kt4 into buffer sbuf: weight words (16 B per lane, four fragments
  // per instruction) and activation rows (4 B per lane, 16 rows per instruction)
  uint32_t sa_src[C::SA_PW];
#pragma unroll
  for (int i = 0; i < C::SA_PW; ++i) {
    const int c = min(wave + C::NW * i, C::SA_PIECES - 1);
    sa_src[i] = (uint32_t)(min((n0 >> 4) + 4 * c + (lane >> 4), NG - 1) * 256 + (lane & 15) * 16);
  }
  uint32_t sb_src[C::SB_PW];
#pragma unroll
  for (int i = 0; i < C::SB_PW; ++i) {
    const int c = min(wave + C::NW * i, C::SB_PIECES - 1);
    sb_src[i] = (uint32_t)(min(m0 + 16 * c + (lane >> 2), M - 1) * KB + (lane & 3) * 4);
  }
  auto copy_scales = [&](int kt4, int sbuf) __attribute__((always_inline)) {
    uint8_t* base = slds + sbuf * C::SCALE_BYTES;
#pragma unroll
    for (int i = 0; i < C::SA_PW; ++i) {
      const int c = wave + C::NW * i;
      dma16((const uint8_t*)wsc + (uint32_t)(kt4 * NG * 256 + sa_src[i]),
            c < C::SA_PIECES ? base + c * 1024 : scratch);
    }
#pragma unroll
    for (int i = 0; i < C::SB_PW; ++i) {
      const int c = wave + C::NW * i;
      dma4(xs + (uint32_t)(sb_src[i] + 16 * kt4), c < C::SB_PIECES ? base + C::SA_BYTES + c * 256 : scratch);
    }
  };
  // this lane's scale words of group kt4: weight block i, K half s -> row R of the block,
  // 32-block 2 s + gq of each step (byte kt % 4); activations likewise, gathered from the
  // row's 16 bytes (byte 4 q + 2 s + gq -> byte q)
  const uint32_t cs0 = (uint32_t)gq, cs1 = (uint32_t)(2 + gq);
  const uint32_t psel0 = cs0 | ((4 + cs0) << 8) | (0x0Cu << 16) | (0x0Cu << 24);
  const uint32_t psel1 = cs1 | ((4 + cs1) << 8) | (0x0Cu << 16) | (0x0Cu << 24);
  auto read_scales = [&](int sbuf, uint32_t (*sa)[2], uint32_t (*sb)[2]) __attribute__((always_inline)) {
    const uint8_t* base = slds + sbuf * C::SCALE_BYTES;
#pragma unroll
    for (int i = 0; i < FNB; ++i) {
      const int ngl = 2 * (wn * FNB + i) + (R >> 4);
      sa[i][0] = *(const uint32_t*)(base + ngl * 256 + (r + 16 * gq) * 4);
      sa[i][1] = *(const uint32_t*)(base + ngl * 256 + (r + 16 * (2 + gq)) * 4);
    }
#pragma unroll
    for (int j = 0; j < FMB; ++j) {
      const v4i w = *(const v4i*)(base + C::SA_BYTES + (wm * 32 * FMB + 32 * j + R) * 16);
      const uint32_t lo0 = __builtin_amdgcn_perm((uint32_t)w[1], (uint32_t)w[0], psel0);
      const uint32_t hi0 = __builtin_amdgcn_perm((uint32_t)w[3], (uint32_t)w[2], psel0);
      const uint32_t lo1 = __builtin_amdgcn_perm((uint32_t)w[1], (uint32_t)w[0], psel1);
      const uint32_t hi1 = __builtin_amdgcn_perm((uint32_t)w[3], (uint32_t)w[2], psel1);
      sb[j][0] = __builtin_amdgcn_perm(hi0, lo0, 0x05040100u);
      sb[j][1] = __builtin_amdgcn_perm(hi1, lo1, 0x05040100u);
    }
  };

  // ---- operand reads from LDS (K half s of the step in stage `stage`)
  // weight block i: fragments 2 (wn FNB + i) and + 1; lane reads fragment row R of it
  const uint32_t a_rd = (uint32_t)((2 * wn * FNB + (R >> 4)) * C::FB);
  const uint32_t b_rd = (uint32_t)((wm * 32 * FMB + R) * 128);
  const uint32_t sw = (uint32_t)swz(R);
  auto load_a = [&](const uint8_t* st, int i, int s) __attribute__((always_inline)) {
    const uint8_t* f = st + a_rd + i * 2 * C::FB;
    if constexpr (WFMT == 0) {
      const v4i lo = *(const v4i*)(f + s * 1024 + (r + 16 * gq) * 16);
      const v4i hi = *(const v4i*)(f + s * 1024 + 512 + (r + 16 * gq) * 16);
      return (AR){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    } else {   // FP6: 32-block 2 s + gq of row R: 16 bytes, then 8
      const v4i lo = *(const v4i*)(f + (r + 16 * (2 * s + gq)) * 16);
      const v2i hi = *(const v2i*)(f + 1024 + (r + 16 * (2 * s + gq)) * 8);
      return (AR){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1]};
    }
  };
  auto load_b = [&](const uint8_t* st, int j, int s) __attribute__((always_inline)) {
    const uint8_t* row = st + C::A_BYTES + b_rd + j * 32 * 128;
    const v4i lo = *(const v4i*)(row + (((uint32_t)(4 * s + gq) ^ sw) << 4));
    const v4i hi = *(const v4i*)(row + (((uint32_t)(4 * s + 2 + gq) ^ sw) << 4));
    return (v8i){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  };

  v16f acc[FNB][FMB];
#pragma unroll
  for (int i = 0; i < FNB; ++i)
#pragma unroll
    for (int j = 0; j < FMB; ++j) acc[i][j] = (v16f){};

  uint32_t sa[FNB][2] = {}, sb[FMB][2] = {};   // this group's scale words
  uint32_t ta[FNB] = {}, tb[FMB] = {};         // the deferred half's, across a group boundary
  AR ay[FNB];                            // second-half operands, used after the next barrier
  v8i by[FMB];
  const int KT4 = KT >> 2;               // whole groups (K % 512 == 0)

  // prologue: group 0's scales and step 0's tiles
  copy_scales(0, 0);
#pragma unroll
  for (int p = 0; p < C::D; ++p) copy_one(0, 0, p);

  // One K step.  After the barrier the wave issues this step's first-half operand reads, then
  // runs the deferred second half of step kt - 1 (its operands are already in registers) with
  // one copy for step kt + 1 after each MFMA; then this step's first half, with the second-half
  // operand reads issued after its first MFMAs.  (Spreading the operand reads one or two per
  // MFMA measured slower: 209 against 195 us on the prefill GEMM.)  FIRST (step 0) has no
  // deferred half.  Copies past the last step re-fetch the last step (or group of scales) into
  // the free buffer, unused, so every step issues the same operations and nothing in the loop
  // depends on kt at run time.
  auto step = [&](int kt, auto qc, auto firstc) __attribute__((always_inline)) {
    constexpr int Q = decltype(qc)::value;
    constexpr bool FIRST = decltype(firstc)::value;
    constexpr int QD = (Q + 3) & 3;      // op-select byte of the deferred half (step kt - 1)
    __builtin_amdgcn_sched_barrier(0);
    wait_vm_barrier<0>();                // step kt's tiles (and its group's scales) landed;
                                         // every wave is done with stage (kt + 1) % 2
    const uint8_t* st = lds + (kt & 1) * C::STAGE;
    if constexpr (Q == 0) {
#pragma unroll
      for (int i = 0; i < FNB; ++i) ta[i] = sa[i][1];
#pragma unroll
      for (int j = 0; j < FMB; ++j) tb[j] = sb[j][1];
      read_scales((kt >> 2) & 1, sa, sb);
    }
    // first-half operands of this step
    AR ax[FNB];
    v8i bx[FMB];
#pragma unroll
    for (int j = 0; j < FMB; ++j) bx[j] = load_b(st, j, 0);
#pragma unroll
    for (int i = 0; i < FNB; ++i) ax[i] = load_a(st, i, 0);
    __builtin_amdgcn_sched_barrier(0);
    const int kn = min(kt + 1, KT - 1);
    if constexpr (Q == 0) copy_scales(min((kt >> 2) + 1, KT4 - 1), ((kt >> 2) + 1) & 1);
    int p = 0;
#pragma unroll
    for (int i = 0; i < FNB; ++i) {
#pragma unroll
      for (int j = 0; j < FMB; ++j) {
        if constexpr (!FIRST) {
          if constexpr (Q == 0) mfma32_inplace<WFMT, QD>(acc[i][j], ay[i], by[j], ta[i], tb[j]);
          else mfma32_inplace<WFMT, QD>(acc[i][j], ay[i], by[j], sa[i][1], sb[j][1]);
        }
        if (p < C::D) copy_one(kn, (kt + 1) & 1, p);
        ++p;
        __builtin_amdgcn_sched_barrier(0);
      }
    }
#pragma unroll
    for (; p < C::D; ++p) copy_one(kn, (kt + 1) & 1, p);
    // scale words written by VALU above: two wait states before the assembly MFMAs read them
    if constexpr (Q == 0) asm volatile("s_nop 2" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    int u = 0;
#pragma unroll
    for (int i = 0; i < FNB; ++i) {
#pragma unroll
      for (int j = 0; j < FMB; ++j) {
        mfma32_inplace<WFMT, Q>(acc[i][j], ax[i], bx[j], sa[i][0], sb[j][0]);
        ++u;
        if (u == 2) {
#pragma unroll
          for (int jj = 0; jj < FMB; ++jj) by[jj] = load_b(st, jj, 1);
        } else if (u == 3) {
#pragma unroll
          for (int ii = 0; ii < FNB; ++ii) ay[ii] = load_a(st, ii, 1);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;
  using T_ = std::true_type;
  using F_ = std::false_type;
  step(0, I0(), T_());
  step(1, I1(), F_());
  step(2, I2(), F_());
  step(3, I3(), F_());
  for (int kt4 = 1; kt4 < KT4; ++kt4) {
    step(4 * kt4 + 0, I0(), F_());
    step(4 * kt4 + 1, I1(), F_());
    step(4 * kt4 + 2, I2(), F_());
    step(4 * kt4 + 3, I3(), F_());
  }
  // the last step's second half
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): its operands are in registers
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int i = 0; i < FNB; ++i)
#pragma unroll
    for (int j = 0; j < FMB; ++j) mfma32_inplace<WFMT, 3>(acc[i][j], ay[i], by[j], sa[i][1], sb[j][1]);
  // every copy landed and every wave done before LDS is reused for the output; the nops give
  // the last (assembly) MFMAs their result latency before the accumulators are read
  wait_vm_barrier<0>();
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_nop 15\n s_nop 15\n s_nop 15\n s_nop 15\n s_nop 15\n s_nop 15" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);

  // ---- epilogue: bias, bf16, through LDS as a [BM][BN] tile, then 16-byte coalesced stores.
  // Lane holds, for u < 4, n = 32 (wn FNB + i) + 8 u + 4 gq + (0..3) of row m = 32 (wm FMB + j) + R
#pragma unroll
  for (int i = 0; i < FNB; ++i) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int nl = 32 * (wn * FNB + i) + 8 * u + 4 * gq;
      float bv[4] = {0.f, 0.f, 0.f, 0.f};
      if (bias && n0 + nl < N) {
#pragma unroll
        for (int e = 0; e < 4; ++e) bv[e] = bf16_to_float(bias[n0 + nl + e]);
      }
#pragma unroll
      for (int j = 0; j < FMB; ++j) {
        const int ml = 32 * (wm * FMB + j) + R;
        const v2i o = {(int)pack_bf16x2(acc[i][j][4 * u + 0] + bv[0], acc[i][j][4 * u + 1] + bv[1]),
                       (int)pack_bf16x2(acc[i][j][4 * u + 2] + bv[2], acc[i][j][4 * u + 3] + bv[3])};
        *(v2i*)(lds + ml * C::OUT_PITCH + nl * 2) = o;
      }
    }
  }
  __syncthreads();
  constexpr int ROW_PIECES = C::BN * 2 / 16;
#pragma unroll 4
  for (int q = tid; q < C::BM * ROW_PIECES; q += C::NW * 64) {
    const int ml = q / ROW_PIECES, cp = q - ml * ROW_PIECES;
    const int m = m0 + ml, n = n0 + cp * 8;
    if (m < M && n < N)
      __builtin_nontemporal_store(*(const v4i*)(lds + ml * C::OUT_PITCH + cp * 16), (v4i*)(y + (int64_t)m * N + n));
  }
}

template <int WFMT, int WGN, int FNB, int FMB>
static void launch_w4(const uint8_t* xq, const uint8_t* xs, int M, int K, const uint8_t* packed,
                      int N, const uint16_t* bias, uint16_t* y, int group_m, hipStream_t s,
                      int batch, const BatchStrides& bs) {
  using C = W4Cfg<WFMT, WGN, FNB, FMB>;
  const int tm = (M + C::BM - 1) / C::BM, tn = (N + C::BN - 1) / C::BN;
  hipLaunchKernelGGL((k_gemm_w4<WFMT, WGN, FNB, FMB>), dim3((unsigned)(tm * tn), (unsigned)batch), dim3(256),
                     0, s, xq, xs, M, K, packed, N, bias, y, tm, tn, group_m, bs);
}


template <int WFMT, int XFMT, int FN, int FM>
static void launch_pp(const uint8_t* xq, const uint8_t* xs, int M, int K, const uint8_t* packed,
                      int N, const uint16_t* bias, uint16_t* y, int group_m, hipStream_t s,
                      int batch, const BatchStrides& bs) {
  using C = TileCfg<WFMT, XFMT, FN, FM, 2>;
  const int tm = (M + C::BM - 1) / C::BM, tn = (N + C::BN - 1) / C::BN;
  hipLaunchKernelGGL((k_gemm_pp<WFMT, XFMT, FN, FM>), dim3((unsigned)(tm * tn), (unsigned)batch),
                     dim3(512), 0, s, xq, xs, M, K, packed, N, bias, y, tm, tn, group_m, bs);
}

template <int WFMT, int XFMT, int FN, int FM, int S>
static void launch_tile(const uint8_t* xq, const uint8_t* xs, int M, int K, const uint8_t* packed,
                        int N, const uint16_t* bias, uint16_t* y, int group_m, hipStream_t s,
                        int batch, const BatchStrides& bs, int parts = 1, float* part = nullptr) {
  using C = TileCfg<WFMT, XFMT, FN, FM, S>;
  const int tm = (M + C::BM - 1) / C::BM, tn = (N + C::BN - 1) / C::BN;
  hipLaunchKernelGGL((k_gemm_tile<WFMT, XFMT, FN, FM, S>),
                     dim3((unsigned)(tm * tn), (unsigned)batch, (unsigned)parts), dim3(512), 0, s,
                     xq, xs, M, K, packed, N, bias, y, tm, tn, group_m, bs, part);
}

// Split K: the K parts' fp32 sums [P][M][N] added in part order, + bias, one bf16 rounding.
// Four outputs per thread (N % 16 == 0), all parts' loads in flight together.
__global__ __launch_bounds__(256) void k_splitk_reduce(const float* __restrict__ part, int P,
                                                      int64_t MN, int N,
                                                      const uint16_t* __restrict__ bias,
                                                      uint16_t* __restrict__ y) {
  for (int64_t i = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 4; i < MN;
       i += (int64_t)gridDim.x * blockDim.x * 4) {
    v4f v[kMaxSplit];
#pragma unroll
    for (int p = 0; p < kMaxSplit; ++p)
      if (p < P) v[p] = __builtin_nontemporal_load((const v4f*)(part + p * MN + i));
    v4f sum = v[0];
#pragma unroll
    for (int p = 1; p < kMaxSplit; ++p)
      if (p < P) sum += v[p];
    float bv[4] = {0.f, 0.f, 0.f, 0.f};
    if (bias) {
      const int n = (int)(i % N);
#pragma unroll
      for (int e = 0; e < 4; ++e) bv[e] = bf16_to_float(bias[n + e]);
    }
    const v2i o = {(int)pack_bf16x2(sum[0] + bv[0], sum[1] + bv[1]),
                   (int)pack_bf16x2(sum[2] + bv[2], sum[3] + bv[3])};
    *(v2i*)(y + i) = o;
  }
}

// K parts for a single-layer tiled GEMM (M > 32) whose 128 x 128 tiles would occupy at most 96
// of the 256 CUs: about 256 workgroups, each at least one group of four K steps, at most
// kMaxSplit parts; 1 = no split.  From 65 rows the parts run on 64 x 128 tiles (64 weight rows)
// where those still give two parts or more, else on 128 x 128 tiles: half the parts for the
// same workgroup count, so half the fp32 bytes written and read back (4096 x 4096 with the
// quantizer and the sum: 18.5 -> 16.4 us at M = 128, 21.0 -> 18.4 at M = 192, 21.4 -> 19.5 at
// M = 256; 8192 x 8192 at M = 128 unchanged; at M <= 64 half of each narrow tile's activation
// rows would be empty, and 8192 x 8192 at M = 64 measured no faster).  Narrow tiles serve E4M3
// operands only: their FP6 builds returned wrong sums in testing, and their assembly has the
// compiler's register copies within two wait states of the assembly MFMAs that read them at
// 15 sites (against 5 in the wide tile).  A call's workspace is sized for the wide plan, whose
// part count is never the smaller.  (At 128 wide tiles, two parts measured slower than none: the
// parts' fp32 traffic then costs more than the idle half of the CUs; at 96 tiles, faster.)
struct SplitPlan { int parts; bool narrow; };
static SplitPlan split_plan(int64_t M, int64_t N, int64_t K, bool narrow_ok) {
  if (M <= 32 || K % 128 != 0 || N < 128) return {1, false};   // up to 32 rows: the decode kernels
  const int64_t t = ((N + 127) / 128) * ((M + 127) / 128);
  if (t > 96) return {1, false};
  const int64_t tn = ((N + 63) / 64) * ((M + 127) / 128);      // 64 x 128 tiles
  const bool narrow = narrow_ok && M > 64 && 256 / tn >= 2;
  const int64_t G = (K / 128 + 3) / 4;
  int64_t p = 256 / (narrow ? tn : t);
  if (p > kMaxSplit) p = kMaxSplit;
  if (p > G) p = G;
  return p < 2 ? SplitPlan{1, false} : SplitPlan{(int)p, narrow};
}
int gemm_split_parts(int64_t M, int64_t N, int64_t K) { return split_plan(M, N, K, false).parts; }

int64_t gemm_split_bytes(int64_t M, int64_t N, int64_t K) {
  const int p = gemm_split_parts(M, N, K);
  return p > 1 ? (int64_t)p * M * N * 4 : 0;
}

// Tile choice: the configurations below are compiled; pick the one whose tile count fills the
// 256 CUs in the fewest (and fullest) waves, preferring larger tiles on ties; a batched launch
// counts the tiles of all its layers.
struct TileChoice { int fn, fm; };
// compiled tiles (fn, fm) -> workgroup tile 32 fn x 64 fm, two LDS stages
//
// The two settings are process-wide atomics; batch-invariant mode can also be set for one
// thread.  A call reads each setting once, when it starts (CallSettings at every launching
// entry point), and all its kernel choices use that snapshot.
static std::atomic<int> g_force_tile{0};   // fn * 256 + fm, 0 = automatic
static std::atomic<bool> g_batch_invariant{false};
static thread_local int tl_batch_invariant = -1;   // this thread's mode; -1: the process-wide one
static thread_local int tl_call_bi = -1;           // the running call's snapshot, -1: none
static thread_local int tl_call_tile = -1;
void force_tile(int fn, int fm) { g_force_tile.store(fn * 256 + fm); }
void set_batch_invariant(bool on) { g_batch_invariant.store(on); }
void set_batch_invariant_thread(int mode) { tl_batch_invariant = mode < 0 ? -1 : (mode != 0); }
static bool batch_invariant_now() {
  return tl_batch_invariant >= 0 ? tl_batch_invariant != 0
                                 : g_batch_invariant.load(std::memory_order_relaxed);
}
bool batch_invariant() { return tl_call_bi >= 0 ? tl_call_bi != 0 : batch_invariant_now(); }
static int forced_tile() {
  return tl_call_tile >= 0 ? tl_call_tile : g_force_tile.load(std::memory_order_relaxed);
}
CallSettings::CallSettings() : bi_(tl_call_bi), tile_(tl_call_tile) {
  if (tl_call_bi < 0) {   // the outermost scope of a call takes the snapshot
    tl_call_bi = batch_invariant_now();
    tl_call_tile = g_force_tile.load(std::memory_order_relaxed);
  }
}
CallSettings::~CallSettings() {
  tl_call_bi = bi_;
  tl_call_tile = tile_;
}
static TileChoice choose_tile(int M, int N, int batch, bool w4_ok) {
  const int f = forced_tile();
  // a forced four-wave tile (fm == 16) applies only where that kernel does
  if (f && ((f % 256 != 16 && f % 256 != 36) || w4_ok)) return TileChoice{f / 256, f % 256};
  static const TileChoice opts[] = {{8, 4}, {7, 4}, {6, 4}, {4, 4}, {4, 2}};
  double best = 1e30;
  TileChoice pick = opts[0];
  for (const TileChoice& o : opts) {
    const int bn = 32 * o.fn, bm = 64 * o.fm;
    const long tiles = (long)((N + bn - 1) / bn) * ((M + bm - 1) / bm) * batch;
    const long waves = (tiles + 255) / 256;
    // time ~ waves x per-tile work, per-tile work ~ bn * bm (+ a fixed operand-load cost)
    const double cost = (double)waves * ((double)bn * bm + 64.0 * (bn + bm));
    if (cost < best * 0.999) { best = cost; pick = o; }
  }
  return pick;
}

template <int WFMT, int XFMT>
static hipError_t launch_tiled(const uint8_t* xq, const uint8_t* xs, int M, int K,
                               const uint8_t* packed, int N, const uint16_t* bias, uint16_t* y,
                               hipStream_t s, int batch, const BatchStrides& bs, float* part) {
  const int group_m = 4;
  const SplitPlan sp = part && batch == 1 && !batch_invariant() && forced_tile() == 0
                          ? split_plan(M, N, K, WFMT == 0 && XFMT == 0) : SplitPlan{1, false};
  const int parts = sp.parts;
  if (parts > 1) {
    // too few 128 x 128 tiles for the CUs: K parts on grid z, then the ordered sum
    if constexpr (WFMT == 0 && XFMT == 0) {
      if (sp.narrow) {
        launch_tile<WFMT, XFMT, 2, 2, 4>(xq, xs, M, K, packed, N, bias, y, group_m, s, 1, bs, parts, part);
      } else {
        launch_tile<WFMT, XFMT, 4, 2, 4>(xq, xs, M, K, packed, N, bias, y, group_m, s, 1, bs, parts, part);
      }
    } else {
      launch_tile<WFMT, XFMT, 4, 2, 4>(xq, xs, M, K, packed, N, bias, y, group_m, s, 1, bs, parts, part);
    }
    const int64_t MN = (int64_t)M * N;
    int64_t blocks = (MN / 4 + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    hipLaunchKernelGGL(k_splitk_reduce, dim3((unsigned)blocks), dim3(256), 0, s, part, parts, MN, N, bias, y);
    return hipGetLastError();
  }
  const TileChoice c = choose_tile(M, N, batch, WFMT == 0 && XFMT == 0 && K % 512 == 0);
  if constexpr (WFMT == 0 && XFMT == 0) {
    // the ping-pong kernel wherever it applies (E4M3 operands, whole scale groups): chosen
    // tiles 224 x 256, 192 x 256 and 128 x 256, or forced as (fn, 36); a forced (fn, 4) keeps
    // the all-waves-in-step kernel
    const int f = forced_tile();
    const bool pp_tile = c.fm == 36 || (f == 0 && c.fm == 4 && (c.fn == 7 || c.fn == 6 || c.fn == 4));
    if (pp_tile && K % 512 == 0) {
      if (c.fn == 6) launch_pp<0, 0, 6, 4>(xq, xs, M, K, packed, N, bias, y, group_m, s, batch, bs);
      else if (c.fn == 4) launch_pp<0, 0, 4, 4>(xq, xs, M, K, packed, N, bias, y, group_m, s, batch, bs);
      else launch_pp<0, 0, 7, 4>(xq, xs, M, K, packed, N, bias, y, group_m, s, batch, bs);
      return hipGetLastError();
    }
    // the four-wave kernel, by the tile override only (tuning and tests): measured slower than
    // the eight-wave kernel on the prefill and outlier shapes (195 - 210 against 183 - 191 us;
    // 56 - 60 against 54 us)
    if (c.fm == 16) {
      if (c.fn == 16) launch_w4<0, 2, 4, 4>(xq, xs, M, K, packed, N, bias, y, group_m, s, batch, bs);
      else if (c.fn == 17) launch_w4<0, 1, 7, 2>(xq, xs, M, K, packed, N, bias, y, group_m, s, batch, bs);
      else if (c.fn == 18) launch_w4<0, 1, 6, 2>(xq, xs, M, K, packed, N, bias, y, group_m, s, batch, bs);
      else launch_w4<0, 2, 4, 2>(xq, xs, M, K, packed, N, bias, y, group_m, s, batch, bs);
      return hipGetLastError();
    }
  }
  if (c.fn == 8 && c.fm == 4) launch_tile<WFMT, XFMT, 8, 4, 2>(xq, xs, M, K, packed, N, bias, y, group_m, s, batch, bs);
  else if (c.fn == 7 && c.fm == 4) launch_tile<WFMT, XFMT, 7, 4, 2>(xq, xs, M, K, packed, N, bias, y, group_m, s, batch, bs);
  else if (c.fn == 6 && c.fm == 4) launch_tile<WFMT, XFMT, 6, 4, 2>(xq, xs, M, K, packed, N, bias, y, group_m, s, batch, bs);
  else if (c.fn == 4 && c.fm == 4) launch_tile<WFMT, XFMT, 4, 4, 2>(xq, xs, M, K, packed, N, bias, y, group_m, s, batch, bs);
  else if ((long)((N + 127) / 128) * ((M + 127) / 128) * batch <= 256)
    // one tile per CU at most: each workgroup runs the whole K of its tile, where deeper
    // prefetch pays off (four LDS stages: 3 % over three, 17 % over two on 512 x 8192 x 8192)
    launch_tile<WFMT, XFMT, 4, 2, 4>(xq, xs, M, K, packed, N, bias, y, group_m, s, batch, bs);
  else
    launch_tile<WFMT, XFMT, 4, 2, 2>(xq, xs, M, K, packed, N, bias, y, group_m, s, batch, bs);
  return hipGetLastError();
}

hipError_t launch_gemm(const uint8_t* xq, const uint8_t* xs, int64_t M, int64_t K,
                       const uint8_t* packed, int64_t N, int fmt, const uint16_t* bias,
                       uint16_t* y, hipStream_t s, int batch, BatchStrides bs, int afmt,
                       float* part) {
  // (weight, activation) formats: any weight format with E4M3 activations, or FP6 with FP6
  const int pair = fmt * 4 + afmt;
  if (afmt != 0 && (fmt == 0 || (afmt != 2 && afmt != 3))) return hipErrorInvalidValue;
  // the small-M kernel splits K over waves (a different summation order); batch-invariant
  // mode keeps every M on the kernels that add the K steps in sequence
  if (afmt == 0 && !batch_invariant() && small_m_quantized(M, K))
    return launch_linear_small_m(xq, xs, true, M, K, packed, N, fmt, bias, y, s, batch, bs);
  const int m = (int)M, k = (int)K, n = (int)N;
  // rows 33..63 go to the tiled kernel when it splits K (weight streamed by 256 workgroups)
  const bool split = part && batch == 1 && !batch_invariant() && gemm_split_parts(M, N, K) > 1;
  const bool tiled = (K % 128 == 0) && (((uintptr_t)xs & 3) == 0) && (M >= 64 || (split && M > 32)) && N >= 128;
  if (tiled) {
    switch (pair) {
      case 0: return launch_tiled<0, 0>(xq, xs, m, k, packed, n, bias, y, s, batch, bs, part);
      case 8: return launch_tiled<2, 0>(xq, xs, m, k, packed, n, bias, y, s, batch, bs, part);
      case 12: return launch_tiled<3, 0>(xq, xs, m, k, packed, n, bias, y, s, batch, bs, part);
      case 10: return launch_tiled<2, 2>(xq, xs, m, k, packed, n, bias, y, s, batch, bs, part);
      case 11: return launch_tiled<2, 3>(xq, xs, m, k, packed, n, bias, y, s, batch, bs, part);
      case 14: return launch_tiled<3, 2>(xq, xs, m, k, packed, n, bias, y, s, batch, bs, part);
      case 15: return launch_tiled<3, 3>(xq, xs, m, k, packed, n, bias, y, s, batch, bs, part);
      default: return hipErrorInvalidValue;
    }
  }
  // one 16-row activation tile per workgroup for M <= 32 (more K steps in flight; at M > 16 two
  // workgroups read each weight fragment, the second mostly from L2), else two
  const int mt = M <= 32 ? 1 : 2;
  dim3 grid((unsigned)(N / 16), (unsigned)((M + 16 * mt - 1) / (16 * mt)), (unsigned)batch), block(64);
#define MX_GENERIC(W, X)                                                                              \
  do {                                                                                                \
    if (mt == 1)                                                                                      \
      hipLaunchKernelGGL((k_gemm_generic<W, X, 1>), grid, block, 0, s, xq, xs, m, k, packed, n, bias, y, bs); \
    else                                                                                              \
      hipLaunchKernelGGL((k_gemm_generic<W, X, 2>), grid, block, 0, s, xq, xs, m, k, packed, n, bias, y, bs); \
  } while (0)
  switch (pair) {
    case 0: MX_GENERIC(0, 0); break;
    case 8: MX_GENERIC(2, 0); break;
    case 12: MX_GENERIC(3, 0); break;
    case 10: MX_GENERIC(2, 2); break;
    case 11: MX_GENERIC(2, 3); break;
    case 14: MX_GENERIC(3, 2); break;
    case 15: MX_GENERIC(3, 3); break;
    default: return hipErrorInvalidValue;
  }
#undef MX_GENERIC
  return hipGetLastError();
}

}  // namespace mx
