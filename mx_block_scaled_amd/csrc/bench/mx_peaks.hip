// mx_peaks.hip — microbenchmarks behind the attainable-peak denominators of bench.py (a library
// of its own, libmxpeaks.so; the layer library does not contain it):
//
//  * mxpk_mfma_loop: every wave of the grid issues chains of independent scaled MFMAs
//    (16x16x128, A / B operand formats as given) with no memory traffic in the loop, so the
//    time is the matrix units' own rate on the running chip; one variant feeds them
//    pseudo-random operands that change on every MFMA, the power draw of layer data.
//  * mxpk_clock_probe: one wave that waits a given time and reports the shader-clock cycles
//    that passed, i.e. the clock the chip runs at while other work fills it.
//  * mxpk_stream_read: a read of n bytes (16-byte loads, a few in flight per lane) whose words
//    are folded into a value that is stored only in a case that never occurs, so the loads
//    cannot be dropped and nothing is written.
//  * mxpk_lds_read: LDS read bandwidth of one workgroup per CU: every wave keeps eight 16-byte
//    (or 8-byte) reads per lane in flight from conflict-free addresses of a 64 KiB buffer.
//  * mxpk_l1_copy: global -> CU bandwidth of one workgroup per CU reading a 256 KiB window that
//    stays in the L2: 16-byte direct-to-LDS loads, 16-byte loads into registers, or 4-byte
//    direct-to-LDS loads, eight per wave in flight.
//
// All are plain launches on the caller's stream; timing is the caller's (HIP events).
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v6i __attribute__((ext_vector_type(6)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kChains = 8;   // independent accumulators per wave

// shader-clock counter and the constant 100 MHz counter (scalar memory-time reads)
__device__ __forceinline__ uint64_t shader_clock() {
  uint64_t v = 0;
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("s_memtime %0\n\ts_waitcnt lgkmcnt(0)" : "=s"(v));
#endif
  return v;
}
__device__ __forceinline__ uint64_t real_clock() {
  uint64_t v = 0;
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("s_memrealtime %0\n\ts_waitcnt lgkmcnt(0)" : "=s"(v));
#endif
  return v;
}

// operand register image: 32 bytes for FP8, 24 for FP6
template <int F> struct Reg { typedef v8i type; };
template <> struct Reg<2> { typedef v6i type; };

// in-place scaled MFMA (D == C), so the accumulators stay put between iterations; the VGPR
// constraints exist only in the device pass
#if defined(__HIP_DEVICE_COMPILE__)
#define MXPK_MFMA(FMT)                                                                        \
  asm volatile("v_mfma_scale_f32_16x16x128_f8f6f4 %0, %1, %2, %0, %3, %4 op_sel_hi:[0,0,0]" \
               FMT : "+v"(acc[c]) : "v"(a), "v"(b), "v"(sa), "v"(sb))
#define MXPK_MFMA32()                                                                         \
  asm volatile("v_mfma_scale_f32_32x32x64_f8f6f4 %0, %1, %2, %0, %3, %4 op_sel_hi:[0,0,0]"  \
               : "+a"(acc[c]) : "v"(a), "v"(b), "v"(sa), "v"(sb))
#else
#define MXPK_MFMA(FMT) (void)0
#define MXPK_MFMA32() (void)0
#endif

// clk (optional): lane 0 of wave 0 of block 0 stores the shader-clock cycles (s_memtime) and
// the 100 MHz real-time ticks (s_memrealtime) its loop took, so the caller gets the clock the
// chip ran the loop at
template <int AF, int BF>
__global__ void __launch_bounds__(256) k_mfma_loop(int iters, float* out, uint64_t* clk) {
  const int t = threadIdx.x;
  const uint64_t c0 = shader_clock();
  const uint64_t r0 = real_clock();
  // operands that the compiler cannot fold: small codes derived from the lane
  typename Reg<AF>::type a;
  typename Reg<BF>::type b;
#pragma unroll
  for (int i = 0; i < (AF == 0 ? 8 : 6); ++i) a[i] = (int)(0x01010101u * (uint32_t)((t + i) & 7));
#pragma unroll
  for (int i = 0; i < (BF == 0 ? 8 : 6); ++i) b[i] = (int)(0x01010101u * (uint32_t)((t * 3 + i) & 7));
  [[maybe_unused]] const int sa = 127 + (t >> 10), sb = 127;   // E8M0 1.0 (t < 256)
  v4f acc[kChains];
#pragma unroll
  for (int c = 0; c < kChains; ++c) acc[c] = (v4f){0.f, 0.f, 0.f, 0.f};
  // the assembly MFMAs are invisible to the compiler's hazard checks: let the VALU writes of
  // the operands retire first
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("s_nop 7\n\ts_nop 7" ::: "memory");
#endif
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < kChains; ++c) {
      if constexpr (AF == 0 && BF == 0) MXPK_MFMA("");
      else if constexpr (AF == 0) MXPK_MFMA(" blgp:2");
      else MXPK_MFMA(" cbsz:2 blgp:2");
    }
  }
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
#endif
  const uint64_t c1 = shader_clock();
  const uint64_t r1 = real_clock();
  if (clk && blockIdx.x == 0 && t == 0) {
    clk[0] = c1 - c0;
    clk[1] = r1 - r0;
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kChains; ++c) s += acc[c][0] + acc[c][1] + acc[c][2] + acc[c][3];
  if (s == -1.0f) out[0] = s;    // never true for these operands; keeps the loop alive
}

// the FP8 x FP8 loop with operands like a real GEMM's: four A and four B register images of
// pseudo-random codes (exponent LSB cleared, so no NaN code) and scale bytes around 1.0, a
// different (A, B, scales) combination on every MFMA, so the matrix unit's datapath switches
// as it does on layer data (the constant small codes above barely toggle it, which lets the
// chip hold a higher clock)
__device__ __forceinline__ uint32_t mix32(uint32_t x) {
  x ^= x >> 16;
  x *= 0x7feb352dU;
  x ^= x >> 15;
  x *= 0x846ca68bU;
  x ^= x >> 16;
  return x;
}
__global__ void __launch_bounds__(256) k_mfma_rand_loop(int iters, float* out, uint64_t* clk) {
  const uint32_t t = threadIdx.x + 256u * blockIdx.x;
  const uint64_t c0 = shader_clock();
  const uint64_t r0 = real_clock();
  v8i a[4], b[4];
  int sa[4], sb[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      a[s][i] = (int)(mix32(t * 64u + s * 16u + i) & 0xF7F7F7F7u);
      b[s][i] = (int)(mix32(t * 64u + s * 16u + 8u + i + 0x9E3779B9u) & 0xF7F7F7F7u);
    }
    sa[s] = 120 + (int)(mix32(t + 77u * s) & 7u);
    sb[s] = 122 + (int)(mix32(t + 91u * s + 5u) & 3u);
  }
  v4f acc[kChains];
#pragma unroll
  for (int c = 0; c < kChains; ++c) acc[c] = (v4f){0.f, 0.f, 0.f, 0.f};
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("s_nop 7\n\ts_nop 7" ::: "memory");
#endif
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < kChains; ++c) {
#if defined(__HIP_DEVICE_COMPILE__)
      // A image c % 4, B image (c + c / 4) % 4: consecutive MFMAs differ in both operands
      asm volatile("v_mfma_scale_f32_16x16x128_f8f6f4 %0, %1, %2, %0, %3, %4 op_sel_hi:[0,0,0]"
                   : "+v"(acc[c])
                   : "v"(a[c % 4]), "v"(b[(c + c / 4) % 4]), "v"(sa[c % 4]),
                     "v"(sb[(c + c / 4) % 4]));
#endif
    }
  }
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
#endif
  const uint64_t c1 = shader_clock();
  const uint64_t r1 = real_clock();
  if (clk && blockIdx.x == 0 && threadIdx.x == 0) {
    clk[0] = c1 - c0;
    clk[1] = r1 - r0;
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kChains; ++c) s += acc[c][0] + acc[c][1] + acc[c][2] + acc[c][3];
  if (s == 1.0e30f) out[0] = s;   // practically never; keeps the loop alive
}

// the same loop with the 32x32x64 scaled MFMA (FP8 operands), accumulators in AGPRs
__global__ void __launch_bounds__(256) k_mfma32_loop(int iters, float* out, uint64_t* clk) {
  typedef float v16f __attribute__((ext_vector_type(16)));
  const int t = threadIdx.x;
  const uint64_t c0 = shader_clock();
  const uint64_t r0 = real_clock();
  v8i a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (int)(0x01010101u * (uint32_t)((t + i) & 7));
    b[i] = (int)(0x01010101u * (uint32_t)((t * 3 + i) & 7));
  }
  [[maybe_unused]] const int sa = 127 + (t >> 10), sb = 127;
  v16f acc[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) acc[c] = (v16f){};
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("s_nop 7\n\ts_nop 7" ::: "memory");
#endif
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < 4; ++c) MXPK_MFMA32();
  }
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("s_nop 15\n\ts_nop 15\n\ts_nop 15\n\ts_nop 15\n\ts_nop 15" ::: "memory");
#endif
  const uint64_t c1 = shader_clock();
  const uint64_t r1 = real_clock();
  if (clk && blockIdx.x == 0 && t == 0) {
    clk[0] = c1 - c0;
    clk[1] = r1 - r0;
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int e = 0; e < 16; ++e) s += acc[c][e];
  if (s == -1.0f) out[0] = s;
}

// n16 16-byte words; each lane takes U words per pass, a pass covering the grid
template <int U>
__global__ void __launch_bounds__(256) k_stream_read(const uint4* __restrict__ p, int64_t n16,
                                                     uint32_t* out) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  uint32_t acc = 0;
  for (; i + (U - 1) * stride < n16; i += U * stride) {
    uint4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = p[i + u * stride];
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n16; i += stride) {
    const uint4 v = p[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (acc == 0x9E3779B9u && out) out[0] = acc;   // data-dependent store that never happens
}

// one wave that waits until `ticks` of the 100 MHz counter have passed (bounded by time, so
// it always ends), then stores the shader-clock cycles and ticks that elapsed: run beside
// other work on a second stream, it gives the clock the chip ran that work at
__global__ void __launch_bounds__(64) k_clock_probe(uint64_t ticks, uint64_t* out) {
  const uint64_t c0 = shader_clock(), r0 = real_clock();
  uint64_t r = r0;
  while (r - r0 < ticks) {
    __builtin_amdgcn_s_sleep(8);
    r = real_clock();
  }
  const uint64_t c1 = shader_clock();
  if (threadIdx.x == 0) {
    out[0] = c1 - c0;
    out[1] = r - r0;
  }
}

// LDS reads: W = 16 (ds_read_b128) or 8 (ds_read_b64); each wave reads 1 KiB windows of a 64 KiB
// buffer, eight in flight, then waits; clk: block 0's shader-clock cycles over the loop
template <int W>
__global__ void __launch_bounds__(1024) k_lds_read(int iters, int* out, uint64_t* clk) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[65536];
  const int t = threadIdx.x, wv = t >> 6, l = t & 63;
  (void)wv;   // read by the device code only
  (void)l;
  for (int i = t; i < 65536 / 4; i += blockDim.x) ((int*)lds)[i] = i * 2654435761u;
  __syncthreads();
  const uint64_t c0 = shader_clock();
  int acc = 0;
#if defined(__HIP_DEVICE_COMPILE__)
  const uint32_t base = (uint32_t)(uintptr_t)lds;
  for (int it = 0; it < iters; ++it) {
    int v[8][4];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const uint32_t off = base + ((wv * 8 + u + it) & 63) * 1024 + l * W;   // < 64 KiB
      if (W == 16) asm volatile("ds_read_b128 %0, %1" : "=v"(*(__attribute__((ext_vector_type(4))) int*)v[u]) : "v"(off));
      else asm volatile("ds_read_b64 %0, %1" : "=v"(*(__attribute__((ext_vector_type(2))) int*)v[u]) : "v"(off));
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
    for (int u = 0; u < 8; ++u) acc ^= v[u][0] ^ v[u][1] ^ (W == 16 ? v[u][2] ^ v[u][3] : 0);
  }
#endif
  __syncthreads();
  const uint64_t c1 = shader_clock();
  if (blockIdx.x == 0 && t == 0 && clk) clk[0] = c1 - c0;
  if (acc == 0x12345 && out) out[0] = acc;   // data-dependent store that never happens
}

// global -> CU copies from a 256 KiB window: MODE 0 = 16-byte direct-to-LDS, 1 = 16-byte loads
// into registers, 2 = 4-byte direct-to-LDS; eight per wave in flight, then a wait
template <int MODE>
__global__ void __launch_bounds__(1024) k_l1_copy(const uint8_t* __restrict__ src, int iters,
                                                 int* out, uint64_t* clk) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds[65536];
  const int t = threadIdx.x, w = t >> 6, l = t & 63;
  const int nw = blockDim.x >> 6, slots = 64 / nw;   // 1 KiB LDS slots per wave
  __syncthreads();
  const uint64_t c0 = shader_clock();
  typedef int v4i_t __attribute__((ext_vector_type(4)));
  v4i_t acc = {0, 0, 0, 0};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const uint32_t off = (uint32_t)((((it * 8 + u) * nw + w + blockIdx.x * 7) & 255) * 1024);
      void __attribute__((address_space(3)))* dst =
          (void __attribute__((address_space(3)))*)(lds + (w * slots + (u % slots)) * 1024);
      if (MODE == 0)
        __builtin_amdgcn_global_load_lds((const void __attribute__((address_space(1)))*)(src + off + l * 16), dst, 16, 0, 0);
      else if (MODE == 1)
        acc ^= *(const v4i_t*)(src + off + l * 16);
      else
        __builtin_amdgcn_global_load_lds((const void __attribute__((address_space(1)))*)(src + off + l * 4), dst, 4, 0, 0);
    }
    __builtin_amdgcn_s_waitcnt(0x70 | (0xF << 8));   // vmcnt(0)
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  const uint64_t c1 = shader_clock();
  if (blockIdx.x == 0 && t == 0 && clk) clk[0] = c1 - c0;
  if ((acc.x ^ acc.y ^ acc.z ^ acc.w ^ lds[t]) == 0x12345 && out) out[0] = 1;
}

}  // namespace

extern "C" {

// out: 2 uint64 (shader-clock cycles, 100 MHz ticks) over a wait of `ticks` ticks
int mxpk_clock_probe(int64_t ticks, uint64_t* out, void* stream) {
  if (ticks <= 0 || ticks > 1000000000 || !out) return -1;
  hipLaunchKernelGGL(k_clock_probe, dim3(1), dim3(64), 0, (hipStream_t)stream, (uint64_t)ticks,
                     out);
  return hipGetLastError() == hipSuccess ? 0 : -6;
}

// flop per launch = blocks * 4 waves * iters * kChains * 2 * 16 * 16 * 128 (the 32x32x64 loop
// has 4 chains of twice the flop each: the same count)
int mxpk_mfma_chains(void) { return kChains; }

// clk: null, or 2 uint64 (shader-clock cycles, 100 MHz ticks) of block 0's loop
int mxpk_mfma_loop(int afmt, int bfmt, int blocks, int iters, float* out, uint64_t* clk,
                   void* stream) {
  if (blocks <= 0 || iters <= 0 || !out) return -1;
  hipStream_t s = (hipStream_t)stream;
  if (afmt == 0 && bfmt == 0)
    hipLaunchKernelGGL((k_mfma_loop<0, 0>), dim3(blocks), dim3(256), 0, s, iters, out, clk);
  else if (afmt == 0 && bfmt == 2)
    hipLaunchKernelGGL((k_mfma_loop<0, 2>), dim3(blocks), dim3(256), 0, s, iters, out, clk);
  else if (afmt == 2 && bfmt == 2)
    hipLaunchKernelGGL((k_mfma_loop<2, 2>), dim3(blocks), dim3(256), 0, s, iters, out, clk);
  else if (afmt == 100 && bfmt == 100)   // 32x32x64, FP8 x FP8: 4 chains, 2x the flop each
    hipLaunchKernelGGL(k_mfma32_loop, dim3(blocks), dim3(256), 0, s, iters, out, clk);
  else if (afmt == 200 && bfmt == 200)   // FP8 x FP8, pseudo-random operands (see above)
    hipLaunchKernelGGL(k_mfma_rand_loop, dim3(blocks), dim3(256), 0, s, iters, out, clk);
  else
    return -1;
  return hipGetLastError() == hipSuccess ? 0 : -6;
}

// read `bytes` (a multiple of 16) from p: `blocks` workgroups of 256 lanes, `unroll` (4, 8 or
// 16) 16-byte loads in flight per lane
int mxpk_stream_read(const void* p, int64_t bytes, int blocks, int unroll, uint32_t* out,
                     void* stream) {
  if (!p || bytes <= 0 || bytes % 16 != 0 || blocks <= 0) return -1;
  hipStream_t s = (hipStream_t)stream;
  const int64_t n16 = bytes / 16;
  if (unroll == 4)
    hipLaunchKernelGGL(k_stream_read<4>, dim3(blocks), dim3(256), 0, s, (const uint4*)p, n16, out);
  else if (unroll == 8)
    hipLaunchKernelGGL(k_stream_read<8>, dim3(blocks), dim3(256), 0, s, (const uint4*)p, n16, out);
  else if (unroll == 16)
    hipLaunchKernelGGL(k_stream_read<16>, dim3(blocks), dim3(256), 0, s, (const uint4*)p, n16, out);
  else
    return -1;
  return hipGetLastError() == hipSuccess ? 0 : -6;
}

// LDS read bandwidth: width 16 or 8 bytes per lane, threads per workgroup a multiple of 64 up
// to 1024; bytes read per workgroup = threads x iters x 8 x width; clk: block 0's cycles
int mxpk_lds_read(int width, int threads, int blocks, int iters, int* out, uint64_t* clk,
                  void* stream) {
  if ((width != 16 && width != 8) || threads < 64 || threads > 1024 || threads % 64 || blocks <= 0 ||
      iters <= 0)
    return -1;
  hipStream_t s = (hipStream_t)stream;
  if (width == 16)
    hipLaunchKernelGGL(k_lds_read<16>, dim3(blocks), dim3(threads), 0, s, iters, out, clk);
  else
    hipLaunchKernelGGL(k_lds_read<8>, dim3(blocks), dim3(threads), 0, s, iters, out, clk);
  return hipGetLastError() == hipSuccess ? 0 : -6;
}

// global -> CU copy bandwidth from a 256 KiB window of src (src must hold 256 KiB): mode 0 / 1 /
// 2 as k_l1_copy; threads 256, 512 or 1024; bytes per workgroup = threads x iters x 8 x (16 or 4)
int mxpk_l1_copy(int mode, const void* src, int threads, int blocks, int iters, int* out,
                 uint64_t* clk, void* stream) {
  if (mode < 0 || mode > 2 || !src || (threads != 256 && threads != 512 && threads != 1024) ||
      blocks <= 0 || iters <= 0)
    return -1;
  hipStream_t s = (hipStream_t)stream;
  const uint8_t* p = (const uint8_t*)src;
  if (mode == 0) hipLaunchKernelGGL(k_l1_copy<0>, dim3(blocks), dim3(threads), 0, s, p, iters, out, clk);
  else if (mode == 1) hipLaunchKernelGGL(k_l1_copy<1>, dim3(blocks), dim3(threads), 0, s, p, iters, out, clk);
  else hipLaunchKernelGGL(k_l1_copy<2>, dim3(blocks), dim3(threads), 0, s, p, iters, out, clk);
  return hipGetLastError() == hipSuccess ? 0 : -6;
}

}  // extern "C"
