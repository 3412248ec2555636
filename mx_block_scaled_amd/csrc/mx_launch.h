// mx_launch.h — internal host-side launchers (implemented next to their kernels).
// Arguments are validated by the C-ABI front (mx_api.cpp) before any of these is called;
// each returns the hipError_t of its launch.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mx {

// Size of the prepacked weight: fragments of 16 rows x 128 K (K zero-padded to a multiple of
// 128), ordered [K step][row group]; then the scales, one 32-bit word per lane per group of
// four K steps, ordered [K step / 4][row group][lane].
struct PackGeom {
  int64_t N, K, NG, KT, KT4, frag, wbytes, sbytes;
};
PackGeom pack_geom(int64_t N, int64_t K, int fmt);

// Batched calls (grid dimension = batch index b): per-batch byte strides of the activations
// (bf16 or E4M3), their scales, the prepacked weight, the output and the bias.  All zero for an
// unbatched call.
struct BatchStrides {
  int64_t x = 0, xs = 0, w = 0, y = 0, bias = 0;
  // FP6 activations: bytes per 128-wide K step of an activation row; 0 = packed (96 bytes), 128 =
  // each step's 96 bytes at the start of a 128-byte slice (K % 128 == 0), the layout the
  // library's own FP6 quantization writes for its GEMM
  int xstep = 0;
};

hipError_t launch_quantize_act(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, uint8_t* xq,
                               uint8_t* xs, hipStream_t s);
// MXFP6 activations (fmt E2M3 = 2 or E3M2 = 3): xq [M, 3K/4] packed codes (xstep 96) or rows of
// K / 128 slices of 128 bytes, each holding one K step's 96 bytes first (xstep 128, K % 128 == 0);
// xs [M, K/32].
hipError_t launch_quantize_act_fp6(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, int fmt,
                                   uint8_t* xq, uint8_t* xs, hipStream_t s, int xstep = 96);
// RMS norm (bf16 weight gamma [K], eps) fused with the E4M3 activation quantization; y
// (optional) receives the normalized bf16 rows [M, K].
hipError_t launch_rmsnorm_quant(const uint16_t* x, int64_t M, int64_t K, int64_t ldx,
                                const uint16_t* gamma, float eps, uint8_t* xq, uint8_t* xs,
                                uint16_t* y, hipStream_t s);
hipError_t launch_quantize_weight(const uint16_t* w, int64_t N, int64_t K, int64_t ldw, int fmt,
                                  uint8_t* wq, uint8_t* ws, hipStream_t s);
hipError_t launch_prepack(const uint8_t* wq, int64_t ldw, const uint8_t* ws, int64_t ld_ws,
                          int64_t N, int64_t K, int fmt, uint8_t* packed, hipStream_t s);
hipError_t launch_unpack(const uint8_t* packed, int64_t N, int64_t K, int fmt, uint8_t* wq,
                         uint8_t* ws, hipStream_t s);

// The same rearrangement from / to the aiter_flydsl page's (16, 16) preshuffled E4M3 layout.
hipError_t launch_prepack_shuffled16(const uint8_t* w16, const uint8_t* ws, int64_t ld_ws,
                                     int64_t N, int64_t K, uint8_t* packed, hipStream_t s);
hipError_t launch_unpack_shuffled16(const uint8_t* packed, int64_t N, int64_t K, uint8_t* w16,
                                    uint8_t* ws, hipStream_t s);

// Force the tiled GEMM's tile (fragments per wave along n and m); (0, 0) = automatic.
void force_tile(int fn, int fm);
// Batch-invariant mode: only kernels that add each output's K steps in order, so a row's result
// does not depend on M.  Process-wide, or for the calling thread (mode 0 / 1; -1 returns the
// thread to the process-wide setting).
void set_batch_invariant(bool on);
void set_batch_invariant_thread(int mode);
// The mode that applies to the call being launched (its snapshot inside a CallSettings scope).
bool batch_invariant();
// Snapshot of the mode and the forced tile for one call: every entry point that launches
// kernels holds one for its duration, so that all of its kernel choices agree even while
// another thread changes the settings.
struct CallSettings {
  CallSettings();
  ~CallSettings();
  CallSettings(const CallSettings&) = delete;
  CallSettings& operator=(const CallSettings&) = delete;
 private:
  int bi_, tile_;
};

// GEMM from quantized activations xq + xs [M, K/32] (row-major): xq is E4M3 [M, K] (afmt 0)
// or, with FP6 weights, packed E2M3 / E3M2 [M, 3K/4] (afmt 2 / 3).  With `part` (room for
// gemm_split_bytes(M, N, K) bytes) a single layer with few tiles splits K across workgroups and
// adds the parts in a second launch; without it K is never split across workgroups.
constexpr int kMaxSplit = 8;
int gemm_split_parts(int64_t M, int64_t N, int64_t K);
int64_t gemm_split_bytes(int64_t M, int64_t N, int64_t K);
hipError_t launch_gemm(const uint8_t* xq, const uint8_t* xs, int64_t M, int64_t K,
                       const uint8_t* packed, int64_t N, int fmt, const uint16_t* bias,
                       uint16_t* y, hipStream_t s, int batch = 1, BatchStrides bs = {},
                       int afmt = 0, float* part = nullptr);

// Small-M (decode) path: one launch, K split over the waves of a workgroup.  x is bf16 [M, K]
// quantized inside the kernel (small_m_fused shapes) or, with quantized = true, E4M3 xq [M, K]
// plus xs [M, K/32] (small_m_quantized shapes).
// Every workspace starts with this many bytes of counters, which must be zero before the
// workspace's first use; every call leaves them zero.  The rest holds the quantized activations
// or the decode kernel's partial sums.
constexpr int64_t kWorkspacePrefix = 64 * 1024;

// Decode with K also split across workgroups, quantizer fused (M <= 64, K % 128 == 0,
// N % 64 == 0): the counters of the workspace prefix, then decode_sk_workspace bytes of
// partial sums.  decode_sk_parts: the number of K parts (workgroups per column group).
bool decode_sk_ok(int64_t M, int64_t N, int64_t K);
int decode_sk_parts(int64_t N, int64_t K);
int64_t decode_sk_workspace(int64_t M, int64_t N, int64_t K);
hipError_t launch_linear_decode_sk(const uint16_t* x, int64_t M, int64_t K, const uint8_t* packed,
                                   int64_t N, int fmt, const uint16_t* bias, uint16_t* y,
                                   void* workspace, hipStream_t s);
bool small_m_fused(int64_t M, int64_t N, int64_t K);
// shapes of small_m_fused that run on the role-split kernel (quantizer waves beside MFMA waves)
bool small_m_rs(int64_t M, int64_t N, int64_t K);
bool small_m_quantized(int64_t M, int64_t K);
// shapes on which the small-M path also runs in batch-invariant mode: the role-split kernel
// (bf16 entry, its shapes: up to 64 rows) with its weight waves extending one accumulator chain
// in K order, which gives each output the bits of the tiled GEMM whatever M is
bool small_m_invariant(int64_t M, int64_t N, int64_t K, bool quantized);
hipError_t launch_linear_small_m(const void* x, const uint8_t* xs, bool quantized, int64_t M,
                                 int64_t K, const uint8_t* packed, int64_t N, int fmt,
                                 const uint16_t* bias, uint16_t* y, hipStream_t s,
                                 int batch = 1, BatchStrides bs = {});

// The C-ABI front's own pieces, shared with the allocation-free entry point: the thread-local
// error message (api_fail sets it and returns code), the per-device gfx950 check, and
// mxfp8_linear split into its argument checks (need = workspace bytes) and its launches.
int api_fail(int code, const char* fmt, ...);
int api_ok();
int api_check_arch();
int linear_check(const void* x_bf16, int64_t M, int64_t K, const void* packed, int64_t N, int fmt,
                 const void* y, int64_t* need);
int linear_launch(const void* x_bf16, int64_t M, int64_t K, const void* packed, int64_t N, int fmt,
                  const void* bias, void* y, void* workspace, void* stream);

}  // namespace mx
