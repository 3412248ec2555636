/*
 * mxfp8.h — C ABI of the MI355X (gfx950) MX block-scaled linear layer
 *
 *     y[M, N] = dequant(x_q, s_x)[M, K] . dequant(W_q, s_w)[N, K]^T  (+ bias[N]),  y in bf16
 *
 * Operation sources (vLLM API pages):
 *  - aiter_flydsl page, AiterFlyDSLMxfp8LinearKernel: weights are prepared once at load
 *    (process_weights_after_loading), then every call quantizes the bf16 activations to MXFP8
 *    with row-major E8M0 scales [M, K/32] (or takes them pre-quantized with the same layout,
 *    apply_weights / input_quant_key), runs the block-scaled GEMM, writes bf16 and adds the bias.
 *    row_major_weight gives the inverse of the load-time weight rearrangement.
 *  - compressed_tensors_w8a8_mxfp8 page, CompressedTensorsW8A8Mxfp8.create_weights: weight
 *    [N, K] float8_e4m3fn, weight_scale [N, K/32] uint8 (E8M0), group size 32.
 *  - mxfp6 page, MxFp6LinearLayerConfig: MXFP6 weights, E2M3 or E3M2, group size 32.
 *  - Mxfp8LinearKernel page: the two-phase kernel contract (prepare weights once, apply per call).
 * The quantizer follows the OCP MX v1.0 rule: scale byte = floor(log2(amax)) - emax + 127
 * clamped to [0, 254] (0 for an all-zero block, 0xFF for a block holding Inf/NaN), elements
 * x / 2^(byte-127) rounded to nearest-even and saturated at the format maximum (E4M3: 448).
 *
 * Conventions for every call
 *  - All data pointers are DEVICE pointers owned by the caller.  The library never allocates,
 *    frees or synchronizes; each call validates its arguments, enqueues its kernels on `stream`
 *    (a hipStream_t; NULL = the null stream) and returns.  Device faults surface at the
 *    caller's next synchronization, as usual for HIP.
 *  - Return value: MX_OK (0) or a negative MX_E* code; mxfp8_last_error() then gives a message
 *    (thread-local, valid until the next call on the same thread).
 *  - Argument validation runs before any HIP call, so bad arguments are reported without a GPU.
 *  - Shapes: M >= 0 (M == 0 is a no-op returning MX_OK), K > 0 with K % 32 == 0 (the MX
 *    block), N > 0 with N % 16 == 0 (the weight tile height).  Otherwise MX_ESHAPE.
 *  - Alignment: pointers marked [16] must be 16-byte aligned, or MX_EALIGN.
 *  - Concurrency: calls on different streams may overlap; each call only writes its outputs
 *    (and its workspace, which must therefore not be shared by overlapping calls).
 */
#ifndef MXFP8_H
#define MXFP8_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element formats.  The numbers are gfx950's MFMA operand format codes. */
typedef enum { MX_FMT_E4M3 = 0, MX_FMT_E2M3 = 2, MX_FMT_E3M2 = 3 } mx_fmt;

enum {
    MX_OK = 0,
    MX_EINVAL = -1,     /* null pointer, bad format code, negative stride              */
    MX_ESHAPE = -2,     /* K % 32, N % 16, a stride smaller than the row, size limits  */
    MX_EALIGN = -3,     /* a [16] pointer or stride not 16-byte aligned               */
    MX_EWORKSPACE = -4, /* workspace smaller than mxfp8_workspace_bytes()             */
    MX_EARCH = -5,      /* the current device is not gfx950 (CDNA4)                   */
    MX_EHIP = -6        /* a HIP runtime call failed (message has the HIP error)      */
};

/* 1 if HIP device `device` is a gfx950 (the only target), 0 if not, MX_EHIP if the device
 * cannot be queried.  aiter_flydsl page, is_supported: native MX needs CDNA4. */
int mxfp8_device_supported(int device);

/* Message for the last failing call on this thread ("" if none). */
const char* mxfp8_last_error(void);

/* ---------------------------------------------------------------- quantization */

/* Dynamic MXFP8 activation quantization (aiter_flydsl page, apply_weights: the call that
 * turns x [M, K] into E4M3 data and row-major [M, K/32] E8M0 scales).
 *   x_bf16 [16]  bf16 [M, ldx] (row stride ldx elements, ldx >= K, ldx % 8 == 0); read only
 *   xq     [16]  out: E4M3 codes, row-major [M, K]
 *   xs           out: E8M0 bytes, row-major [M, K/32]
 * Bit-exact with the OCP rule above (a block with Inf/NaN: scale 0xFF, codes 0x7F). */
int mxfp8_quantize_act(const void* x_bf16, int64_t M, int64_t K, int64_t ldx,
                       void* xq, void* xs, void* stream);

/* Fused producer of a pre-quantized activation: RMS norm, then the quantization above (the
 * Mxfp8LinearKernel page's input_quant_key: a layer may take activations quantized outside
 * it, with row-major [M, K/32] E8M0 scales; the pages name no producer, and the norm here is
 * the usual RMS norm with a bf16 weight computed in fp32, each fp32 quantity being the value
 * nearest to its exact definition):
 *     r32 = fp32(1 / sqrt(sum_k x_k^2 / K + eps)),   p_k = fp32(x_k r32),
 *     t_k = bf16(p_k),                               y_k = bf16(t_k gamma_k),
 * all roundings to nearest even; then y is quantized exactly as mxfp8_quantize_act quantizes
 * a bf16 input.  The sum of squares is taken in fp64, so r32 is the correctly rounded value
 * except for a row whose r lies within about 2^-45 (relative) of an fp32 rounding boundary.
 *   x_bf16 [16]  bf16 [M, ldx] (ldx >= K, ldx % 8 == 0)
 *   gamma  [16]  bf16 [K]
 *   eps          finite, >= 0
 *   xq [16], xs  out: E4M3 [M, K], E8M0 [M, K/32], both row-major (feed mxfp8_linear_prequant)
 *   y_bf16 [16]  optional out: the normalized rows y, bf16 [M, K]; NULL = not written */
int mxfp8_rmsnorm_quantize_act(const void* x_bf16, int64_t M, int64_t K, int64_t ldx,
                               const void* gamma_bf16, float eps, void* xq, void* xs,
                               void* y_bf16, void* stream);

/* The same MX quantization for weights, in any supported element format, producing the
 * checkpoint layout that mxfp8_prepack_weight takes (compressed_tensors_w8a8_mxfp8 page,
 * create_weights; mxfp6 page for E2M3 / E3M2):
 *   w_bf16 [16]  bf16 [N, ldw] (ldw >= K, ldw % 8 == 0)
 *   wq     [16]  out: E4M3 [N, K] bytes, or FP6 [N, 3K/4] bytes (four 6-bit codes per three
 *                bytes, little-endian along K: c0 | c1<<6 | c2<<12 | c3<<18)
 *   ws           out: E8M0 [N, K/32] */
int mxfp8_quantize_weight(const void* w_bf16, int64_t N, int64_t K, int64_t ldw, int fmt,
                          void* wq, void* ws, void* stream);

/* ---------------------------------------------------------------- load-time weight prepack */

/* Bytes of the prepacked weight for (N, K, fmt); 0 for invalid arguments. */
int64_t mxfp8_prepacked_bytes(int64_t N, int64_t K, int fmt);

/* Load-time rearrangement of a quantized weight into this library's MFMA-ready tiled layout,
 * with its scales interleaved for direct per-lane loads (aiter_flydsl page,
 * process_weights_after_loading: rearranged once, scales sliced to [:N, :K/32]).
 *   wq           E4M3 [N, ldw_bytes] or FP6 [N, ldw_bytes] bytes (ldw_bytes >= K or 3K/4)
 *   ws           E8M0, row stride ld_ws >= K/32; only the top-left [N, K/32] is read
 *   packed [16]  out: mxfp8_prepacked_bytes(N, K, fmt) bytes, owned by the caller; its layout
 *                is private to this library (read it back with mxfp8_unpack_weight). */
int mxfp8_prepack_weight(const void* wq, int64_t ldw_bytes, const void* ws, int64_t ld_ws,
                         int64_t N, int64_t K, int fmt, void* packed, void* stream);

/* Exact inverse of mxfp8_prepack_weight (cf. aiter_flydsl page, row_major_weight):
 * writes wq [N, K] (E4M3) or [N, 3K/4] (FP6) and ws [N, K/32], both row-major; packed [16]. */
int mxfp8_unpack_weight(const void* packed, int64_t N, int64_t K, int fmt,
                        void* wq, void* ws, void* stream);

/* Import of a weight stored in the aiter_flydsl page's (16, 16) preshuffled layout (E4M3
 * only; aiter_flydsl page, process_weights_after_loading / row_major_weight: the logical byte
 * array [N/16, 16, K/32, 2, 16] of W [N, K] is stored as [N/16, K/32, 2, 16, 16], i.e. byte
 * W[16 n0 + n1][32 k0 + 16 k1 + k2] at ((((n0 K/32 + k0) 2 + k1) 16 + n1) 16 + k2)).
 *   w16          N x K bytes in that order
 *   ws           E8M0, row stride ld_ws >= K/32 (as for mxfp8_prepack_weight)
 *   packed [16]  out: the same bytes mxfp8_prepack_weight writes for the row-major weight */
int mxfp8_prepack_weight_shuffled16(const void* w16, const void* ws, int64_t ld_ws, int64_t N,
                                    int64_t K, void* packed, void* stream);

/* Export of a prepacked E4M3 weight to that preshuffled layout: w16 (N x K bytes) and
 * ws [N, K/32] row-major.  Exact inverse of mxfp8_prepack_weight_shuffled16. */
int mxfp8_unpack_weight_shuffled16(const void* packed, int64_t N, int64_t K, void* w16,
                                   void* ws, void* stream);

/* ---------------------------------------------------------------- the linear layer */

/* Workspace bytes mxfp8_linear needs for (M, N, K, fmt) (0 for M == 0 or invalid arguments).
 * Layout: 64 KiB of counters, then the quantized activations between the quantizer and the
 * GEMM, or, for decode shapes (16 <= M <= 64, N % 64 == 0, K % 128 == 0; above 32 rows only
 * while a workgroup's share of x, M x K / P bf16 for its K part, is at most 256 KiB), the
 * partial sums of the workgroups that split K.  Otherwise, when M > 32 and the layer has at most 96 tiles of 128 x 128
 * outputs (K % 128 == 0, N >= 128), the quantized activations are followed (at the next
 * 256-byte boundary) by fp32 partial sums [P][M][N] of the P <= 8 K parts that the GEMM then
 * computes in separate workgroups and adds in part order in a second launch, so that the call
 * fills the GPU.  The counters must be zero before a workspace is first used
 * (allocate it zero-filled); every call leaves them zero, so a workspace stays valid for any
 * later call of any entry point, shape or stream order.  The same layout serves
 * mxfp8_linear_batched and mxfp8_linear_fmt. */
int64_t mxfp8_workspace_bytes(int64_t M, int64_t N, int64_t K, int fmt);

/* y = dequant(quantize(x)) . dequant(W)^T (+ bias), bf16 out (aiter_flydsl page,
 * AiterFlyDSLMxfp8LinearKernel.apply_weights, bf16-input branch).
 *   x_bf16    [16]  bf16 [M, K] row-major
 *   packed    [16]  from mxfp8_prepack_weight with the same N, K, fmt
 *   bias            bf16 [N] or NULL; added in fp32 before the single bf16 rounding
 *   y         [16]  out: bf16 [M, N] row-major (round to nearest even)
 *   workspace [16]  device buffer of ws_bytes >= mxfp8_workspace_bytes(M, N, K, fmt), its first
 *                   64 KiB zero before its first use (see mxfp8_workspace_bytes) */
int mxfp8_linear(const void* x_bf16, int64_t M, int64_t K, const void* packed, int64_t N,
                 int fmt, const void* bias, void* y, void* workspace, int64_t ws_bytes,
                 void* stream);

/* mxfp8_linear for callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc.  Same arguments as mxfp8_linear minus
 * the workspace, same kernels and results.  The library's own device array of
 * MXFP8_NOALLOC_SCRATCH_BYTES (held on each GPU it runs on until the process ends) serves as
 * the workspace; the call itself allocates and frees nothing.
 *   - A call whose mxfp8_workspace_bytes(M, N, K, fmt) exceeds the array returns MX_EWORKSPACE
 *     (before any HIP call); use mxfp8_linear with a workspace for such shapes.
 *   - The first call on a device looks up the array's device address and enqueues one small
 *     kernel that clears its counters (on `stream`; under capture it becomes part of the
 *     graph, which is harmless since every call leaves them zero).
 *   - All calls on one GPU share the array: calls that overlap on one GPU (several streams or
 *     threads) race and must be serialized by the caller. */
#define MXFP8_NOALLOC_SCRATCH_BYTES ((int64_t)64 << 20)
int mxfp8_linear_noalloc(const void* x_bf16, int64_t M, int64_t K, const void* packed, int64_t N,
                         int fmt, const void* bias, void* y, void* stream);

/* The same layer from pre-quantized activations (aiter_flydsl page, apply_weights with a
 * QuantizedActivation; the scales must be row-major [M, K/32] E8M0 exactly, as its assert
 * requires):
 *   xq [16] E4M3 [M, K];  xs  E8M0 [M, K/32];  other arguments as mxfp8_linear.
 * Needs no workspace. */
int mxfp8_linear_prequant(const void* xq, const void* xs, int64_t M, int64_t K,
                          const void* packed, int64_t N, int fmt, const void* bias, void* y,
                          void* stream);

/* Batched layer (Mxfp8LinearKernel page, Mxfp8LinearLayerConfig.bmm_batch_size; the
 * aiter_flydsl page's can_implement turns such layers away): for every b < B,
 *     y[b] = dequant(quantize(x[b])) . dequant(W[b])^T (+ bias[b])
 * with the same kernels, hence the same results, as B separate mxfp8_linear calls, with one
 * exception: a layer that mxfp8_linear would split along K (M > 32 with at most 96 output tiles
 * of 128 x 128; see mxfp8_workspace_bytes) runs unsplit here, as in mxfp8_linear_prequant, so its
 * fp32 sums add in another order than the separate call's.
 *   x_bf16    [16]  bf16 [B, M, K], contiguous
 *   packed    [16]  B prepacked weights back to back, mxfp8_prepacked_bytes(N, K, fmt) each
 *   bias            bf16 [B, N] or NULL
 *   y         [16]  out: bf16 [B, M, N]
 *   workspace [16]  ws_bytes >= mxfp8_workspace_bytes(B * M, N, K, fmt)
 * 0 <= B <= 65535; B * M obeys the limits on M; B == 0 or M == 0 is a no-op. */
int mxfp8_linear_batched(const void* x_bf16, int64_t B, int64_t M, int64_t K, const void* packed,
                         int64_t N, int fmt, const void* bias, void* y, void* workspace,
                         int64_t ws_bytes, void* stream);

/* The batched layer from pre-quantized activations: xq [B, M, K] E4M3 [16], xs [B, M, K/32]
 * E8M0 (row-major per batch, contiguous); other arguments as mxfp8_linear_batched.  Needs no
 * workspace. */
int mxfp8_linear_prequant_batched(const void* xq, const void* xs, int64_t B, int64_t M,
                                  int64_t K, const void* packed, int64_t N, int fmt,
                                  const void* bias, void* y, void* stream);

/* ---------------------------------------------------------------- MXFP6 activations */

/* MXFP6 activations (mxfp6 page, MxFp6LinearLayerConfig.activation_quant_key: the activation
 * quantization format of an MXFP6 layer).  afmt selects the activations' element format:
 * MX_FMT_E4M3 (the MXFP8 layer above) or MX_FMT_E2M3 / MX_FMT_E3M2.  FP6 activations require
 * FP6 weights (fmt E2M3 or E3M2): with both operands FP6 the scaled MFMA runs at its FP6 rate.
 * FP6 activations use the same rule as FP6 weights: E8M0 scale per 32 along K from the format's
 * emax (E2M3: 2, E3M2: 4), round-to-nearest-even, saturating, four 6-bit codes per three bytes
 * little-endian along K (a block with Inf/NaN: scale 0xFF, codes 0). */

/* Dynamic activation quantization in format afmt:
 *   x_bf16 [16]  bf16 [M, ldx] (ldx >= K, ldx % 8 == 0)
 *   xq     [16]  out: E4M3 [M, K] bytes (afmt E4M3) or packed FP6 [M, 3K/4] bytes
 *   xs           out: E8M0 [M, K/32] row-major
 * afmt == MX_FMT_E4M3 is mxfp8_quantize_act. */
int mxfp8_quantize_act_fmt(const void* x_bf16, int64_t M, int64_t K, int64_t ldx, int afmt,
                           void* xq, void* xs, void* stream);

/* Workspace bytes mxfp8_linear_fmt needs (0 for invalid arguments or M == 0).  With FP6
 * activations the workspace holds their codes in the layout the GEMM reads fastest: where
 * K % 128 == 0, each 128-wide K step's 96 bytes at the start of a 128-byte slice (K bytes a row),
 * else packed [M, 3K/4]; then the scales and, where the GEMM splits K, its partial sums. */
int64_t mxfp8_workspace_bytes_fmt(int64_t M, int64_t N, int64_t K, int fmt, int afmt);

/* mxfp8_linear with activations quantized to afmt (fmt = the weight's format; FP6 afmt needs
 * FP6 fmt, otherwise MX_EINVAL).  workspace [16]: ws_bytes >= mxfp8_workspace_bytes_fmt. */
int mxfp8_linear_fmt(const void* x_bf16, int64_t M, int64_t K, const void* packed, int64_t N,
                     int fmt, int afmt, const void* bias, void* y, void* workspace,
                     int64_t ws_bytes, void* stream);

/* mxfp8_linear_prequant with activations in format afmt: xq [16] E4M3 [M, K] or packed FP6
 * [M, 3K/4]; xs E8M0 [M, K/32] row-major.  Needs no workspace. */
int mxfp8_linear_prequant_fmt(const void* xq, const void* xs, int64_t M, int64_t K, int afmt,
                              const void* packed, int64_t N, int fmt, const void* bias, void* y,
                              void* stream);

/* ---------------------------------------------------------------- modes and tuning */

/* Batch-invariant mode (aiter_flydsl page, is_supported: its split-K kernel is not batch
 * invariant).  on != 0: every M runs on kernels that add the K steps of each output in order,
 * one MFMA per 128-wide step from a zero start (the tiled and generic GEMMs, and up to 64 rows
 * on the bf16 entry (K <= 4096; 16 rows for K <= 8192) the role-split small-M kernel with its
 * waves extending one accumulator chain in turn), so a row's result does not depend on how many
 * rows the call has; the split-K
 * kernels are not used.  on == 0 (default): fastest kernel per shape.  Returns MX_OK.
 * Thread safety: the mode is one process-wide atomic flag.  Each call reads the mode that
 * applies to it once, when it starts, and picks all of its kernels under that mode, so a call
 * running on another thread while the mode changes runs entirely under the old mode or
 * entirely under the new one.  Already enqueued work is never affected.  A thread that must
 * not depend on other threads' settings uses mxfp8_set_batch_invariant_thread. */
int mxfp8_set_batch_invariant(int on);

/* Batch-invariant mode for the calling thread only (for callers that cannot share a
 * process-wide mode): mode 1 = on, 0 = off for this thread's calls whatever the process-wide
 * setting; -1 = follow mxfp8_set_batch_invariant again (the initial state of every thread).
 * Other threads are not affected.  Returns MX_OK, or MX_EINVAL for any other mode. */
int mxfp8_set_batch_invariant_thread(int mode);


/* Tuning / testing hook: force the tile of the LDS-tiled GEMM used for large M.
 *   (fn, fm) in (8,4) (7,4) (6,4) (4,4) (4,2): the eight-wave kernel with all waves in step,
 *     fn, fm = 16-row weight fragments and 16-row activation groups per wave; the workgroup
 *     covers 32 fn weight rows x 64 fm activation rows;
 *   (7,36) (6,36) (4,36): the eight-wave ping-pong kernel (two groups of four waves taking
 *     turns between MFMAs and operand reads; E4M3 weights and activations and K % 512 == 0
 *     only, other layers keep the automatic choice) with the tile of (fn, 4).  The automatic
 *     choice runs it wherever it picks one of these tiles and the layer qualifies;
 *   (16,16) (17,16) (18,16) (19,16): the four-wave kernel (one wave per SIMD, 32x32x64 scaled
 *     MFMAs, E4M3 weights and K % 512 == 0 only; other layers keep the automatic choice), with
 *     workgroup tiles 256 x 256, 224 x 256, 192 x 256 and 256 x 128 (weight rows x activation
 *     rows);
 *   (0,0) restores the automatic choice.  MX_EINVAL for any other pair.
 * A forced tile also turns off the split-K tiled path.  Thread safety as for
 * mxfp8_set_batch_invariant: one process-wide atomic setting, read once by each call when it
 * starts; a call concurrent with a change runs entirely with the old or the new setting. */
int mxfp8_set_tile_config(int fn, int fm);

#ifdef __cplusplus
}
#endif
#endif /* MXFP8_H */
