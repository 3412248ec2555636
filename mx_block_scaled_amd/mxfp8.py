"""Python binding of libmxfp8 (the C ABI in include/mxfp8.h): argument marshalling only.

Every step of the layer runs in the HIP library; PyTorch only provides device memory and the
current stream.  If the library is not built this module raises; there is no fallback.

Two-phase use (Mxfp8LinearKernel page: weights processed once after loading, then applied per
call; aiter_flydsl page for the shapes and layouts):

    packed = prepack_weight(wq, ws, fmt)          # once, at load
    y = linear(x, packed, N, fmt, bias)           # per call, x bf16 [..., K] -> y bf16 [..., N]
    y = linear_prequant(xq, xs, packed, N, fmt)   # pre-quantized activations, xs [M, K/32]
"""
import ctypes
import os

import torch  # loaded first: libmxfp8 then binds to the HIP runtime torch already loaded

__all__ = [
    "FMT", "MXError", "lib", "library_path", "device_supported", "quantize_act",
    "quantize_weight", "prepack_weight", "unpack_weight", "prepacked_bytes", "workspace_bytes",
    "linear", "linear_prequant", "MxLinear", "set_tile_config", "set_batch_invariant",
    "prepack_weight_shuffled16", "unpack_weight_shuffled16", "linear_batched",
    "linear_prequant_batched", "quantize_act_fmt", "workspace_bytes_fmt", "linear_fmt",
    "linear_prequant_fmt", "rmsnorm_quantize_act", "new_workspace", "linear_noalloc",
    "set_batch_invariant_thread",
    "NOALLOC_SCRATCH_BYTES",
]

FMT = {"e4m3": 0, "e2m3": 2, "e3m2": 3}
_ERR = {0: "MX_OK", -1: "MX_EINVAL", -2: "MX_ESHAPE", -3: "MX_EALIGN", -4: "MX_EWORKSPACE",
        -5: "MX_EARCH", -6: "MX_EHIP"}

library_path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmxfp8.so")
_lib = None


class MXError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__("%s (%d): %s" % (_ERR.get(code, "?"), code, msg))
        self.code = code


def lib():
    """The loaded library; raises if it has not been built (no fallback path exists)."""
    global _lib
    if _lib is None:
        if not os.path.exists(library_path):
            raise RuntimeError("libmxfp8.so is not built (%s); run __graft_entry__.build()"
                               % library_path)
        L = ctypes.CDLL(library_path)
        P, I64, I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        sig = {
            "mxfp8_device_supported": (I, [I]),
            "mxfp8_last_error": (ctypes.c_char_p, []),
            "mxfp8_quantize_act": (I, [P, I64, I64, I64, P, P, P]),
            "mxfp8_quantize_weight": (I, [P, I64, I64, I64, I, P, P, P]),
            "mxfp8_prepacked_bytes": (I64, [I64, I64, I]),
            "mxfp8_prepack_weight": (I, [P, I64, P, I64, I64, I64, I, P, P]),
            "mxfp8_unpack_weight": (I, [P, I64, I64, I, P, P, P]),
            "mxfp8_workspace_bytes": (I64, [I64, I64, I64, I]),
            "mxfp8_linear": (I, [P, I64, I64, P, I64, I, P, P, P, I64, P]),
            "mxfp8_linear_prequant": (I, [P, P, I64, I64, P, I64, I, P, P, P]),
            "mxfp8_set_tile_config": (I, [I, I]),
            "mxfp8_set_batch_invariant": (I, [I]),
            "mxfp8_set_batch_invariant_thread": (I, [I]),
            "mxfp8_linear_batched": (I, [P, I64, I64, I64, P, I64, I, P, P, P, I64, P]),
            "mxfp8_linear_prequant_batched": (I, [P, P, I64, I64, I64, P, I64, I, P, P, P]),
            "mxfp8_prepack_weight_shuffled16": (I, [P, P, I64, I64, I64, P, P]),
            "mxfp8_unpack_weight_shuffled16": (I, [P, I64, I64, P, P, P]),
            "mxfp8_quantize_act_fmt": (I, [P, I64, I64, I64, I, P, P, P]),
            "mxfp8_workspace_bytes_fmt": (I64, [I64, I64, I64, I, I]),
            "mxfp8_linear_fmt": (I, [P, I64, I64, P, I64, I, I, P, P, P, I64, P]),
            "mxfp8_linear_prequant_fmt": (I, [P, P, I64, I64, I, P, I64, I, P, P, P]),
            "mxfp8_rmsnorm_quantize_act": (I, [P, I64, I64, I64, P, ctypes.c_float, P, P, P, P]),
            "mxfp8_linear_noalloc": (I, [P, I64, I64, P, I64, I, P, P, P]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype, fn.argtypes = res, args
        _lib = L
    return _lib


def _check(rc):
    if rc != 0:
        raise MXError(rc, lib().mxfp8_last_error().decode())


def _fmt(fmt):
    return FMT[fmt] if isinstance(fmt, str) else int(fmt)


def _u8(t, name):
    if t.dtype not in (torch.uint8, torch.float8_e4m3fn, torch.float8_e8m0fnu):
        raise TypeError("%s must be uint8 / float8 bytes, got %s" % (name, t.dtype))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    return t.view(torch.uint8)


def _bf16(t, name):
    if t.dtype != torch.bfloat16:
        raise TypeError("%s must be bfloat16, got %s" % (name, t.dtype))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    return t


def _on_gpu(ref, **tensors):
    """Every tensor handed to the library must be a CUDA tensor on ref's device.  Checked after
    the shape checks, so those run (and raise) without a GPU too."""
    for name, t in (("x", ref),) + tuple(tensors.items()):
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("%s must be a CUDA tensor" % name)
        if t.device != ref.device:
            raise ValueError("%s is on %s, the activations on %s" % (name, t.device, ref.device))


def _stream(t):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _out(out, shape, ref):
    """The caller's output tensor (bf16, contiguous, exactly ``shape``), or a new one on ref's
    device.  The kernels write every element of it, so a wrong shape would be an out-of-bounds
    write: it is rejected here."""
    if out is None:
        return torch.empty(shape, dtype=torch.bfloat16, device=ref.device)
    _bf16(out, "out")
    if tuple(out.shape) != tuple(shape):
        raise ValueError("out has shape %s, the layer writes %s"
                         % (tuple(out.shape), tuple(shape)))
    return out


def _bias(bias, shape):
    """None, or a contiguous bf16 tensor of exactly ``shape`` ([N], or [B, N] when batched)."""
    if bias is None:
        return None
    _bf16(bias, "bias")
    if tuple(bias.shape) != tuple(shape):
        raise ValueError("bias has shape %s, need %s" % (tuple(bias.shape), tuple(shape)))
    return bias


def _packed(packed, N, K, f, batch=1):
    """A prepacked weight buffer of exactly ``batch`` weights of N x K in format f."""
    packed = _u8(packed, "packed")
    need = batch * prepacked_bytes(N, K, f)
    if need <= 0 or packed.numel() != need:
        raise ValueError("packed holds %d bytes; %d prepacked weight(s) of N = %d, K = %d in "
                         "format %d hold %d" % (packed.numel(), batch, N, K, f, need))
    return packed


def _workspace_arg(workspace, need):
    if workspace.dtype != torch.uint8 or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous uint8 tensor (new_workspace)")
    if workspace.numel() < need:
        raise ValueError("workspace holds %d bytes, the call needs %d"
                         % (workspace.numel(), need))
    return workspace


def _ptr(t):
    return 0 if t is None else t.data_ptr()


def set_tile_config(fn=0, fm=0):
    """Force the tiled GEMM's tile (tuning/testing); (0, 0) = automatic."""
    _check(lib().mxfp8_set_tile_config(int(fn), int(fm)))


def set_batch_invariant(on=True):
    """Batch-invariant mode: a row's result no longer depends on the number of rows M."""
    _check(lib().mxfp8_set_batch_invariant(1 if on else 0))


def set_batch_invariant_thread(mode):
    """Batch-invariant mode for the calling thread only: True / False, or None to follow the
    process-wide setting again."""
    _check(lib().mxfp8_set_batch_invariant_thread(-1 if mode is None else (1 if mode else 0)))


def device_supported(device=0):
    return lib().mxfp8_device_supported(int(device)) == 1


def prepacked_bytes(N, K, fmt="e4m3"):
    return int(lib().mxfp8_prepacked_bytes(N, K, _fmt(fmt)))


def workspace_bytes(M, N, K, fmt="e4m3"):
    return int(lib().mxfp8_workspace_bytes(M, N, K, _fmt(fmt)))


def new_workspace(nbytes, device="cuda"):
    """A workspace for the ``workspace=`` arguments: ``nbytes`` (from workspace_bytes) of device
    memory, zero-filled.  Its first 64 KiB are counters that must be zero before the first call
    and that every call leaves zero; a workspace allocated otherwise must be zeroed once."""
    return torch.zeros(max(int(nbytes), 1), dtype=torch.uint8, device=device)


def _rows(x, name):
    """x [..., K] -> (x as [M, K], leading shape, K)."""
    if x.dim() < 1:
        raise ValueError("%s must have a last dimension K" % name)
    K = x.shape[-1]
    return x.reshape(-1, K), x.shape[:-1], K


def quantize_act(x):
    """bf16 x [..., K] -> (xq uint8 [M, K] E4M3, xs uint8 [M, K/32] E8M0), M = prod(lead)."""
    x = _bf16(x, "x")
    x2, _, K = _rows(x, "x")
    M = x2.shape[0]
    _on_gpu(x)
    xq = torch.empty((M, K), dtype=torch.uint8, device=x.device)
    xs = torch.empty((M, K // 32), dtype=torch.uint8, device=x.device)
    _check(lib().mxfp8_quantize_act(x2.data_ptr(), M, K, K, xq.data_ptr(), xs.data_ptr(),
                                    _stream(x)))
    return xq, xs


def rmsnorm_quantize_act(x, gamma, eps=1e-6, return_y=False):
    """Fused RMS norm + MXFP8 quantization of bf16 x [..., K] with bf16 weight gamma [K]:
    (xq [M, K] E4M3, xs [M, K/32] E8M0) ready for linear_prequant, plus the normalized bf16
    rows y [M, K] when return_y."""
    x = _bf16(x, "x")
    gamma = _bf16(gamma, "gamma")
    x2, _, K = _rows(x, "x")
    if tuple(gamma.shape) != (K,):
        raise ValueError("gamma must be [K]")
    M = x2.shape[0]
    _on_gpu(x, gamma=gamma)
    xq = torch.empty((M, K), dtype=torch.uint8, device=x.device)
    xs = torch.empty((M, K // 32), dtype=torch.uint8, device=x.device)
    y = torch.empty((M, K), dtype=torch.bfloat16, device=x.device) if return_y else None
    _check(lib().mxfp8_rmsnorm_quantize_act(x2.data_ptr(), M, K, K, gamma.data_ptr(), float(eps),
                                            xq.data_ptr(), xs.data_ptr(), _ptr(y), _stream(x)))
    return (xq, xs, y) if return_y else (xq, xs)


def quantize_weight(w, fmt="e4m3"):
    """bf16 W [N, K] -> (wq [N, K] E4M3 or [N, 3K/4] packed FP6, ws [N, K/32] E8M0)."""
    w = _bf16(w, "w")
    if w.dim() != 2:
        raise ValueError("w must be [N, K]")
    N, K = w.shape
    f = _fmt(fmt)
    _on_gpu(w)
    wq = torch.empty((N, K if f == 0 else K // 4 * 3), dtype=torch.uint8, device=w.device)
    ws = torch.empty((N, K // 32), dtype=torch.uint8, device=w.device)
    _check(lib().mxfp8_quantize_weight(w.data_ptr(), N, K, K, f, wq.data_ptr(), ws.data_ptr(),
                                       _stream(w)))
    return wq, ws


def _weight_scales(ws):
    if ws.dtype not in (torch.uint8, torch.float8_e8m0fnu):
        raise TypeError("ws must be uint8 / float8_e8m0fnu")
    if ws.dim() != 2 or ws.stride(-1) != 1:
        raise ValueError("ws must be 2-D with contiguous rows")
    return ws.view(torch.uint8)


def prepack_weight(wq, ws, fmt="e4m3", K=None):
    """Quantized weight (wq [N, row bytes], ws [>=N, >=K/32]) -> prepacked uint8 buffer."""
    f = _fmt(fmt)
    wq = _u8(wq, "wq")
    ws = _weight_scales(ws)
    if wq.dim() != 2:
        raise ValueError("wq must be [N, row bytes]")
    N = wq.shape[0]
    if K is None:
        K = wq.shape[1] if f == 0 else wq.shape[1] // 3 * 4
    if wq.shape[1] < (K if f == 0 else K // 4 * 3):
        raise ValueError("wq rows hold %d bytes, K = %d needs more" % (wq.shape[1], K))
    if ws.shape[0] < N or ws.shape[1] < K // 32:
        raise ValueError("ws %s is smaller than [N, K/32] = [%d, %d]"
                         % (tuple(ws.shape), N, K // 32))
    _on_gpu(wq, ws=ws)
    out = torch.empty(prepacked_bytes(N, K, f), dtype=torch.uint8, device=wq.device)
    _check(lib().mxfp8_prepack_weight(wq.data_ptr(), wq.stride(0), ws.data_ptr(), ws.stride(0),
                                      N, K, f, out.data_ptr(), _stream(wq)))
    return out


def prepack_weight_shuffled16(w16, ws, N, K):
    """E4M3 weight in the aiter (16, 16) preshuffled order (N * K bytes) + scales -> prepacked."""
    w16 = _u8(w16, "w16")
    if w16.numel() != N * K:
        raise ValueError("w16 must hold N * K = %d bytes" % (N * K))
    ws = _weight_scales(ws)
    if ws.shape[0] < N or ws.shape[1] < K // 32:
        raise ValueError("ws %s is smaller than [N, K/32] = [%d, %d]"
                         % (tuple(ws.shape), N, K // 32))
    _on_gpu(w16, ws=ws)
    out = torch.empty(prepacked_bytes(N, K, 0), dtype=torch.uint8, device=w16.device)
    _check(lib().mxfp8_prepack_weight_shuffled16(w16.data_ptr(), ws.data_ptr(), ws.stride(0), N, K,
                                                 out.data_ptr(), _stream(w16)))
    return out


def unpack_weight_shuffled16(packed, N, K):
    """Prepacked E4M3 weight -> (w16 uint8 [N * K] in the aiter (16, 16) order, ws [N, K/32])."""
    packed = _packed(packed, N, K, 0)
    _on_gpu(packed)
    w16 = torch.empty(N * K, dtype=torch.uint8, device=packed.device)
    ws = torch.empty((N, K // 32), dtype=torch.uint8, device=packed.device)
    _check(lib().mxfp8_unpack_weight_shuffled16(packed.data_ptr(), N, K, w16.data_ptr(),
                                                ws.data_ptr(), _stream(packed)))
    return w16, ws


def unpack_weight(packed, N, K, fmt="e4m3"):
    """Prepacked weight -> (wq [N, K] E4M3 or [N, 3K/4] FP6, ws [N, K/32]): the exact inverse."""
    f = _fmt(fmt)
    packed = _packed(packed, N, K, f)
    _on_gpu(packed)
    wq = torch.empty((N, K if f == 0 else K // 4 * 3), dtype=torch.uint8, device=packed.device)
    ws = torch.empty((N, K // 32), dtype=torch.uint8, device=packed.device)
    _check(lib().mxfp8_unpack_weight(packed.data_ptr(), N, K, f, wq.data_ptr(), ws.data_ptr(),
                                     _stream(packed)))
    return wq, ws


_ws_cache = {}


def _workspace(device, stream, nbytes):
    key = (device, stream)
    t = _ws_cache.get(key)
    if t is None or t.numel() < nbytes:
        t = new_workspace(nbytes, device)
        _ws_cache[key] = t
    return t


def _act_row_bytes(K, afmt):
    return K if afmt == 0 else K // 4 * 3


def _prequant_acts(xq, xs, K, a, lead=()):
    """Checks pre-quantized activations: xq [*lead, M, row bytes of K in format a], xs
    [*lead, M, K/32] (the aiter_flydsl page asserts exactly this scale shape)."""
    xq = _u8(xq, "xq")
    xs = _u8(xs, "xs")
    nl = len(lead)
    if xq.dim() != nl + 2:
        raise ValueError("xq must be %d-D" % (nl + 2))
    M = xq.shape[nl]
    if tuple(xq.shape) != tuple(lead) + (M, _act_row_bytes(K, a)) or \
            tuple(xs.shape) != tuple(lead) + (M, K // 32):
        raise ValueError("activation codes %s / scales %s do not match K = %d in format %d: "
                         "need %s and %s row-major"
                         % (tuple(xq.shape), tuple(xs.shape), K, a,
                            tuple(lead) + (M, _act_row_bytes(K, a)), tuple(lead) + (M, K // 32)))
    return xq, xs, M


def linear_fmt(x, packed, N, fmt, afmt, bias=None, out=None, workspace=None):
    """linear() with the activations quantized to afmt (FP6 afmt needs an FP6 weight fmt)."""
    x = _bf16(x, "x")
    f, a = _fmt(fmt), _fmt(afmt)
    x2, lead, K = _rows(x, "x")
    M = x2.shape[0]
    packed = _packed(packed, N, K, f)
    bias = _bias(bias, (N,))
    y = _out(out, (M, N) if out is None or out.dim() == 2 else tuple(lead) + (N,), x)
    need = workspace_bytes_fmt(M, N, K, f, a)
    if workspace is not None:
        workspace = _workspace_arg(workspace, need)
    _on_gpu(x, packed=packed, bias=bias, out=y, workspace=workspace)
    st = _stream(x)
    ws = workspace if workspace is not None else _workspace(x.device, st.value, need)
    _check(lib().mxfp8_linear_fmt(x2.data_ptr(), M, K, packed.data_ptr(), N, f, a, _ptr(bias),
                                  y.data_ptr(), ws.data_ptr(), ws.numel(), st))
    return y.reshape(*lead, N)


def linear(x, packed, N, fmt="e4m3", bias=None, out=None, workspace=None):
    """y = MX-quantized x [..., K] times the prepacked weight, (+ bias), bf16 [..., N].

    ``out``: optional bf16 tensor of shape [M, N] or [..., N].  ``workspace``: a uint8 device
    tensor of at least workspace_bytes(M, N, K, fmt) bytes from new_workspace (zero-filled); by
    default one is kept per device and stream."""
    return linear_fmt(x, packed, N, fmt, "e4m3", bias, out, workspace)


NOALLOC_SCRATCH_BYTES = 64 << 20


def linear_noalloc(x, packed, N, fmt="e4m3", bias=None, out=None):
    """linear() without a workspace: the library's static per-GPU scratch array serves as one
    (mxfp8_linear_noalloc), so the call allocates nothing on the library side.  Pass ``out`` to
    allocate nothing at all.  Shapes whose workspace exceeds NOALLOC_SCRATCH_BYTES are refused;
    calls that overlap on one GPU race on the shared array."""
    x = _bf16(x, "x")
    f = _fmt(fmt)
    x2, lead, K = _rows(x, "x")
    M = x2.shape[0]
    packed = _packed(packed, N, K, f)
    bias = _bias(bias, (N,))
    y = _out(out, (M, N) if out is None or out.dim() == 2 else tuple(lead) + (N,), x)
    _on_gpu(x, packed=packed, bias=bias, out=y)
    _check(lib().mxfp8_linear_noalloc(x2.data_ptr(), M, K, packed.data_ptr(), N, f, _ptr(bias),
                                      y.data_ptr(), _stream(x)))
    return y.reshape(*lead, N)


def linear_prequant_fmt(xq, xs, packed, N, K, fmt, afmt, bias=None, out=None):
    """linear_prequant() with activations in format afmt: xq [M, K] E4M3 or [M, 3K/4] FP6."""
    f, a = _fmt(fmt), _fmt(afmt)
    xq, xs, M = _prequant_acts(xq, xs, K, a)
    packed = _packed(packed, N, K, f)
    bias = _bias(bias, (N,))
    y = _out(out, (M, N), xq)
    _on_gpu(xq, xs=xs, packed=packed, bias=bias, out=y)
    _check(lib().mxfp8_linear_prequant_fmt(xq.data_ptr(), xs.data_ptr(), M, K, a,
                                           packed.data_ptr(), N, f, _ptr(bias), y.data_ptr(),
                                           _stream(xq)))
    return y


def linear_prequant(xq, xs, packed, N, fmt="e4m3", bias=None, out=None, lead_shape=None):
    """Same layer from pre-quantized activations: xq [M, K] E4M3, xs [M, K/32] row-major."""
    if xq.dim() != 2:
        raise ValueError("xq must be [M, K]")
    y = linear_prequant_fmt(xq, xs, packed, N, xq.shape[1], fmt, "e4m3", bias, out)
    return y if lead_shape is None else y.reshape(*lead_shape, N)


def linear_batched(x, packed, N, fmt="e4m3", bias=None, out=None, workspace=None):
    """x bf16 [B, M, K], packed = B prepacked weights back to back (torch.cat of
    prepack_weight outputs), bias bf16 [B, N] or None -> y bf16 [B, M, N]."""
    x = _bf16(x, "x")
    f = _fmt(fmt)
    if x.dim() != 3:
        raise ValueError("x must be [B, M, K]")
    B, M, K = x.shape
    packed = _packed(packed, N, K, f, batch=B)
    bias = _bias(bias, (B, N))
    y = _out(out, (B, M, N), x)
    need = workspace_bytes(B * M, N, K, f)
    if workspace is not None:
        workspace = _workspace_arg(workspace, need)
    _on_gpu(x, packed=packed, bias=bias, out=y, workspace=workspace)
    st = _stream(x)
    ws = workspace if workspace is not None else _workspace(x.device, st.value, need)
    _check(lib().mxfp8_linear_batched(x.data_ptr(), B, M, K, packed.data_ptr(), N, f, _ptr(bias),
                                      y.data_ptr(), ws.data_ptr(), ws.numel(), st))
    return y


def linear_prequant_batched(xq, xs, packed, N, fmt="e4m3", bias=None, out=None):
    """xq E4M3 [B, M, K], xs E8M0 [B, M, K/32] -> y bf16 [B, M, N] (weights as linear_batched)."""
    f = _fmt(fmt)
    if xq.dim() != 3:
        raise ValueError("xq must be [B, M, K]")
    B, K = xq.shape[0], xq.shape[2]
    xq, xs, M = _prequant_acts(xq, xs, K, 0, lead=(B,))
    packed = _packed(packed, N, K, f, batch=B)
    bias = _bias(bias, (B, N))
    y = _out(out, (B, M, N), xq)
    _on_gpu(xq, xs=xs, packed=packed, bias=bias, out=y)
    _check(lib().mxfp8_linear_prequant_batched(xq.data_ptr(), xs.data_ptr(), B, M, K,
                                               packed.data_ptr(), N, f, _ptr(bias), y.data_ptr(),
                                               _stream(xq)))
    return y


# ---------------------------------------------------------------- MXFP6 activations
# (mxfp6 page, MxFp6LinearLayerConfig.activation_quant_key): activations quantized to E2M3 or
# E3M2 (packed four codes per three bytes), with FP6 weights; afmt "e4m3" gives the layer above.

def workspace_bytes_fmt(M, N, K, fmt, afmt):
    return int(lib().mxfp8_workspace_bytes_fmt(M, N, K, _fmt(fmt), _fmt(afmt)))


def quantize_act_fmt(x, afmt):
    """bf16 x [..., K] -> (xq uint8 [M, K] E4M3 or [M, 3K/4] packed FP6, xs uint8 [M, K/32])."""
    x = _bf16(x, "x")
    a = _fmt(afmt)
    x2, _, K = _rows(x, "x")
    M = x2.shape[0]
    _on_gpu(x)
    xq = torch.empty((M, _act_row_bytes(K, a)), dtype=torch.uint8, device=x.device)
    xs = torch.empty((M, K // 32), dtype=torch.uint8, device=x.device)
    _check(lib().mxfp8_quantize_act_fmt(x2.data_ptr(), M, K, K, a, xq.data_ptr(), xs.data_ptr(),
                                        _stream(x)))
    return xq, xs


class MxLinear:
    """A linear layer whose quantized weight is prepacked once (load time) and applied per call.

    ``wq``/``ws`` are the checkpoint tensors (weight [N, K] E4M3 or [N, 3K/4] FP6 bytes,
    weight_scale [N', K'/32] E8M0 with N' >= N, K' >= K, sliced to [:N, :K/32])."""

    def __init__(self, wq, ws, fmt="e4m3", bias=None, K=None):
        self.fmt = _fmt(fmt)
        self.N = wq.shape[0]
        self.K = K if K is not None else (wq.shape[1] if self.fmt == 0 else wq.shape[1] // 3 * 4)
        self.packed = prepack_weight(wq, ws, self.fmt, K=self.K)
        self.bias = bias

    def __call__(self, x):
        return linear(x, self.packed, self.N, self.fmt, self.bias)

    def apply_quantized(self, xq, xs, lead_shape=None):
        return linear_prequant(xq, xs, self.packed, self.N, self.fmt, self.bias,
                               lead_shape=lead_shape)

    def row_major_weight(self):
        """The weight back in checkpoint layout (exact inverse of the prepack)."""
        return unpack_weight(self.packed, self.N, self.K, self.fmt)
