"""numpy / ctypes driver for the C oracle in ``mx_oracle.c`` (test infrastructure only).

Every array argument is a numpy array on the host; nothing here touches a GPU.
Format ids: E4M3 = 0, E2M3 = 2, E3M2 = 3 (elements), E8M0 scales as uint8.
"""
import ctypes
import os
import subprocess

import numpy as np

__all__ = [
    "E4M3", "E2M3", "E3M2", "build", "lib", "threads",
    "bf16_to_f64", "f64_to_bf16", "decode", "encode", "encode_many", "scale_byte", "scale_value",
    "quantize", "dequantize", "fp6_pack", "fp6_unpack", "shuffle16", "unshuffle16",
    "matmul_nt", "linear_entries", "linear_ref", "rmsnorm",
]

E4M3, E2M3, E3M2 = 0, 2, 3

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "mx_oracle.c")
_LIB = os.path.join(_HERE, "libmxoracle.so")
_lib = None


def build(force=True):
    """Compile the oracle with gcc (-O2, no fast-math: fp64 semantics are the point)."""
    if not force and os.path.exists(_LIB) and os.path.getmtime(_LIB) >= os.path.getmtime(_SRC):
        return _LIB
    tmp = _LIB + ".tmp%d" % os.getpid()
    subprocess.run(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-Wall",
                    "-o", tmp, _SRC, "-lm"], check=True)
    os.replace(tmp, _LIB)
    return _LIB


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        L = ctypes.CDLL(_LIB)
        P, I64, I, D = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_double
        sig = {
            "orc_bf16_to_double": (D, [ctypes.c_uint16]),
            "orc_double_to_bf16": (ctypes.c_uint16, [D]),
            "orc_decode": (D, [I, I]),
            "orc_encode": (I, [D, I]),
            "orc_encode_many": (I, [P, I64, I, P]),
            "orc_scale_byte": (I, [D, I]),
            "orc_scale_value": (D, [I]),
            "orc_quantize": (I, [P, I64, I64, I64, I, P, P]),
            "orc_dequantize": (I, [P, P, I64, I64, I, P]),
            "orc_fp6_pack": (I, [P, I64, I64, P]),
            "orc_fp6_unpack": (I, [P, I64, I64, P]),
            "orc_shuffle16": (I, [P, I64, I64, P]),
            "orc_unshuffle16": (I, [P, I64, I64, P]),
            "orc_matmul_nt": (None, [P, P, P, I64, I64, I64, P]),
            "orc_linear_entries": (I, [P, P, I64, P, P, I, P, P, P, I64, P]),
            "orc_linear_entries_fmt": (I, [P, P, I, I64, P, P, I, P, P, P, I64, P]),
            "orc_threads": (I, []),
            "orc_rmsnorm": (I, [P, I64, I64, I64, P, D, P, P]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype, fn.argtypes = res, args
        _lib = L
    return _lib


def _p(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def threads():
    return lib().orc_threads()


# ---------------------------------------------------------------- scalars

def bf16_to_f64(bits):
    """uint16 bf16 bit patterns -> exact float64 (vectorised through the C routine's rule)."""
    b = _c(bits, np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def f64_to_bf16(v):
    """float64 -> bf16 bits, round to nearest even (reporting only)."""
    L = lib()
    v = np.asarray(v, dtype=np.float64)
    return np.array([L.orc_double_to_bf16(float(t)) for t in v.ravel()],
                    dtype=np.uint16).reshape(v.shape)


def decode(code, fmt=E4M3):
    return lib().orc_decode(int(code), int(fmt))


def encode(v, fmt=E4M3):
    return lib().orc_encode(float(v), int(fmt))


def encode_many(v, fmt=E4M3):
    """orc_encode over a float64 array -> uint8 codes of the same shape."""
    a = _c(v, np.float64)
    out = np.empty(a.shape, np.uint8)
    if lib().orc_encode_many(_p(a), a.size, fmt, _p(out)) != 0:
        raise ValueError("bad format")
    return out


def scale_byte(amax, fmt=E4M3):
    return lib().orc_scale_byte(float(amax), int(fmt))


def scale_value(byte):
    return lib().orc_scale_value(int(byte))


# ---------------------------------------------------------------- arrays

def quantize(x_bf16, fmt=E4M3):
    """bf16 bits [rows, K] -> (codes uint8 [rows, K], scales uint8 [rows, K/32])."""
    x = _c(x_bf16, np.uint16)
    rows, K = x.shape
    codes = np.empty((rows, K), np.uint8)
    scales = np.empty((rows, K // 32), np.uint8)
    if lib().orc_quantize(_p(x), rows, K, K, fmt, _p(codes), _p(scales)) != 0:
        raise ValueError("orc_quantize: bad format or K %% 32 != 0")
    return codes, scales


def dequantize(codes, scales, fmt=E4M3):
    c, s = _c(codes, np.uint8), _c(scales, np.uint8)
    rows, K = c.shape
    assert s.shape == (rows, K // 32)
    out = np.empty((rows, K), np.float64)
    if lib().orc_dequantize(_p(c), _p(s), rows, K, fmt, _p(out)) != 0:
        raise ValueError("orc_dequantize: bad format or K")
    return out


def fp6_pack(codes):
    c = _c(codes, np.uint8)
    rows, K = c.shape
    out = np.empty((rows, 3 * K // 4), np.uint8)
    if lib().orc_fp6_pack(_p(c), rows, K, _p(out)) != 0:
        raise ValueError("K % 4 != 0")
    return out


def fp6_unpack(packed, K):
    p = _c(packed, np.uint8)
    rows = p.shape[0]
    assert p.shape[1] == 3 * K // 4
    out = np.empty((rows, K), np.uint8)
    if lib().orc_fp6_unpack(_p(p), rows, K, _p(out)) != 0:
        raise ValueError("K % 4 != 0")
    return out


def shuffle16(w):
    """Row-major [N, K] bytes -> the (16, 16) preshuffled order, flat [N*K]."""
    w = _c(w, np.uint8)
    N, K = w.shape
    out = np.empty(N * K, np.uint8)
    if lib().orc_shuffle16(_p(w), N, K, _p(out)) != 0:
        raise ValueError("N % 16 or K % 32")
    return out


def unshuffle16(s, N, K):
    s = _c(s, np.uint8).reshape(-1)
    assert s.size == N * K
    out = np.empty((N, K), np.uint8)
    if lib().orc_unshuffle16(_p(s), N, K, _p(out)) != 0:
        raise ValueError("N % 16 or K % 32")
    return out


def matmul_nt(xd, wd, bias=None):
    xd, wd = _c(xd, np.float64), _c(wd, np.float64)
    M, K = xd.shape
    N = wd.shape[0]
    assert wd.shape[1] == K
    b = None if bias is None else _c(bias, np.float64)
    y = np.empty((M, N), np.float64)
    lib().orc_matmul_nt(_p(xd), _p(wd), None if b is None else _p(b), M, N, K, _p(y))
    return y


def linear_entries(xq, xs, wq, ws, rows, cols, wfmt=E4M3, bias=None, xfmt=E4M3):
    """Reference y[rows[i], cols[i]] straight from quantized operands (codes one per byte);
    xfmt is the activation codes' format (E4M3, or E2M3 / E3M2 for MXFP6 activations)."""
    xq, xs, wq, ws = (_c(a, np.uint8) for a in (xq, xs, wq, ws))
    K = xq.shape[1]
    assert wq.shape[1] == K and xs.shape[1] == K // 32 and ws.shape[1] == K // 32
    r, c = _c(rows, np.int64), _c(cols, np.int64)
    assert r.shape == c.shape
    b = None if bias is None else _c(bias, np.float64)
    out = np.empty(r.shape, np.float64)
    rc = lib().orc_linear_entries_fmt(_p(xq), _p(xs), xfmt, K, _p(wq), _p(ws), wfmt,
                                      None if b is None else _p(b), _p(r), _p(c), r.size, _p(out))
    if rc != 0:
        raise ValueError("orc_linear_entries: bad format or K")
    return out


def linear_ref(x_bf16, wq, ws, wfmt=E4M3, bias_bf16=None, xfmt=E4M3):
    """Full fp64 reference of the linear layer from bf16 activations:
    quantize x (format xfmt, E4M3 by default; row-major scales), dequantize both operands,
    multiply, add bias.  Returns (y, x codes one per byte, x scales)."""
    xq, xs = quantize(x_bf16, xfmt)
    xd = dequantize(xq, xs, xfmt)
    wd = dequantize(wq, ws, wfmt)
    bias = None if bias_bf16 is None else bf16_to_f64(bias_bf16)
    return matmul_nt(xd, wd, bias), xq, xs


def rmsnorm(x_bf16, gamma_bf16, eps):
    """RMS norm of bf16 rows [rows, K] with a bf16 weight [K] (mx_oracle.c, orc_rmsnorm) ->
    (y bf16 bits [rows, K], p = fp32(x * fp32(r)) as float64, the value t = bf16(p) rounds)."""
    x = _c(x_bf16, np.uint16)
    g = _c(gamma_bf16, np.uint16)
    rows, K = x.shape
    assert g.shape == (K,)
    y = np.empty((rows, K), np.uint16)
    pre = np.empty((rows, K), np.float64)
    if lib().orc_rmsnorm(_p(x), rows, K, K, _p(g), float(eps), _p(y), _p(pre)) != 0:
        raise ValueError("orc_rmsnorm: bad K or eps")
    return y, pre
