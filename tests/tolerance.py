"""Acceptance check for the bf16 output of the linear layer against the fp64 oracle.

Per element:   |y - ref| <= 2 * ulp_bf16(|ref|) + 1e-3 * rms(ref)
Whole output:  ||y - ref||_F / ||ref||_F <= 5e-3
with ulp_bf16(a) = 2^(max(floor(log2 a), -126) - 7) and ulp_bf16(0) = 2^-133.

Why this is the right size: the E4M3 x E4M3 (or FP6) products are exact and each 32-block's
partial sum is exact in fp32; what differs from the fp64 reference is the fp32 accumulation
across K/32 blocks (relative error ~ sqrt(K/32) * 2^-24 of the running sum) and the final bf16
rounding (half an ulp).  Two ulps cover the rounding; 1e-3 * rms covers accumulation error on
outputs that cancel to near zero.  A dropped block, a wrong scale index or a transposed operand
moves outputs by O(rms), which this bound rejects (see tests/test_oracle_gemm.py).
"""
import numpy as np


def bf16_to_f64(bits):
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def ulp_bf16(a):
    a = np.abs(np.asarray(a, np.float64))
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.maximum(e, -126)
    return np.where(a > 0, np.ldexp(1.0, (e - 7).astype(np.int64)), 2.0 ** -133)


def check(y_bits, ref, rms=None, name=""):
    """Return (ok, report).  ``y_bits`` bf16 bit patterns, ``ref`` fp64 of the same shape;
    ``rms`` of the full reference when ``ref`` is a sample of a larger output."""
    y = bf16_to_f64(y_bits).reshape(ref.shape)
    ref = np.asarray(ref, np.float64)
    if rms is None:
        rms = float(np.sqrt(np.mean(ref ** 2))) if ref.size else 0.0
    err = np.abs(y - ref)
    bound = 2.0 * ulp_bf16(ref) + 1e-3 * rms
    finite = np.isfinite(y).all()
    viol = err > bound
    nref = float(np.linalg.norm(ref))
    rel_frob = float(np.linalg.norm(y - ref) / nref) if nref > 0 else float(np.linalg.norm(y))
    ok = bool(finite and not viol.any() and rel_frob <= 5e-3)
    rep = dict(name=name, n=int(ref.size), violations=int(viol.sum()), rel_frob=rel_frob,
               max_err_over_bound=float((err / bound).max()) if ref.size else 0.0,
               finite=bool(finite))
    return ok, rep
