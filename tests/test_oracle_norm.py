"""Pins for the oracle's RMS-norm producer of pre-quantized activations (CPU only).

Reading (the Mxfp8LinearKernel page's input_quant_key: activations may arrive quantized from an
upstream op; the pages name no producer): y = bf16(bf16(fp32(x * fp32(r))) * gamma) with
r = 1 / sqrt(mean(x^2) + eps) in fp64.  Pins: constant rows (y = sign(c) * gamma exactly),
invariance under power-of-two scaling, a hand-computed row with exact rationals, and torch's
fp64 / fp32 computation (bit-equal wherever fp32(r) agrees).
"""
from fractions import Fraction

import numpy as np
import torch

from mx_block_scaled_amd import synth
from tests import tolerance


def _bf16_exact(f):
    """bf16 bits of the value nearest to Fraction f (ties to even), by brute force over the
    bf16 values of the right binade (no float arithmetic)."""
    sign = 0x8000 if f < 0 else 0
    a = abs(f)
    if a == 0:
        return sign
    e = 0
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    ulp = Fraction(2) ** (e - 7)
    q = a / ulp                       # in [128, 256)
    lo = int(q)
    frac = q - lo
    n = lo + (1 if frac > Fraction(1, 2) or (frac == Fraction(1, 2) and lo % 2 == 1) else 0)
    v = n * ulp
    bits = np.array([float(v)], np.float32).view(np.uint32)[0] >> 16
    return sign | int(bits)


def test_constant_rows(orc):
    K = 96
    g = np.random.default_rng(0)
    gamma = synth.bf16_bits((g.standard_normal(K) * 2).astype(np.float32))
    for c in (1.0, -3.0, 0.15625, 1e-3, -250.0):
        x = synth.bf16_bits(np.full((1, K), c, np.float32))
        y, pre = orc.rmsnorm(x, gamma, 0.0)
        expect = gamma if c > 0 else gamma ^ 0x8000
        assert np.array_equal(y[0], expect), c
        # fp32(x * fp32(1/|x|)) is within two fp32 roundings of +-1
        np.testing.assert_allclose(np.abs(pre), 1.0, rtol=2.0 ** -22)


def test_power_of_two_scaling(orc):
    g = np.random.default_rng(1)
    x = g.standard_normal((4, 256)).astype(np.float32)
    gamma = synth.bf16_bits(g.uniform(0.5, 2.0, 256).astype(np.float32))
    xb = synth.bf16_bits(x)
    y0, p0 = orc.rmsnorm(xb, gamma, 0.0)
    for j in (-20, -3, 5, 30):
        xj = synth.bf16_bits(np.ldexp(tolerance.bf16_to_f64(xb), j).astype(np.float32))
        yj, pj = orc.rmsnorm(xj, gamma, 0.0)
        assert np.array_equal(yj, y0) and np.array_equal(pj, p0), j


def _f32(bits):
    return Fraction(float(np.array([bits], np.uint32).view(np.float32)[0]))


def _nearest_f32(f):
    """bits of the fp32 value nearest to the positive Fraction f (ties to even)."""
    b = int(np.array([float(f)], np.float32).view(np.uint32)[0])    # within an ulp
    best = None
    for c in range(b - 2, b + 3):
        d = abs(_f32(c) - f)
        if best is None or d < best[0] or (d == best[0] and c % 2 == 0):
            best = (d, c)
    return best[1]


def test_hand_computed_row(orc):
    """x = (3, 4, 0, ..., 0), K = 32, eps = 1/8, gamma = (1.5, -0.5, 1, ...): mean of squares
    25/32, r = 1 / sqrt(29/32).  r32 is found with exact rationals (r enters through r^2 only:
    the nearest fp32 to r is the candidate c with the smallest |c - r|, decided by comparing
    squares of midpoints with 32/29); the rest follows the reading step by step."""
    K = 32
    x = np.zeros((1, K), np.float32)
    x[0, 0], x[0, 1] = 3.0, 4.0
    gamma = np.ones(K, np.float32)
    gamma[0], gamma[1] = 1.5, -0.5
    y, pre = orc.rmsnorm(synth.bf16_bits(x), synth.bf16_bits(gamma), 0.125)
    r2 = Fraction(32, 29)
    c0 = int(np.array([float(29 / 32) ** -0.5], np.float32).view(np.uint32)[0])
    cands = list(range(c0 - 2, c0 + 3))
    r32 = None
    for a, b in zip(cands, cands[1:]):
        mid = (_f32(a) + _f32(b)) / 2
        if r2 < mid * mid:            # r below the midpoint of a and b
            r32 = _f32(a) if r32 is None else r32
    assert r32 is not None
    p0 = _f32(_nearest_f32(3 * r32))
    p1 = _f32(_nearest_f32(4 * r32))
    t0, t1 = _bf16_exact(p0), _bf16_exact(p1)
    f0 = Fraction(float(np.array([t0 << 16], np.uint32).view(np.float32)[0]))
    f1 = Fraction(float(np.array([t1 << 16], np.uint32).view(np.float32)[0]))
    assert y[0, 0] == _bf16_exact(f0 * Fraction(3, 2))
    assert y[0, 1] == _bf16_exact(-f1 / 2)
    assert np.all(y[0, 2:] == 0)
    assert Fraction(pre[0, 0]) == p0 and Fraction(pre[0, 1]) == p1


def test_against_torch(orc):
    d = synth.make("prefill", M=64, with_w=False)
    x = d["x"]
    g = np.random.default_rng(2)
    gamma = synth.bf16_bits(g.uniform(0.25, 2.0, x.shape[1]).astype(np.float32))
    eps = 1e-6
    y, pre = orc.rmsnorm(x, gamma, eps)
    xt = torch.from_numpy(tolerance.bf16_to_f64(x))
    r = 1.0 / torch.sqrt((xt * xt).mean(dim=1, keepdim=True) + eps)     # fp64, pairwise order
    r32 = r.float()
    p = xt.float() * r32                                                # fp32, one rounding
    t = p.bfloat16()
    yt = (t.float() * torch.from_numpy(tolerance.bf16_to_f64(gamma)).float()).bfloat16()
    ybits = yt.view(torch.int16).numpy().view(np.uint16)
    same_r = (r32.double() == torch.from_numpy(np.asarray(
        [[float(np.float32(1.0 / np.sqrt(np.sum(tolerance.bf16_to_f64(row) ** 2) / row.size + eps)))]
         for row in x]))).numpy().ravel()
    assert same_r.mean() > 0.9
    np.testing.assert_array_equal(pre[same_r], p.double().numpy()[same_r])
    np.testing.assert_array_equal(y[same_r], ybits[same_r])
