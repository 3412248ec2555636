"""Pins for the oracle's RMS-norm producer of pre-quantized activations (CPU only).

Reading (the Mxfp8LinearKernel page's input_quant_key: activations may arrive quantized from an
upstream op; the pages name no producer): y = bf16(bf16(x * r) * gamma) with
r = 1 / sqrt(mean(x^2) + eps) in fp64.  Pins: constant rows (y = sign(c) * gamma exactly),
invariance under power-of-two scaling, a hand-computed row with exact rationals, and torch's
fp64 computation (equal up to the last bit of r; bf16 results equal away from rounding ties).
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
        # x * r is within one fp64 rounding of +-1
        np.testing.assert_allclose(np.abs(pre), 1.0, rtol=4e-16)


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


def test_hand_computed_row(orc):
    """x = (3, 4, 0, ..., 0), K = 32, eps = 1/8, gamma = (1.5, -0.5, 1, ...): mean of squares
    25/32, r = 1 / sqrt(25/32 + 1/8) = 1 / sqrt(29/32); values checked with exact rationals
    (r enters only through its square: t = bf16(3 r) is the nearest bf16 to the real 3 r)."""
    K = 32
    x = np.zeros((1, K), np.float32)
    x[0, 0], x[0, 1] = 3.0, 4.0
    gamma = np.ones(K, np.float32)
    gamma[0], gamma[1] = 1.5, -0.5
    y, pre = orc.rmsnorm(synth.bf16_bits(x), synth.bf16_bits(gamma), 0.125)
    r2 = Fraction(32, 29)              # r^2

    def nearest_bf16_of_root(c):       # bf16 nearest to c * r = sqrt(c^2 r^2), c > 0
        target = c * c * r2
        cands = []
        for bits in range(0x3F80, 0x4200):
            v = Fraction(float(np.array([bits << 16], np.uint32).view(np.float32)[0]))
            cands.append((abs(v * v - target), bits))   # monotone in |v - c r| for v > 0
        return min(cands)[1]

    t0 = nearest_bf16_of_root(3)
    t1 = nearest_bf16_of_root(4)
    f0 = Fraction(float(np.array([t0 << 16], np.uint32).view(np.float32)[0]))
    f1 = Fraction(float(np.array([t1 << 16], np.uint32).view(np.float32)[0]))
    assert y[0, 0] == _bf16_exact(f0 * Fraction(3, 2))
    assert y[0, 1] == _bf16_exact(-f1 / 2)
    assert np.all(y[0, 2:] == 0)
    assert abs(Fraction(pre[0, 0]) ** 2 - 9 * r2) < Fraction(1, 10 ** 14)


def test_against_torch_fp64(orc):
    d = synth.make("prefill", M=64, with_w=False)
    x = d["x"]
    g = np.random.default_rng(2)
    gamma = synth.bf16_bits(g.uniform(0.25, 2.0, x.shape[1]).astype(np.float32))
    eps = 1e-6
    y, pre = orc.rmsnorm(x, gamma, eps)
    xt = torch.from_numpy(tolerance.bf16_to_f64(x))
    r = 1.0 / torch.sqrt((xt * xt).mean(dim=1, keepdim=True) + eps)
    tp = (xt * r).numpy()
    np.testing.assert_allclose(pre, tp, rtol=1e-15, atol=0)
    # bf16 results: equal wherever x * r is not close to a bf16 rounding tie (the reference
    # here rounds fp64 -> fp32 -> bf16, which differs from one rounding only within 2^-16 of
    # a bf16 ulp from a tie)
    t_ref = synth.bf16_bits(tp.astype(np.float32))
    g64 = tolerance.bf16_to_f64(gamma)
    y_ref = synth.bf16_bits((tolerance.bf16_to_f64(t_ref) * g64).astype(np.float32))
    a = np.abs(pre)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    q = a / np.exp2(e - 7)
    near_tie = np.abs(q - np.floor(q) - 0.5) < 2.0 ** -15
    assert near_tie.sum() < 100
    assert np.array_equal(y[~near_tie], y_ref[~near_tie])
