"""Pins for the oracle's RMS-norm producer of pre-quantized activations (CPU only).

Reading (the Mxfp8LinearKernel page's input_quant_key: activations may arrive quantized from an
upstream op; the pages name no producer): each fp32 quantity of an fp32 RMS norm is the value
nearest to its exact definition,
    r32 = fp32(1 / sqrt(sum_k x_k^2 / K + eps)),   p_k = fp32(x_k * r32),
    t_k = bf16(p_k),                               y_k = bf16(t_k * gamma_k).
Pins, none of which re-types the oracle's float arithmetic:
  * closed forms: constant rows (y = sign(c) * gamma), an eps-dominated row whose r is a power
    of two, invariance under power-of-two scaling, a hand-computed row;
  * an exact-rational evaluation of the reading (every rounding decided on Fractions, the
    square root by comparing squares) on rows of several K and eps, bit for bit;
  * rows found by search where each plausible misreading (r left unrounded, p not rounded to
    fp32, gamma applied before t is rounded, sum instead of mean, eps outside the root) gives
    other bits than the reading, so that a mistake of that kind in the oracle fails.
"""
from fractions import Fraction

import numpy as np
import pytest

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


# ---------------------------------------------------------------- exact-rational evaluation

_F32 = (23, -126)          # stored mantissa bits, smallest normal exponent
_BF16 = (7, -126)
_HALF = Fraction(1, 2)


def _floor_log2(a):
    """floor(log2 a) for a positive Fraction, exactly."""
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    return e


def _rne(v, fmt):
    """v (Fraction) rounded to the nearest value of a binary format, ties to the even code."""
    if v == 0:
        return Fraction(0)
    mb, emin = fmt
    a = abs(v)
    ulp = Fraction(2) ** (max(_floor_log2(a), emin) - mb)
    q = a / ulp
    n = q.numerator // q.denominator
    rem = q - n
    if rem > _HALF or (rem == _HALF and n % 2 == 1):
        n += 1
    return n * ulp if v > 0 else -n * ulp


def _f32_neighbours(c):
    b = int(np.array([float(c)], np.float32).view(np.uint32)[0])
    return [_f32(v) for v in range(b - 3, b + 4)]


def _rne_f32_of_ratio_root(num, D):
    """fp32 value nearest to num / sqrt(D) (num a Fraction, D > 0 a Fraction): the candidate
    interval is chosen by comparing squares, so no square root is ever rounded."""
    if num == 0:
        return Fraction(0)
    a2 = num * num / D                                  # the square of the exact magnitude
    est = abs(float(num)) / float(D) ** 0.5
    cands = _f32_neighbours(est)
    best = None
    for lo, hi in zip(cands, cands[1:]):
        mid = (lo + hi) / 2
        if lo * lo <= a2 <= hi * hi:
            if a2 < mid * mid:
                best = lo
            elif a2 > mid * mid:
                best = hi
            else:                                       # exact tie: the even code
                bl = int(np.array([float(lo)], np.float32).view(np.uint32)[0])
                best = lo if bl % 2 == 0 else hi
            break
    assert best is not None, "estimate too far from the exact value"
    return best if num > 0 else -best


def _bf16_bits_of(v):
    """bits of a Fraction that is exactly a bf16 value."""
    if v == 0:
        return 0
    f = np.array([float(v)], np.float32)
    assert Fraction(float(f[0])) == v
    return int(f.view(np.uint32)[0] >> 16)


def _bf16_frac(bits):
    return Fraction(float(np.array([int(bits) << 16], np.uint32).view(np.float32)[0]))


def _rne_f32_eps_outside(m, e):
    """fp32 value nearest to 1 / (sqrt(m) + e) (a misreading of where eps goes): c lies at or
    below the exact value iff c * e <= 1 and c^2 m <= (1 - c e)^2."""
    at_or_below = lambda c: c * e <= 1 and c * c * m <= (1 - c * e) ** 2
    cands = _f32_neighbours(1.0 / (float(m) ** 0.5 + float(e)))
    for lo, hi in zip(cands, cands[1:]):
        if at_or_below(lo) and not at_or_below(hi):
            mid = (lo + hi) / 2
            if not at_or_below(mid):
                return lo
            if mid * mid * m == (1 - mid * e) ** 2:
                bl = int(np.array([float(lo)], np.float32).view(np.uint32)[0])
                return lo if bl % 2 == 0 else hi
            return hi
    raise AssertionError("estimate too far from the exact value")


def exact_row(xb, gb, eps, variant="reading"):
    """y bits of one row under the reading (or a named misreading), all in exact arithmetic."""
    K = len(xb)
    xs = [_bf16_frac(v) for v in xb]
    gs = [_bf16_frac(v) for v in gb]
    e = Fraction(float(eps))
    S = sum(v * v for v in xs)
    D = (S if variant == "sum_not_mean" else S / K) + (0 if variant == "eps_outside" else e)
    if variant == "eps_outside":
        r32 = _rne_f32_eps_outside(D, e)
    else:
        r32 = _rne_f32_of_ratio_root(Fraction(1), D)
    out = []
    sign = lambda bits: int(bits) >> 15                   # IEEE signed zero: sign of x * gamma
    for xbits, gbits, xv, gv in zip(xb, gb, xs, gs):
        if variant == "r_exact":
            p = _rne_f32_of_ratio_root(xv, D)          # fp32(x * r), r unrounded
        elif variant == "single":
            p = xv * r32                               # no fp32 rounding of the product
        else:
            p = _rne(xv * r32, _F32)
        if variant == "gamma_first":
            y = _rne(p * gv, _BF16)                    # t never rounded to bf16
        else:
            t = _rne(p, _BF16)
            y = _rne(t * gv, _BF16)
        out.append(_bf16_bits_of(y) if y != 0 else 0x8000 * (sign(xbits) ^ sign(gbits)))
    return np.array(out, np.uint16)


def _rows(seed, R, K):
    g = np.random.default_rng(seed)
    x = synth.bf16_bits(g.standard_normal((R, K)).astype(np.float32))
    gamma = synth.bf16_bits(g.uniform(0.25, 2.0, K).astype(np.float32))
    return x, gamma


def test_eps_dominated_row_closed_form(orc):
    """x_k = 2^-16 for all k, eps = 3 * 2^-32: mean(x^2) = 2^-32, so r = 1 / sqrt(2^-30) =
    2^15 exactly, p = t = 1/2 and y = bf16(gamma / 2) = gamma with its exponent lowered by one.
    Without eps r would be 2^16 (y = gamma); eps added outside the root, or to the sum rather
    than the mean, gives neither."""
    K = 64
    x = synth.bf16_bits(np.full((1, K), 2.0 ** -16, np.float32))
    g = np.random.default_rng(3)
    gamma = synth.bf16_bits(g.uniform(-2.0, 2.0, K).astype(np.float32))
    eps = 3.0 * 2.0 ** -32
    y, pre = orc.rmsnorm(x, gamma, eps)
    assert np.all(pre == 0.5)
    expect = synth.bf16_bits((tolerance.bf16_to_f64(gamma) / 2).astype(np.float32))
    assert np.array_equal(y[0], expect)
    for v in ("eps_outside", "sum_not_mean"):
        assert not np.array_equal(exact_row(x[0], gamma, eps, v), expect), v


@pytest.mark.parametrize("K,eps", [(32, 0.0), (96, float(np.float32(1e-6))), (608, 0.5),
                                   (4096, float(np.float32(1e-5)))])
def test_exact_evaluation_several_k_and_eps(orc, K, eps):
    """The oracle equals the exact-rational evaluation of the reading, bit for bit, on seeded
    N(0,1) rows with outliers (eps = 0.5 with K = 608 makes eps comparable to the mean of
    rows scaled down by 2^-1..2^-3)."""
    R = 3 if K >= 4096 else 6
    x, gamma = _rows(K + R, R, K)
    if eps == 0.5:
        xd = tolerance.bf16_to_f64(x) * np.ldexp(1.0, -np.arange(1, R + 1))[:, None]
        x = synth.bf16_bits(xd.astype(np.float32))
    y, _ = orc.rmsnorm(x, gamma, eps)
    for i in range(R):
        assert np.array_equal(y[i], exact_row(x[i], gamma, eps)), (K, eps, i)


def _find(pred, seed, K=32, R=1 << 16, eps=float(np.float32(1e-6))):
    """First seeded row (K = 32) that a cheap float screen flags for pred; the flag is then
    confirmed in exact arithmetic by the caller."""
    x, gamma = _rows(seed, R, K)
    xd = tolerance.bf16_to_f64(x)
    r = 1.0 / np.sqrt((xd * xd).sum(1) / K + eps)
    r32 = r.astype(np.float32)
    p = xd.astype(np.float32) * r32[:, None]
    idx = np.nonzero(pred(xd, r, r32, p).any(1))[0]
    return x, gamma, eps, idx


def _midpoint_screen(xd, r, r32, p):
    # the fp32 product sits exactly on a bf16 rounding midpoint but the exact product does not
    on_mid = (p.view(np.uint32) & 0xFFFF) == 0x8000
    return on_mid & (xd * r32.astype(np.float64)[:, None] != p.astype(np.float64))


def _root_screen(xd, r, r32, p):
    # rounding r to fp32 moves the product across a bf16 rounding boundary
    return synth.bf16_bits((xd * r[:, None]).astype(np.float32)) != synth.bf16_bits(p)


@pytest.mark.parametrize("variant,screen", [("single", _midpoint_screen),
                                            ("r_exact", _root_screen)])
def test_rows_where_a_rounding_step_decides_the_bits(orc, variant, screen):
    """Rows where leaving out one of the reading's fp32 roundings (of the product, or of r)
    changes at least one output bit: the oracle must agree with the reading there, so a
    mistake of that kind in it fails."""
    x, gamma, eps, idx = _find(screen, seed=11)
    found = 0
    for i in idx[:40]:
        want = exact_row(x[i], gamma, eps)
        alt = exact_row(x[i], gamma, eps, variant)
        if np.array_equal(want, alt):
            continue
        y, _ = orc.rmsnorm(x[i:i + 1], gamma, eps)
        assert np.array_equal(y[0], want), (variant, int(i))
        found += 1
        if found == 3:
            break
    assert found >= 1, "no discriminating row in the seeded sample"


def test_gamma_applied_after_t_is_rounded(orc):
    """t = bf16(p) is rounded before the gamma product: applying gamma to p instead changes
    bits on ordinary rows, and the oracle follows the reading."""
    x, gamma = _rows(5, 4, 256)
    y, _ = orc.rmsnorm(x, gamma, 1e-6)
    for i in range(4):
        want = exact_row(x[i], gamma, 1e-6)
        assert np.array_equal(y[i], want)
        assert not np.array_equal(want, exact_row(x[i], gamma, 1e-6, "gamma_first"))
        assert not np.array_equal(want, exact_row(x[i], gamma, 1e-6, "sum_not_mean"))
