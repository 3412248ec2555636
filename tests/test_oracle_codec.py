"""Pins for the oracle's element codec and E8M0 scale rule (CPU only).

The pages (compressed_tensors_w8a8_mxfp8: E4M3 float8_e4m3fn values, uint8 E8M0 scales per 32;
mxfp6: E2M3 / E3M2) name the formats; the conversion rule is the OCP MX v1.0 one.  Each check
below pins the oracle to something other than itself: hand-derived blocks, brute-force nearest
search over the enumerated code values, torch's own float8_e4m3fn cast, closed forms.
"""
import os

import numpy as np
import pytest
import torch

from mx_block_scaled_amd.synth import bf16_bits

FMTS = {"E4M3": 0, "E2M3": 2, "E3M2": 3}
# magnitude bits of each format's largest finite code, from the format definitions
MAXCODE = {0: 0x7E, 2: 0x1F, 3: 0x1F}
SIGN = {0: 0x80, 2: 0x20, 3: 0x20}
EMAX = {0: 8, 2: 2, 3: 4}


def _all_bf16_finite():
    b = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    finite = (b & 0x7F80) != 0x7F80
    return b[finite]


def _bf16_f64(b):
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _value_table(orc, fmt):
    """(codes, values) of every finite non-negative code, increasing — enumerated by decode,
    then cross-checked below against the format's definition for a few known codes."""
    codes = np.arange(MAXCODE[fmt] + 1)
    vals = np.array([orc.decode(int(c), fmt) for c in codes])
    return codes, vals


def _brute_nearest(a, codes, vals):
    """Nearest code to |v| by search over the enumerated values, ties to the even code,
    saturating at the largest value.  Independent of the oracle's exponent arithmetic."""
    idx = np.searchsorted(vals, a, side="right") - 1      # vals[idx] <= a
    idx = np.clip(idx, 0, len(vals) - 1)
    hi = np.clip(idx + 1, 0, len(vals) - 1)
    dl = a - vals[idx]
    dh = vals[hi] - a
    pick = np.where(dl < dh, idx, np.where(dh < dl, hi, np.where(codes[idx] % 2 == 0, idx, hi)))
    pick = np.where(a >= vals[-1], len(vals) - 1, pick)
    return codes[pick]


# ---------------------------------------------------------------- known code values

def test_known_code_values(orc):
    # E4M3 (OCP "fn"): bias 7, 3 mantissa bits; max 448, NaN at S.1111.111
    assert orc.decode(0x00, 0) == 0.0
    assert orc.decode(0x01, 0) == 2.0 ** -9          # smallest subnormal
    assert orc.decode(0x07, 0) == 7 * 2.0 ** -9
    assert orc.decode(0x08, 0) == 2.0 ** -6          # smallest normal
    assert orc.decode(0x38, 0) == 1.0
    assert orc.decode(0x7E, 0) == 448.0
    assert np.isnan(orc.decode(0x7F, 0)) and np.isnan(orc.decode(0xFF, 0))
    assert orc.decode(0xB8, 0) == -1.0
    assert np.signbit(orc.decode(0x80, 0))
    # E2M3: bias 1, max 7.5, subnormal step 1/8
    assert orc.decode(0x01, 2) == 0.125 and orc.decode(0x08, 2) == 1.0
    assert orc.decode(0x1F, 2) == 7.5 and orc.decode(0x3F, 2) == -7.5
    # E3M2: bias 3, max 28, subnormal step 1/16
    assert orc.decode(0x01, 3) == 0.0625 and orc.decode(0x04, 3) == 0.25
    assert orc.decode(0x0C, 3) == 1.0 and orc.decode(0x1F, 3) == 28.0
    # tables are strictly increasing in the code (what the brute force relies on)
    for fmt in FMTS.values():
        _, v = _value_table(orc, fmt)
        assert np.all(np.diff(v) > 0)


def test_torch_e4m3_decode_agrees(orc):
    # torch's float8_e4m3fn is the OCP E4M3FN type the pages store weights in
    codes = np.arange(256, dtype=np.uint8)
    tv = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ov = np.array([orc.decode(int(c), 0) for c in codes])
    same = (tv == ov) | (np.isnan(tv) & np.isnan(ov))
    assert same.all()


# ---------------------------------------------------------------- element encode

@pytest.mark.parametrize("name", list(FMTS))
def test_encode_exhaustive_vs_bruteforce(orc, name):
    """Every finite bf16 x every scale byte 0..254: v = x * 2^(127 - byte) (exact in fp64)."""
    fmt = FMTS[name]
    codes, vals = _value_table(orc, fmt)
    xb = _all_bf16_finite()
    x = _bf16_f64(xb)
    for byte in range(0, 255):
        v = np.ldexp(x, 127 - byte)
        got = orc.encode_many(v, fmt)
        exp = _brute_nearest(np.abs(v), codes, vals).astype(np.int64)
        exp = exp | np.where(np.signbit(v), SIGN[fmt], 0)
        bad = np.nonzero(got.astype(np.int64) != exp)[0]
        assert bad.size == 0, (name, byte, hex(int(xb[bad[0]])), int(got[bad[0]]), int(exp[bad[0]]))


def test_encode_vs_torch_cast(orc):
    """torch CPU clamp(v, -448, 448).to(float8_e4m3fn) on values exact in fp32."""
    g = np.random.default_rng(1)
    xb = _all_bf16_finite()
    x = _bf16_f64(xb)
    for e in range(-20, 21, 3):
        v = np.ldexp(x, -e)
        ok = (np.abs(v) < 2.0 ** 100) & ((np.abs(v) > 2.0 ** -100) | (v == 0))
        v = v[ok]
        t = torch.from_numpy(v.astype(np.float32)).clamp(-448, 448)
        tc = t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        oc = orc.encode_many(v, 0)
        assert np.array_equal(tc, oc), e
    # random fp32 values inside the range, finer than bf16
    v = g.standard_normal(200000).astype(np.float32) * np.float32(100.0)
    tc = torch.from_numpy(v).clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(tc, orc.encode_many(v.astype(np.float64), 0))


def test_encode_special_points(orc):
    assert orc.encode(464.0, 0) == 0x7E          # tie 448 / 480 -> even mantissa (448)
    assert orc.encode(1e30, 0) == 0x7E           # saturate, never NaN
    assert orc.encode(-1e30, 0) == 0xFE
    assert orc.encode(float("inf"), 0) == 0x7E
    assert orc.encode(2.0 ** -10, 0) == 0x00     # tie 0 / 2^-9 -> even (0)
    assert orc.encode(3 * 2.0 ** -10, 0) == 0x02
    assert orc.encode(-1e-4, 0) == 0x80          # negative underflow keeps the sign
    assert orc.encode(-0.0, 0) == 0x80
    assert orc.encode(0.0, 0) == 0x00
    assert orc.encode(7.75, 2) == 0x1F and orc.encode(100.0, 3) == 0x1F
    # binade edge: 15.5 is halfway between 15 (0x57, odd) and 16 (0x58, even) -> 16
    assert orc.encode(15.5, 0) == 0x58


# ---------------------------------------------------------------- E8M0 scale

@pytest.mark.parametrize("name", list(FMTS))
def test_scale_byte_closed_forms(orc, name):
    fmt = FMTS[name]
    assert orc.scale_byte(0.0, fmt) == 0
    assert orc.scale_byte(float("inf"), fmt) == 0xFF
    assert orc.scale_byte(float("nan"), fmt) == 0xFF
    for j in range(-133, 128):                     # every power of two bf16 can hold
        lo = 2.0 ** j
        hi = (2.0 - 2.0 ** -7) * 2.0 ** j          # largest bf16 in the same binade
        want = min(max(j - EMAX[fmt] + 127, 0), 254)
        assert orc.scale_byte(lo, fmt) == want, j
        if j >= -126:
            assert orc.scale_byte(hi, fmt) == want, j


def test_scale_value(orc):
    assert orc.scale_value(127) == 1.0
    assert orc.scale_value(0) == 2.0 ** -127
    assert orc.scale_value(254) == 2.0 ** 127
    assert np.isnan(orc.scale_value(255))
    # torch's E8M0 type reads the same bytes the same way
    b = np.arange(255, dtype=np.uint8)
    tv = torch.from_numpy(b).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    assert np.array_equal(tv, np.array([orc.scale_value(int(i)) for i in b]))


# ---------------------------------------------------------------- whole blocks

def _parse_golden():
    path = os.path.join(os.path.dirname(__file__), "golden", "mx_blocks.txt")
    cases = []
    for line in open(path):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        fmt, byte, vals, codes = (t.strip() for t in line.split("|"))

        def expand(tok, conv):
            out = []
            for t in tok.split():
                if "*" in t:
                    v, n = t.split("*")
                    out += [conv(v)] * int(n)
                else:
                    out.append(conv(t))
            return out
        v = expand(vals, float)
        c = expand(codes, lambda t: int(t, 16))
        assert len(v) == 32 and len(c) == 32, line
        cases.append((FMTS[fmt], int(byte), v, c))
    return cases


def test_golden_blocks(orc):
    cases = _parse_golden()
    assert len(cases) >= 8
    for fmt, byte, vals, codes in cases:
        xb = bf16_bits(np.array(vals, np.float32)).reshape(1, 32)
        q, s = orc.quantize(xb, fmt)
        assert int(s[0, 0]) == byte, (fmt, vals[:4])
        assert q[0].tolist() == codes, (fmt, vals[:8], q[0][:8].tolist())


def test_quantize_idempotent(orc):
    """Re-quantizing a dequantized block (scales not clamped) reproduces codes and scales."""
    g = np.random.default_rng(5)
    for fmt in FMTS.values():
        x = bf16_bits((g.standard_normal((64, 256)) * np.exp(g.uniform(-20, 20, (64, 1))))
                      .astype(np.float32))
        q, s = orc.quantize(x, fmt)
        d = orc.dequantize(q, s, fmt)
        xb2 = bf16_bits(d.astype(np.float32))
        assert np.array_equal(_bf16_f64(xb2), d)           # dequantized values fit bf16
        q2, s2 = orc.quantize(xb2, fmt)
        assert np.array_equal(s, s2) and np.array_equal(q, q2)


def test_quantize_block_structure(orc):
    """Scale bytes come from each block's own amax; the largest element lands in the top binade."""
    g = np.random.default_rng(7)
    x = bf16_bits((g.standard_normal((8, 512)) * 3).astype(np.float32))
    q, s = orc.quantize(x, 0)
    xf = _bf16_f64(x).reshape(8, 16, 32)
    amax = np.abs(xf).max(axis=2)
    assert np.array_equal(s, np.floor(np.log2(amax)).astype(int) - 8 + 127)
    top = np.abs(np.array([[orc.decode(int(c), 0) for c in row] for row in q])).reshape(8, 16, 32)
    assert np.all((top.max(axis=2) >= 256) & (top.max(axis=2) <= 448))


def test_nonfinite_block_convention(orc):
    """Reading c-6 (the pages print no case): a block holding Inf or NaN has a NaN shared scale
    (the OCP MX rule), and every element of it is NaN.  Pinned against torch's own formats, not
    the oracle's decoder: the scale byte is the NaN of float8_e8m0fnu, the E4M3 codes are NaN
    under float8_e4m3fn, so the block dequantizes to NaN element by element; FP6 has no NaN
    code, and its elements are NaN through the scale.  The other block is quantized as usual."""
    import torch
    for bad in (0x7F80, 0xFF80, 0x7FC0):   # +Inf, -Inf, NaN
        x = np.zeros((1, 64), np.uint16)
        x[0, 3] = bad                      # block 0
        x[0, 40] = 0x3F80                  # 1.0 in block 1
        for fmt in (0, 2, 3):
            q, s = orc.quantize(x, fmt)
            sv = torch.tensor(s[0].astype(np.uint8)).view(torch.float8_e8m0fnu).float()
            assert torch.isnan(sv[0]) and not torch.isnan(sv[1])
            if fmt == 0:
                qv = torch.tensor(q[0].astype(np.uint8)).view(torch.float8_e4m3fn).float()
                deq = qv.reshape(2, 32) * sv[:, None]
                assert torch.isnan(deq[0]).all() and deq[1, 8] == 1.0
                assert not torch.isnan(deq[1]).any()
            else:
                deq0 = np.array([orc.decode(int(c), fmt) for c in q[0, :32]]) * float(sv[0])
                assert np.isnan(deq0).all()
    # the codes the oracle writes: E4M3's NaN code, FP6 zero
    x = np.zeros((1, 64), np.uint16)
    x[0, 3] = 0x7F80
    q, s = orc.quantize(x, 0)
    assert s[0].tolist() == [0xFF, 0] and set(q[0, :32].tolist()) == {0x7F}
