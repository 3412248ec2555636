"""Pins for the oracle's fp64 linear layer and the tolerance check (CPU only).

The layer is y = dequant(x_q, s_x) . dequant(W_q, s_w)^T (+ bias), bf16 out (aiter_flydsl page,
AiterFlyDSLMxfp8LinearKernel.apply_weights; weight/scale shapes from the
compressed_tensors_w8a8_mxfp8 page, create_weights).  Pins: exact integer products against numpy
int64 matmul, one-hot identity, scale linearity, zero blocks, torch's fp64 matmul, agreement of
the two oracle paths, and planted mistakes that the tolerance must reject.
"""
import numpy as np
import pytest
import torch

from mx_block_scaled_amd import synth
from tests import tolerance


def _e4m3_code_of_int(orc):
    """code for each small integer -16..16, found by decode search (not by the encoder)."""
    table = {}
    for c in range(256):
        v = orc.decode(c, 0)
        if np.isfinite(v) and v == int(v) and abs(v) <= 16 and not (v == 0 and c != 0):
            table[int(v)] = c
    assert len(table) == 33
    return table


def test_exact_integer_gemm(orc):
    g = np.random.default_rng(0)
    M, N, K = 7, 24, 96
    xi = g.integers(-8, 9, (M, K))
    wi = g.integers(-8, 9, (N, K))
    t = _e4m3_code_of_int(orc)
    xq = np.vectorize(t.get)(xi).astype(np.uint8)
    wq = np.vectorize(t.get)(wi).astype(np.uint8)
    s1 = np.full((M, K // 32), 127, np.uint8)
    s2 = np.full((N, K // 32), 127, np.uint8)
    y = orc.matmul_nt(orc.dequantize(xq, s1), orc.dequantize(wq, s2))
    assert np.array_equal(y, (xi @ wi.T).astype(np.float64))
    ye = orc.linear_entries(xq, s1, wq, s2, np.repeat(np.arange(M), N), np.tile(np.arange(N), M))
    assert np.array_equal(ye.reshape(M, N), y)


def test_identity_weight(orc):
    g = np.random.default_rng(1)
    K = 128
    x = synth.bf16_bits(g.standard_normal((5, K)).astype(np.float32))
    xq, xs = orc.quantize(x)
    wq = np.zeros((K, K), np.uint8)
    wq[np.arange(K), np.arange(K)] = 0x38          # 1.0
    ws = np.full((K, K // 32), 127, np.uint8)
    y = orc.matmul_nt(orc.dequantize(xq, xs), orc.dequantize(wq, ws))
    assert np.array_equal(y, orc.dequantize(xq, xs))


def test_scale_linearity_and_zero_blocks(orc):
    d = synth.make("tiny")
    wq, ws = orc.quantize(d["w"])
    xq, xs = orc.quantize(d["x"])
    xd = orc.dequantize(xq, xs)
    y = orc.matmul_nt(xd, orc.dequantize(wq, ws))
    y2 = orc.matmul_nt(xd, orc.dequantize(wq, ws + 1))
    assert np.array_equal(y2, 2 * y)
    # zeroing one activation block removes exactly that block's contribution
    xq0 = xq.copy()
    xq0[:, 64:96] = 0
    y0 = orc.matmul_nt(orc.dequantize(xq0, xs), orc.dequantize(wq, ws))
    part = orc.matmul_nt(orc.dequantize(xq, xs)[:, 64:96].copy(),
                         orc.dequantize(wq, ws)[:, 64:96].copy())
    np.testing.assert_allclose(y - part, y0, rtol=0, atol=1e-12)


def test_against_torch_fp64(orc):
    d = synth.make("decode8", M=8)
    wq, ws = orc.quantize(d["w"][:512])
    ref, xq, xs = orc.linear_ref(d["x"], wq, ws, bias_bf16=d["bias"][:512])
    xd = torch.from_numpy(orc.dequantize(xq, xs))
    wd = torch.from_numpy(orc.dequantize(wq, ws))
    b = torch.from_numpy(tolerance.bf16_to_f64(d["bias"][:512]))
    tref = (xd @ wd.T + b).numpy()
    np.testing.assert_allclose(ref, tref, rtol=1e-12, atol=1e-12)


def test_entries_match_full(orc):
    d = synth.make("tiny")
    wq, ws = orc.quantize(d["w"])
    ref, xq, xs = orc.linear_ref(d["x"], wq, ws)
    g = np.random.default_rng(2)
    r = g.integers(0, 16, 300)
    c = g.integers(0, 256, 300)
    e = orc.linear_entries(xq, xs, wq, ws, r, c)
    np.testing.assert_allclose(e, ref[r, c], rtol=1e-13, atol=1e-13)


def test_fp6_weights_dequant(orc):
    """FP6 weights: the same linear with E2M3 / E3M2 codes equals torch's fp64 matmul."""
    g = np.random.default_rng(3)
    w = synth.bf16_bits((g.standard_normal((64, 256)) * 0.02).astype(np.float32))
    x = synth.laplace_bf16((8, 256), 0, 0)
    xq, xs = orc.quantize(x)
    for fmt in (2, 3):
        wq, ws = orc.quantize(w, fmt)
        assert wq.max() < 64
        ref = orc.matmul_nt(orc.dequantize(xq, xs), orc.dequantize(wq, ws, fmt))
        wd = torch.tensor([[orc.decode(int(c), fmt) for c in row] for row in wq], dtype=torch.float64)
        wd = wd * torch.from_numpy(np.ldexp(1.0, ws.astype(np.int64) - 127)).repeat_interleave(32, 1)
        tref = (torch.from_numpy(orc.dequantize(xq, xs)) @ wd.T).numpy()
        np.testing.assert_allclose(ref, tref, rtol=1e-12, atol=1e-14)
        e = orc.linear_entries(xq, xs, wq, ws, np.arange(8), np.arange(8), wfmt=fmt)
        np.testing.assert_allclose(e, ref[np.arange(8), np.arange(8)], rtol=1e-13)


# ---------------------------------------------------------------- the tolerance itself

def _bf16_of(ref):
    return synth.bf16_bits(ref.astype(np.float32))


def test_tolerance_accepts_rounded_reference(orc):
    d = synth.make("tiny")
    wq, ws = orc.quantize(d["w"])
    ref, _, _ = orc.linear_ref(d["x"], wq, ws)
    ok, rep = tolerance.check(_bf16_of(ref), ref)
    assert ok, rep
    # an fp32 accumulation in another order, then bf16 rounding (what a correct GPU result
    # looks like) passes too
    xq, xs = orc.quantize(d["x"])
    y32 = (orc.dequantize(xq, xs).astype(np.float32)[:, ::-1] @
           orc.dequantize(wq, ws).astype(np.float32)[:, ::-1].T)
    ok, rep = tolerance.check(_bf16_of(y32.astype(np.float64)), ref)
    assert ok, rep


@pytest.mark.parametrize("mistake", ["drop_block", "scale_off_by_one_block", "transposed_scale",
                                     "missing_bias", "x_scale_from_w", "sign_flip_one_block"])
def test_tolerance_rejects_planted_mistakes(orc, mistake):
    """A plausible mistake planted in the oracle's computation must fail the acceptance check."""
    d = synth.make("decode8", M=8)
    N = 256
    w, bias = d["w"][:N], d["bias"][:N]
    wq, ws = orc.quantize(w)
    ref, xq, xs = orc.linear_ref(d["x"], wq, ws, bias_bf16=bias)
    xd = orc.dequantize(xq, xs)
    wd = orc.dequantize(wq, ws)
    b = tolerance.bf16_to_f64(bias)
    if mistake == "drop_block":
        xd2 = xd.copy()
        xd2[:, 32 * 57:32 * 58] = 0
        bad = orc.matmul_nt(xd2, wd, b)
    elif mistake == "scale_off_by_one_block":
        ws2 = np.roll(ws, 1, axis=1)
        bad = orc.matmul_nt(xd, orc.dequantize(wq, ws2), b)
    elif mistake == "transposed_scale":
        ws2 = ws.reshape(-1)[: N * 128].reshape(128, N).T.copy()
        bad = orc.matmul_nt(xd, orc.dequantize(wq, ws2), b)
    elif mistake == "missing_bias":
        bad = orc.matmul_nt(xd, wd, None)
    elif mistake == "x_scale_from_w":
        bad = orc.matmul_nt(orc.dequantize(xq, ws[:8]), wd, b)
    else:
        wd2 = wd.copy()
        wd2[:, 32 * 3:32 * 4] *= -1
        bad = orc.matmul_nt(xd, wd2, b)
    ok, rep = tolerance.check(_bf16_of(bad), ref)
    assert not ok, (mistake, rep)


# ---------------------------------------------------------------- MXFP6 activations

def _fp6_code_of_int(orc, fmt):
    """code of each integer in -7..7 representable in the format (found by decode search)."""
    table = {}
    for c in range(64):
        v = orc.decode(c, fmt)
        if v == int(v) and abs(v) <= 7 and not (v == 0 and c != 0):
            table[int(v)] = c
    return table


@pytest.mark.parametrize("xfmt,wfmt", [(2, 2), (3, 2), (2, 3), (3, 3), (2, 0)])
def test_exact_integer_gemm_fp6_activations(orc, xfmt, wfmt):
    """MXFP6 activations (the mxfp6 page's activation_quant_key): small integers with scale
    byte 127 give exactly numpy's int64 matmul, through both oracle paths."""
    g = np.random.default_rng(10 + xfmt * 4 + wfmt)
    M, N, K = 6, 20, 160
    tx = _fp6_code_of_int(orc, xfmt)
    tw = _fp6_code_of_int(orc, wfmt) if wfmt else _e4m3_code_of_int(orc)
    vals = sorted(set(tx) & set(tw))
    assert {-7, -4, -3, 0, 1, 3, 4, 7} <= set(vals) or {-4, -3, 0, 1, 3, 4} <= set(vals)
    xi = g.choice(vals, (M, K))
    wi = g.choice(vals, (N, K))
    xq = np.vectorize(tx.get)(xi).astype(np.uint8)
    wq = np.vectorize(tw.get)(wi).astype(np.uint8)
    s1 = np.full((M, K // 32), 127, np.uint8)
    s2 = np.full((N, K // 32), 127, np.uint8)
    exact = (xi @ wi.T).astype(np.float64)
    y = orc.matmul_nt(orc.dequantize(xq, s1, xfmt), orc.dequantize(wq, s2, wfmt))
    assert np.array_equal(y, exact)
    ye = orc.linear_entries(xq, s1, wq, s2, np.repeat(np.arange(M), N), np.tile(np.arange(N), M),
                            wfmt=wfmt, xfmt=xfmt)
    assert np.array_equal(ye.reshape(M, N), exact)


def test_fp6_activation_scales_and_reference(orc):
    """linear_ref with MXFP6 activations: x is quantized with the format's own emax (E2M3: a
    block whose amax is 2^j gets byte j - 2 + 127), and scaling one activation block's scale
    byte by +1 doubles exactly that block's contribution."""
    K = 64
    x = np.zeros((2, K), np.float32)
    x[0, :32] = 1.0                      # amax 2^0 -> E2M3 byte 125, E3M2 byte 123
    x[0, 32:] = 3.0                      # amax 1.5 * 2^1 -> E2M3 byte 126, E3M2 byte 124
    x[1, :] = -0.25                      # amax 2^-2 -> E2M3 byte 123, E3M2 byte 121
    xb = synth.bf16_bits(x)
    wq = np.zeros((16, K), np.uint8)
    wq[:, :] = 0x38                      # E4M3 1.0
    ws = np.full((16, K // 32), 127, np.uint8)
    for fmt, emax in ((2, 2), (3, 4)):
        ref, xq, xs = orc.linear_ref(xb, wq, ws, xfmt=fmt)
        assert xs.tolist() == [[127 - emax, 128 - emax], [125 - emax, 125 - emax]]
        # every value is exactly representable, so y is the exact row sum
        np.testing.assert_array_equal(ref[:, 0], [32 * 1.0 + 32 * 3.0, -0.25 * 64])
        xs2 = xs.copy()
        xs2[0, 1] += 1
        y2 = orc.matmul_nt(orc.dequantize(xq, xs2, fmt), orc.dequantize(wq, ws))
        np.testing.assert_array_equal(y2[0, 0], 32 * 1.0 + 2 * 32 * 3.0)
