"""GPU parity of MXFP6 activations (mxfp6 page, MxFp6LinearLayerConfig.activation_quant_key:
the activation format of an MXFP6 layer) against the CPU oracle.

Quantizer: bf16 -> E2M3 / E3M2 codes packed four per three bytes + row-major E8M0 [M, K/32],
bit-exact, on an exhaustive (bf16 value, scale byte) sweep and on Inf/NaN/-0 blocks.  Layer:
FP6 activations times FP6 weights (both operands FP6, the MFMA's FP6 rate), per element within
the bar of tests/tolerance.py on shapes that exercise every compiled tile, ragged M / N tails,
remainder K steps and the generic kernel; sampled outputs at the MXFP6 workload's full size.
The pre-quantized entry fed the oracle's quantization reproduces the bf16 entry bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle as orc
from mx_block_scaled_amd import mxfp8, synth
from tests import tolerance
from tests.gpu_helpers import banner, bf16_dev, host_bf16_bits, host_u8, u8_dev
from tests.test_gpu_quant import _sweep_matrix

pytestmark = pytest.mark.gpu

FP6 = [2, 3]
PAIRS = [(2, 2), (2, 3), (3, 2), (3, 3)]     # (weight format, activation format)


@pytest.mark.parametrize("afmt", FP6)
def test_quantize_act_fp6_exhaustive_sweep(afmt):
    x = _sweep_matrix()
    banner("quantize_act fp6 sweep", afmt, x.shape)
    xq, xs = mxfp8.quantize_act_fmt(bf16_dev(x), afmt)
    rq, rs = orc.quantize(x, afmt)
    gs = host_u8(xs)
    bad = np.argwhere(gs != rs)
    assert bad.size == 0, bad[:5]
    gq = host_u8(xq)
    assert gq.shape == (x.shape[0], x.shape[1] // 4 * 3)
    codes = orc.fp6_unpack(gq, x.shape[1])
    bad = np.argwhere(codes != rq)
    assert bad.size == 0, [(int(x[i, j]), int(codes[i, j]), int(rq[i, j])) for i, j in bad[:5]]
    assert np.array_equal(gq, orc.fp6_pack(rq))


@pytest.mark.parametrize("afmt", FP6)
def test_quantize_act_fp6_nonfinite_ragged_strided(afmt):
    g = np.random.default_rng(30 + afmt)
    x = synth.bf16_bits((g.standard_normal((7, 96)) * 4).astype(np.float32))
    x[2, 5] = 0x7F80            # +Inf
    x[4, 70] = 0xFFC1           # NaN
    x[5, 32:64] = 0x8000        # a block of -0.0
    x[6, 0:32] = 0x0001         # bf16 subnormals only
    banner("quantize_act fp6 nonfinite", afmt)
    xq, xs = mxfp8.quantize_act_fmt(bf16_dev(x), afmt)
    rq, rs = orc.quantize(x, afmt)
    assert np.array_equal(host_u8(xs), rs)
    assert np.array_equal(host_u8(xq), orc.fp6_pack(rq))
    assert rs[2, 0] == 0xFF and rs[4, 2] == 0xFF and rs[5, 1] == 0
    # a row stride larger than K, through the C ABI
    big = synth.bf16_bits(g.standard_normal((5, 200)).astype(np.float32))
    t = bf16_dev(big)
    q = torch.empty((5, 120), dtype=torch.uint8, device=t.device)
    s = torch.empty((5, 5), dtype=torch.uint8, device=t.device)
    st = torch.cuda.current_stream().cuda_stream
    assert mxfp8.lib().mxfp8_quantize_act_fmt(t.data_ptr(), 5, 160, 200, afmt, q.data_ptr(),
                                              s.data_ptr(), st) == 0
    rq, rs = orc.quantize(np.ascontiguousarray(big[:, :160]), afmt)
    assert np.array_equal(host_u8(s), rs) and np.array_equal(host_u8(q), orc.fp6_pack(rq))


def _fp6_layer(w_bits, wfmt, bias_bits):
    wq, ws = orc.quantize(w_bits, wfmt)
    layer = mxfp8.MxLinear(u8_dev(orc.fp6_pack(wq)), u8_dev(ws), wfmt,
                           bias=None if bias_bits is None else bf16_dev(bias_bits))
    return layer, wq, ws


def _check_pair(x, w, b, wfmt, afmt, name):
    M, K = x.shape
    N = w.shape[0]
    layer, wq, ws = _fp6_layer(w, wfmt, b)
    y = mxfp8.linear_fmt(bf16_dev(x), layer.packed, N, wfmt, afmt, layer.bias)
    ref, xq, xs = orc.linear_ref(x, wq, ws, wfmt, b, xfmt=afmt)
    ok, rep = tolerance.check(host_bf16_bits(y), ref, name=name)
    assert ok, rep
    # the pre-quantized entry on the oracle's quantization: the same kernel, the same bits
    y2 = mxfp8.linear_prequant_fmt(u8_dev(orc.fp6_pack(xq)), u8_dev(xs), layer.packed, N, K,
                                   wfmt, afmt, layer.bias)
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16))
    return y


def _inputs(M, N, K, seed, bias=True):
    g = np.random.default_rng(seed)
    x = g.laplace(0.0, 1.0, (M, K)).astype(np.float32)
    x[:, g.choice(K, max(1, K // 100), replace=False)] *= 30.0       # outlier channels
    x = synth.bf16_bits(x)
    w = synth.bf16_bits((g.standard_normal((N, K)) * 0.02).astype(np.float32))
    b = synth.bf16_bits((g.standard_normal(N) * 0.01).astype(np.float32)) if bias else None
    return x, w, b


# tiled kernel (whole and remainder K-step groups, ragged tails) and the generic kernel (M < 64,
# K not a multiple of 128)
SHAPES = [(300, 592, 1024), (300, 592, 640), (64, 128, 512), (5, 48, 384), (33, 80, 1056),
          (100, 144, 544)]


@pytest.mark.parametrize("wfmt,afmt", PAIRS)
@pytest.mark.parametrize("M,N,K", SHAPES)
def test_w6a6_layer(M, N, K, wfmt, afmt):
    x, w, b = _inputs(M, N, K, M + N + K + 10 * wfmt + afmt, bias=(M % 2 == 0))
    banner("w6a6", M, N, K, wfmt, afmt)
    _check_pair(x, w, b, wfmt, afmt, "w6a6-%d-%d-%d-%d-%d" % (M, N, K, wfmt, afmt))


TILES = [(8, 4), (7, 4), (6, 4), (4, 4), (4, 2)]


@pytest.mark.parametrize("fn,fm", TILES)
def test_w6a6_every_tile(fn, fm):
    x, w, b = _inputs(300, 592, 640, fn * 10 + fm)
    banner("w6a6 tile", fn, fm)
    mxfp8.set_tile_config(fn, fm)
    try:
        _check_pair(x, w, b, 3, 2, "w6a6-tile-%d-%d" % (fn, fm))
    finally:
        mxfp8.set_tile_config(0, 0)


def test_w6a6_many_tiles_three_stages():
    """More tiles than CUs with 128 x 128 tiles, and one wave of tiles (the 3-stage pipeline)."""
    for M, N in ((2100, 2080), (512, 2048)):
        x, w, b = _inputs(M, N, 1024, M)
        banner("w6a6 many tiles", M, N)
        mxfp8.set_tile_config(4, 2)
        try:
            _check_pair(x, w, b, 2, 2, "w6a6-many-%d-%d" % (M, N))
        finally:
            mxfp8.set_tile_config(0, 0)


@pytest.mark.parametrize("wfmt,afmt", [(2, 2), (3, 3)])
def test_w6a6_full_size_sampled(wfmt, afmt):
    """The MXFP6 workload's shape (512 x 8192 x 8192, Laplace activations) with FP6 activations."""
    d = synth.make("mxfp6")
    x, w = d["x"], d["w"]
    M, K = x.shape
    N = w.shape[0]
    banner("w6a6 full size", M, N, K, wfmt, afmt)
    layer, wq, ws = _fp6_layer(w, wfmt, None)
    y = mxfp8.linear_fmt(bf16_dev(x), layer.packed, N, wfmt, afmt)
    xq, xs = orc.quantize(x, afmt)
    gq, gs = mxfp8.quantize_act_fmt(bf16_dev(x), afmt)
    assert np.array_equal(host_u8(gs), xs) and np.array_equal(host_u8(gq), orc.fp6_pack(xq))
    g = np.random.default_rng(5)
    r = np.concatenate([g.integers(0, M, 2000), np.full(N, 7), np.arange(M)])
    c = np.concatenate([g.integers(0, N, 2000), np.arange(N), np.full(M, 4095)])
    ref = orc.linear_entries(xq, xs, wq, ws, r, c, wfmt=wfmt, xfmt=afmt)
    ok, rep = tolerance.check(host_bf16_bits(y)[r, c], ref, name="w6a6-full")
    assert ok, rep
