"""GPU parity of the quantizers against the CPU oracle: bit-exact codes and scales.

Activation quantizer (aiter_flydsl page, apply_weights: bf16 -> E4M3 + row-major [M, K/32]
E8M0) on every workload's activations and on an exhaustive sweep of (bf16 value, scale) pairs;
weight quantizer in E4M3 / E2M3 / E3M2 (compressed_tensors_w8a8_mxfp8 and mxfp6 pages).
"""
import numpy as np
import pytest
import torch

import oracle as orc
from mx_block_scaled_amd import mxfp8, synth
from tests.gpu_helpers import banner, bf16_dev, host_u8

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", ["tiny", "decode1", "decode8", "decode32", "outlier", "mxfp6",
                                  "prefill"])
def test_quantize_act_workloads(name):
    d = synth.make(name, with_w=False)
    banner("quantize_act", name, d["x"].shape)
    xq, xs = mxfp8.quantize_act(bf16_dev(d["x"]))
    rq, rs = orc.quantize(d["x"], orc.E4M3)
    assert np.array_equal(host_u8(xs), rs)
    assert np.array_equal(host_u8(xq), rq)


def _sweep_matrix():
    """Blocks [amax setter 2^(E-127), 31 values with |x| <= amax] for every exponent field E,
    covering every bf16 pattern against every scale byte it can meet; rows of 1024."""
    allb = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    mag = allb & 0x7FFF
    blocks = []
    for E in range(0, 255):
        vals = allb[mag <= (E << 7)]
        pad = (-vals.size) % 31
        vals = np.concatenate([vals, np.zeros(pad, np.uint16)]).reshape(-1, 31)
        setter = np.full((vals.shape[0], 1), E << 7, np.uint16)
        blocks.append(np.concatenate([setter, vals], axis=1))
    b = np.concatenate(blocks)
    b = np.concatenate([b, np.zeros(((-b.shape[0]) % 32, 32), np.uint16)])
    return b.reshape(-1, 1024)


def test_quantize_act_exhaustive_sweep():
    x = _sweep_matrix()
    banner("quantize_act sweep", x.shape)
    xq, xs = mxfp8.quantize_act(bf16_dev(x))
    rq, rs = orc.quantize(x, orc.E4M3)
    gs = host_u8(xs)
    assert set(np.unique(rs).tolist()) >= set(range(0, 247))   # every reachable scale byte
    bad = np.argwhere(gs != rs)
    assert bad.size == 0, bad[:5]
    gq = host_u8(xq)
    bad = np.argwhere(gq != rq)
    assert bad.size == 0, [(int(x[i, j]), int(gq[i, j]), int(rq[i, j])) for i, j in bad[:5]]


def test_quantize_act_nonfinite_and_ragged():
    g = np.random.default_rng(3)
    x = synth.bf16_bits(g.standard_normal((7, 96)).astype(np.float32))
    x[2, 5] = 0x7F80            # +Inf
    x[4, 70] = 0xFFC1           # NaN
    x[5, 32:64] = 0x8000        # a block of -0.0
    xq, xs = mxfp8.quantize_act(bf16_dev(x))
    rq, rs = orc.quantize(x, orc.E4M3)
    assert np.array_equal(host_u8(xs), rs) and np.array_equal(host_u8(xq), rq)
    assert rs[2, 0] == 0xFF and rs[4, 2] == 0xFF and rs[5, 1] == 0


def test_quantize_act_leading_dims_and_stride():
    g = np.random.default_rng(4)
    x = synth.bf16_bits(g.standard_normal((2, 3, 160)).astype(np.float32))
    xq, xs = mxfp8.quantize_act(bf16_dev(x))
    rq, rs = orc.quantize(x.reshape(6, 160), orc.E4M3)
    assert np.array_equal(host_u8(xq), rq) and np.array_equal(host_u8(xs), rs)
    # a row stride larger than K through the C ABI
    big = synth.bf16_bits(g.standard_normal((5, 200)).astype(np.float32))
    t = bf16_dev(big)
    q = torch.empty((5, 192), dtype=torch.uint8, device=t.device)
    s = torch.empty((5, 6), dtype=torch.uint8, device=t.device)
    rc = mxfp8.lib().mxfp8_quantize_act(t.data_ptr(), 5, 192, 200, q.data_ptr(), s.data_ptr(), None)
    assert rc == 0
    rq, rs = orc.quantize(np.ascontiguousarray(big[:, :192]), orc.E4M3)
    assert np.array_equal(host_u8(q), rq) and np.array_equal(host_u8(s), rs)


@pytest.mark.parametrize("fmt", [0, 2, 3])
@pytest.mark.parametrize("name", ["tiny", "decode1", "mxfp6"])
def test_quantize_weight(fmt, name):
    d = synth.make(name, M=1)
    banner("quantize_weight", name, fmt, d["w"].shape)
    wq, ws = mxfp8.quantize_weight(bf16_dev(d["w"]), fmt)
    rq, rs = orc.quantize(d["w"], fmt)
    if fmt != 0:
        rq = orc.fp6_pack(rq)
    assert np.array_equal(host_u8(ws), rs)
    assert np.array_equal(host_u8(wq), rq)


@pytest.mark.parametrize("fmt", [0, 2, 3])
def test_quantize_weight_sweep(fmt):
    x = _sweep_matrix()[:2048]
    # FP6 emax differs from E4M3: the sweep still meets every scale the format can reach
    wq, ws = mxfp8.quantize_weight(bf16_dev(x), fmt)
    rq, rs = orc.quantize(x, fmt)
    if fmt != 0:
        rq = orc.fp6_pack(rq)
    assert np.array_equal(host_u8(ws), rs)
    assert np.array_equal(host_u8(wq), rq)


def test_quantize_act_large_ragged_and_strided():
    """A prefill-sized input one row past 4096 (the grid-stride loop's last pass partly past
    the end) and a row stride of 4160 elements through the C ABI (every row start moved);
    non-finite blocks at both ends."""
    g = np.random.default_rng(41)
    M, K, LD = 4097, 4096, 4160
    big = synth.bf16_bits(g.standard_normal((M, LD)).astype(np.float32))
    big[0, 3] = 0x7F80          # +Inf in the first block
    big[M - 1, K - 1] = 0xFFC1  # NaN in the last block
    banner("quantize_act large", M, K, LD)
    x = np.ascontiguousarray(big[:, :K])
    rq, rs = orc.quantize(x, orc.E4M3)
    xq, xs = mxfp8.quantize_act(bf16_dev(x))
    assert np.array_equal(host_u8(xs), rs) and np.array_equal(host_u8(xq), rq)
    t = bf16_dev(big)
    q = torch.empty((M, K), dtype=torch.uint8, device=t.device)
    s = torch.empty((M, K // 32), dtype=torch.uint8, device=t.device)
    rc = mxfp8.lib().mxfp8_quantize_act(t.data_ptr(), M, K, LD, q.data_ptr(), s.data_ptr(), None)
    assert rc == 0
    assert np.array_equal(host_u8(q), rq) and np.array_equal(host_u8(s), rs)
    assert rs[0, 0] == 0xFF and rs[M - 1, K // 32 - 1] == 0xFF
