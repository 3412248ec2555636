"""GPU parity of the tiled GEMM with K split across workgroups (single layers whose 128 x 128
tiles would fill at most 96 of the 256 CUs; the parts on 64 x 128 or 128 x 128 tiles), through
an entry point with a workspace: with bf16 activations from 33 rows on where the split-K decode
kernel is not taken (M > 64, or a workgroup's share of x above 256 KiB there), with MXFP6
activations from 33 rows on).

Each workgroup computes one tile over one K part (whole groups of four K steps) and writes
fp32 sums; a second kernel adds the parts in part order, adds the bias and rounds once.
Checked: the layer against the fp64 oracle to the usual bar for two to eight parts, ragged K
(a last part with fewer steps), ragged M and N, every weight format, MXFP6 activations, with
and without bias; run-to-run determinism; and that batch-invariant mode, which never splits,
still agrees with the oracle at the same shapes.
"""
import numpy as np
import pytest
import torch

import oracle as orc
from mx_block_scaled_amd import mxfp8, synth
from tests import tolerance
from tests.gpu_helpers import DEV, banner, bf16_dev, host_bf16_bits, u8_dev

pytestmark = pytest.mark.gpu

FMTS = {0: "e4m3", 2: "e2m3", 3: "e3m2"}

# (M, N, K): parts = min(8, 256 // tiles, groups of four K steps).  E4M3 weights from 65 rows:
# 64 x 128 ("narrow") tiles while they give two parts or more; else, and for FP6 weights,
# 128 x 128 ("wide") tiles.  Comments: E4M3 / FP6.
SHAPES = [
    (65, 4096, 4096),    # 64 narrow tiles, 4 parts of two groups / 32 wide, 8 parts of one
    (80, 2048, 4096),    # 32 narrow tiles, 8 parts / 16 wide, 8 parts
    (100, 4096, 4480),   # 35 K steps in 9 groups: 64 narrow tiles, 4 parts, the last of 8 + 3
                         # steps / 32 wide, 8 parts, the last of 4 + 3
    (128, 4096, 4096),   # 64 narrow tiles, 4 parts / 32 wide, 8 parts
    (256, 1040, 8192),   # 34 narrow tiles (ragged N), 7 parts / 18 wide, 8 parts of 2 groups
    (300, 4096, 2048),   # 96 wide tiles (192 narrow: one part), 2 parts of 2 groups (ragged M)
    (48, 8192, 8192),    # 64 wide tiles, 4 parts: a workgroup's share of x would exceed 256 KiB
                         # in the split-K decode kernel, so 48 rows take this path
]


def _inputs(M, N, K, seed):
    g = np.random.default_rng(seed)
    x = g.standard_normal((M, K)).astype(np.float32)
    x[:, g.choice(K, max(1, K // 100), replace=False)] *= 30.0
    w = synth.bf16_bits((g.standard_normal((N, K)) * 0.02).astype(np.float32))
    b = synth.bf16_bits((g.standard_normal(N) * 0.05).astype(np.float32))
    return synth.bf16_bits(x), w, b


def _layer(w_bits, fmt, b_bits):
    wq, ws = orc.quantize(w_bits, fmt)
    wstore = wq if fmt == 0 else orc.fp6_pack(wq)
    return mxfp8.MxLinear(u8_dev(wstore), u8_dev(ws), fmt,
                          bias=None if b_bits is None else bf16_dev(b_bits)), wq, ws


@pytest.mark.parametrize("M,N,K", SHAPES)
@pytest.mark.parametrize("fmt", [0, 2, 3])
def test_split_k_matches_oracle(M, N, K, fmt):
    x, w, b = _inputs(M, N, K, M + N + K + fmt)
    use_bias = (M + fmt) % 2 == 0
    layer, wq, ws = _layer(w, fmt, b if use_bias else None)
    banner("tiled split-K", M, N, K, FMTS[fmt], "bias" if use_bias else "no bias")
    y = layer(bf16_dev(x))
    y2 = layer(bf16_dev(x))
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16))      # deterministic
    ref, _, _ = orc.linear_ref(x, wq, ws, fmt, b if use_bias else None)
    ok, rep = tolerance.check(host_bf16_bits(y), ref, name="splitk-%d-%d-%d-%d" % (M, N, K, fmt))
    assert ok, rep


@pytest.mark.parametrize("fmt", [2, 3])
def test_split_k_fp6_activations(fmt):
    """W6A6 (mxfp8_linear_fmt): the same split with FP6 activation rows of 96 bytes per K step,
    from 33 rows on."""
    M, N, K = 33, 2048, 2048
    x, w, b = _inputs(M, N, K, 40 + fmt)
    layer, wq, ws = _layer(w, fmt, b)
    banner("tiled split-K, W6A6", M, N, K, FMTS[fmt])
    wsp = mxfp8.new_workspace(mxfp8.workspace_bytes_fmt(M, N, K, fmt, fmt), DEV)
    y = mxfp8.linear_fmt(bf16_dev(x), layer.packed, N, fmt, fmt, bf16_dev(b), workspace=wsp)
    ref, _, _ = orc.linear_ref(x, wq, ws, fmt, b, xfmt=fmt)
    ok, rep = tolerance.check(host_bf16_bits(y), ref, name="splitk-w6a6-%d" % fmt)
    assert ok, rep


def test_split_k_off_in_batch_invariant_mode():
    """Batch-invariant mode never splits K: the same layer then runs unsplit and still agrees
    with the oracle; its rows equal the rows of a larger call."""
    M, N, K = 128, 4096, 4096
    x, w, b = _inputs(M, N, K, 9)
    layer, wq, ws = _layer(w, 0, b)
    banner("split-K off under batch invariance", M, N, K)
    mxfp8.set_batch_invariant(True)
    try:
        y = layer(bf16_dev(x))
        y_big = layer(bf16_dev(np.concatenate([x, x[:40]])))
    finally:
        mxfp8.set_batch_invariant(False)
    assert torch.equal(y.view(torch.int16), y_big[:M].view(torch.int16))
    ref, _, _ = orc.linear_ref(x, wq, ws, 0, b)
    ok, rep = tolerance.check(host_bf16_bits(y), ref, name="splitk-bi")
    assert ok, rep
