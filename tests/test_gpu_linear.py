"""GPU parity of the MX linear layer against the fp64 CPU oracle.

Acceptance (tests/tolerance.py): per element |y - ref| <= 2 ulp_bf16(|ref|) + 1e-3 rms(ref) and
relative Frobenius error <= 5e-3.  Weights are quantized by the oracle (as the workloads say),
uploaded and prepacked on the GPU; activations go through the GPU quantizer (bf16 entry) or are
pre-quantized by the oracle (pre-quantized entry).  Full-size workloads are checked on sampled
outputs (plus whole rows and columns) that the oracle computes one by one; reduced sizes that
span several tiles and ragged tails are checked element by element.
"""
import numpy as np
import pytest
import torch

import oracle as orc
from mx_block_scaled_amd import mxfp8, synth
from tests import tolerance
from tests.gpu_helpers import DEV, banner, bf16_dev, host_bf16_bits, host_u8, u8_dev

pytestmark = pytest.mark.gpu

FMTS = {0: "e4m3", 2: "e2m3", 3: "e3m2"}


def _layer(w_bits, fmt, bias_bits=None):
    wq, ws = orc.quantize(w_bits, fmt)
    wstore = wq if fmt == 0 else orc.fp6_pack(wq)
    layer = mxfp8.MxLinear(u8_dev(wstore), u8_dev(ws), fmt,
                           bias=None if bias_bits is None else bf16_dev(bias_bits))
    return layer, wq, ws


def _full_check(x_bits, w_bits, fmt, bias_bits=None, name=""):
    layer, wq, ws = _layer(w_bits, fmt, bias_bits)
    y = layer(bf16_dev(x_bits))
    ref, _, _ = orc.linear_ref(x_bits, wq, ws, fmt, bias_bits)
    ok, rep = tolerance.check(host_bf16_bits(y), ref, name=name)
    assert ok, rep
    return y, layer


def _sampled_check(y, xq, xs, wq, ws, fmt, bias_bits, M, N, n_samples=3000, seed=0, name=""):
    g = np.random.default_rng(seed)
    rows = [g.integers(0, M, n_samples), np.array([0, 0, M - 1, M - 1])]
    cols = [g.integers(0, N, n_samples), np.array([0, N - 1, 0, N - 1])]
    # one whole output row and one whole output column
    rows += [np.full(N, g.integers(0, M)), np.arange(M)]
    cols += [np.arange(N), np.full(M, g.integers(0, N))]
    r, c = np.concatenate(rows), np.concatenate(cols)
    bias = None if bias_bits is None else tolerance.bf16_to_f64(bias_bits)
    ref = orc.linear_entries(xq, xs, wq, ws, r, c, wfmt=fmt, bias=bias)
    yb = host_bf16_bits(y)[r, c]
    ok, rep = tolerance.check(yb, ref, name=name)
    assert ok, rep


def test_tiny_full():
    d = synth.make("tiny")
    banner("linear tiny")
    _full_check(d["x"], d["w"], 0, name="tiny")


@pytest.mark.parametrize("M", [1, 8, 32])
def test_decode_full(M):
    d = synth.make("decode%d" % M)
    banner("linear decode", M)
    _full_check(d["x"], d["w"], 0, d["bias"], name="decode%d" % M)


def test_prefill_full_size_sampled():
    d = synth.make("prefill")
    banner("linear prefill 4096x14336x4096")
    layer, wq, ws = _layer(d["w"], 0)
    y = layer(bf16_dev(d["x"]))
    xq, xs = orc.quantize(d["x"], orc.E4M3)
    _sampled_check(y, xq, xs, wq, ws, 0, None, d["M"], d["N"], name="prefill")


def test_outlier_prequant_full_size_sampled():
    d = synth.make("outlier")
    banner("linear_prequant outlier 2048x6144x4096")
    xq, xs = orc.quantize(d["x"], orc.E4M3)          # quantized once, by the oracle
    assert (xs == 0).sum() >= 262                     # the zeroed blocks
    layer, wq, ws = _layer(d["w"], 0)
    y = layer.apply_quantized(u8_dev(xq), u8_dev(xs))
    _sampled_check(y, xq, xs, wq, ws, 0, None, d["M"], d["N"], name="outlier")


def test_outlier_prequant_reduced_full():
    d = synth.make("outlier", N=512)
    xq, xs = orc.quantize(d["x"][:256], orc.E4M3)
    layer, wq, ws = _layer(d["w"], 0)
    y = layer.apply_quantized(u8_dev(xq), u8_dev(xs))
    ref = orc.matmul_nt(orc.dequantize(xq, xs), orc.dequantize(wq, ws))
    ok, rep = tolerance.check(host_bf16_bits(y), ref, name="outlier-256x512")
    assert ok, rep


@pytest.mark.parametrize("fmt", [2, 3])
def test_mxfp6_full_size_sampled(fmt):
    d = synth.make("mxfp6")
    banner("linear mxfp6", FMTS[fmt], "512x8192x8192")
    layer, wq, ws = _layer(d["w"], fmt)
    y = layer(bf16_dev(d["x"]))
    xq, xs = orc.quantize(d["x"], orc.E4M3)
    _sampled_check(y, xq, xs, wq, ws, fmt, None, d["M"], d["N"], name="mxfp6-%d" % fmt)


@pytest.mark.parametrize("fmt", [2, 3])
def test_mxfp6_reduced_full(fmt):
    d = synth.make("mxfp6", M=64, N=512)
    _full_check(d["x"], d["w"], fmt, name="mxfp6-small-%d" % fmt)


RAGGED = [(1, 16, 32), (3, 48, 96), (17, 272, 160), (33, 64, 544), (100, 80, 1056), (65, 16, 4096)]


@pytest.mark.parametrize("fmt", [0, 2, 3])
@pytest.mark.parametrize("M,N,K", RAGGED)
def test_ragged_shapes(M, N, K, fmt):
    g = np.random.default_rng(M * 7 + N + K)
    x = synth.bf16_bits(g.standard_normal((M, K)).astype(np.float32))
    w = synth.bf16_bits((g.standard_normal((N, K)) * 0.05).astype(np.float32))
    b = synth.bf16_bits((g.standard_normal(N) * 0.1).astype(np.float32))
    banner("linear ragged", M, N, K, FMTS[fmt])
    _full_check(x, w, fmt, b, name="ragged-%d-%d-%d-%d" % (M, N, K, fmt))


def test_gpu_weight_quantizer_path_matches_oracle_path():
    d = synth.make("decode8", N=1024)
    wq, ws = mxfp8.quantize_weight(bf16_dev(d["w"]), 0)
    p1 = mxfp8.prepack_weight(wq, ws, 0)
    layer, _, _ = _layer(d["w"], 0)
    x = bf16_dev(d["x"])
    y1 = mxfp8.linear(x, p1, d["N"], 0)
    y2 = layer(x)
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))


def test_zero_rows_and_bias_none():
    d = synth.make("tiny")
    layer, _, _ = _layer(d["w"], 0)
    y = layer(bf16_dev(d["x"][:0]))
    assert y.shape == (0, 256)


def test_deterministic_and_no_out_of_bounds_writes():
    d = synth.make("decode32", N=512)
    layer, wq, ws = _layer(d["w"], 0, d["bias"][:512])
    x = bf16_dev(d["x"])
    M, N = 32, 512
    guard = 4096
    big = torch.full((2 * guard + M * N,), -7777.0, dtype=torch.bfloat16, device=DEV)
    out = big[guard:guard + M * N].view(M, N)
    y1 = mxfp8.linear(x, layer.packed, N, 0, layer.bias, out=out).clone()
    y2 = mxfp8.linear(x, layer.packed, N, 0, layer.bias)
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
    assert bool((big[:guard] == -7777.0).all()) and bool((big[guard + M * N:] == -7777.0).all())


def test_leading_dims():
    d = synth.make("tiny")
    layer, wq, ws = _layer(d["w"], 0)
    x3 = d["x"].reshape(2, 8, 512)
    y = layer(bf16_dev(x3))
    assert y.shape == (2, 8, 256)
    ref, _, _ = orc.linear_ref(d["x"], wq, ws)
    ok, rep = tolerance.check(host_bf16_bits(y).reshape(16, 256), ref)
    assert ok, rep


def test_prequant_rejects_wrong_scale_shape():
    d = synth.make("tiny")
    layer, _, _ = _layer(d["w"], 0)
    xq, xs = mxfp8.quantize_act(bf16_dev(d["x"]))
    with pytest.raises(ValueError):
        layer.apply_quantized(xq, xs[:, :8].contiguous())


TILES = [(8, 4), (7, 4), (6, 4), (4, 4), (4, 2)]


@pytest.mark.parametrize("fmt", [0, 2, 3])
@pytest.mark.parametrize("fn,fm", TILES)
def test_tiled_kernel_every_tile(fn, fm, fmt):
    """Each compiled tile of the LDS-tiled kernel, on a shape with ragged M and N tails and a K
    that is not a multiple of 512 (remainder K steps), against the oracle element by element."""
    g = np.random.default_rng(fn * 10 + fm + fmt)
    M, N, K = 300, 592, 640
    x = synth.bf16_bits(g.standard_normal((M, K)).astype(np.float32))
    w = synth.bf16_bits((g.standard_normal((N, K)) * 0.02).astype(np.float32))
    b = synth.bf16_bits((g.standard_normal(N) * 0.01).astype(np.float32))
    banner("tiled", fn, fm, FMTS[fmt], M, N, K)
    mxfp8.set_tile_config(fn, fm)
    try:
        _full_check(x, w, fmt, b, name="tile-%d-%d-%d" % (fn, fm, fmt))
    finally:
        mxfp8.set_tile_config(0, 0)


# The four-wave kernel (32x32x64 scaled MFMAs, accumulators in the AGPRs; E4M3 weights,
# K % 512 == 0), each of its tiles (forced: 256 x 256 and 256 x 128 on a 2 x 2 wave grid,
# 224 x 256 and 192 x 256 on a 1 x 4 wave grid): ragged M and N tails, one tile smaller than
# the workgroup tile, several tiles over the XCD ranges, with and without bias.
W4_SHAPES = [(300, 592, 1024), (96, 256, 512), (520, 1040, 2048), (1024, 2048, 4096), (257, 272, 1536)]


@pytest.mark.parametrize("tile", [(16, 16), (17, 16), (18, 16), (19, 16)])
@pytest.mark.parametrize("M,N,K", W4_SHAPES)
def test_four_wave_kernel(M, N, K, tile):
    g = np.random.default_rng(M + N + K)
    xf = g.standard_normal((M, K)).astype(np.float32)
    xf[:, g.choice(K, 5, replace=False)] *= 40.0                     # outlier channels
    x = synth.bf16_bits(xf)
    w = synth.bf16_bits((g.standard_normal((N, K)) * 0.02).astype(np.float32))
    b = synth.bf16_bits((g.standard_normal(N) * 0.01).astype(np.float32)) if M % 2 == 0 else None
    banner("four-wave tile", tile, M, N, K, "bias" if b is not None else "no bias")
    mxfp8.set_tile_config(*tile)
    try:
        _full_check(x, w, 0, b, name="w4-%d-%d-%d-%d" % (M, N, K, tile[0]))
    finally:
        mxfp8.set_tile_config(0, 0)


# The ping-pong kernel (two groups of four waves taking turns between MFMAs and operand reads;
# E4M3 weights and activations, K % 512 == 0), each of its tiles (forced: 224 x 256, 192 x 256
# and 128 x 256): against the oracle, and bit-equal to the all-waves-in-step kernel of the same
# tile, which issues the same MFMAs in the same order per accumulator.
@pytest.mark.parametrize("tile", [(7, 36), (6, 36), (4, 36)])
@pytest.mark.parametrize("M,N,K", W4_SHAPES)
def test_ping_pong_kernel(M, N, K, tile):
    g = np.random.default_rng(M * 3 + N + K + tile[0])
    xf = g.standard_normal((M, K)).astype(np.float32)
    xf[:, g.choice(K, 5, replace=False)] *= 40.0                     # outlier channels
    x = synth.bf16_bits(xf)
    w = synth.bf16_bits((g.standard_normal((N, K)) * 0.02).astype(np.float32))
    b = synth.bf16_bits((g.standard_normal(N) * 0.01).astype(np.float32)) if M % 2 == 0 else None
    banner("ping-pong tile", tile, M, N, K, "bias" if b is not None else "no bias")
    mxfp8.set_tile_config(*tile)
    try:
        y, layer = _full_check(x, w, 0, b, name="pp-%d-%d-%d-%d" % (M, N, K, tile[0]))
        mxfp8.set_tile_config(tile[0], 4)
        y2 = layer(bf16_dev(x))
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), y2.view(torch.int16))
    finally:
        mxfp8.set_tile_config(0, 0)


# Small-M (decode) paths, one launch with the activation quantizer fused in.  bf16 entry up to
# 16 rows with K <= 8192 and up to 24 with K <= 4096: the role-split kernel (quantizer waves
# beside MFMA waves); other rows up to 64 (N % 64 == 0): the split-K decode kernel.  The
# pre-quantized entry (M <= 32) runs the small-M kernel with K split over its 8 waves.  K values
# give idle waves (K = 384), partial 4-step groups (K = 640, 1152, 3968) and a wave with two
# groups, the second partial (K = 4224).
SMALL = [(1, 16, 128), (5, 48, 384), (16, 272, 640), (15, 80, 4224), (17, 64, 512),
         (31, 80, 3968), (32, 32, 1152), (24, 48, 4096), (32, 4096, 4096)]


def _small_inputs(M, N, K, seed):
    g = np.random.default_rng(seed)
    x = g.standard_normal((M, K)).astype(np.float32)
    x[:, g.choice(K, max(1, K // 100), replace=False)] *= 100.0      # outlier channels
    x = x.reshape(M, K // 32, 32)
    x[g.integers(0, M, 3), g.integers(0, K // 32, 3)] = 0.0           # all-zero blocks
    x = synth.bf16_bits(x.reshape(M, K))
    w = synth.bf16_bits((g.standard_normal((N, K)) * 0.05).astype(np.float32))
    b = synth.bf16_bits((g.standard_normal(N) * 0.1).astype(np.float32))
    return x, w, b


@pytest.mark.parametrize("fmt", [0, 2, 3])
@pytest.mark.parametrize("M,N,K", SMALL)
def test_small_m_fused(M, N, K, fmt):
    x, w, b = _small_inputs(M, N, K, M * 131 + N + K + fmt)
    banner("linear small-M", M, N, K, FMTS[fmt])
    y, layer = _full_check(x, w, fmt, b, name="small-%d-%d-%d-%d" % (M, N, K, fmt))
    xq, xs = orc.quantize(x, orc.E4M3)
    y2 = layer.apply_quantized(u8_dev(xq), u8_dev(xs))
    if _entries_differ(M, N, K):
        # the bf16 entry runs another kernel here and adds in another order: both entries
        # against the oracle
        ref, _, _ = orc.linear_ref(x, *orc.quantize(w, fmt), fmt, b)
        ok, rep = tolerance.check(host_bf16_bits(y2), ref, name="small-prequant")
        assert ok, rep
    else:
        # the pre-quantized entry runs the same kernel with the same summation order, so
        # feeding it the oracle's quantization of x must reproduce the bf16 entry's result bit
        # for bit
        assert torch.equal(y.view(torch.int16), y2.view(torch.int16))


def _row_split(M, N, K):
    """shapes on which the role-split kernel splits the rows into tiles: two of up to 16 rows
    (two weight fragments per workgroup) or three or four (four fragments)"""
    return K % 128 == 0 and K <= 4096 and ((17 <= M <= 32 and N % 32 == 0)
                                           or (33 <= M <= 64 and N % 64 == 0))


def _role_split(M, N, K):
    """shapes on which mxfp8_linear runs the role-split small-M kernel"""
    return K % 128 == 0 and ((1 <= M <= 16 and K <= 8192) or (1 <= M <= 24 and K <= 4096)
                             or _row_split(M, N, K))


def _entries_differ(M, N, K):
    """shapes on which mxfp8_linear (bf16 entry) runs another kernel than the pre-quantized
    entry's small-M kernel: the role-split kernel or the split-K decode kernel"""
    return _role_split(M, N, K) or (16 <= M <= 64 and N % 64 == 0 and K % 128 == 0)


# The role-split kernel on each of its row counts (1, 2, 4, 8, 12 and 16 rows with one tile, 24
# with two 16-row activation tiles, two row tiles of 9 to 16 rows, three or four of 11 to 16),
# both code-image sizes (K <= 4096, K <= 8192), partial last K groups, quantizer and weight
# waves with no K group, columns that are not a multiple of 64, and a full decode width.  Row
# tiles: column-group counts that are a multiple of 8 (row tiles of a group on one XCD) and
# not (1, 3, 33), row tiles of unequal rows.  From 4 rows, grids of at least 512 workgroups take
# two or four fragments per workgroup (N = 8192: two; N = 16384, and 31 rows in two tiles at
# N = 8192: four); 1 and 3 rows at N = 16384 keep one.
RS = [(1, 64, 128), (2, 80, 8192), (3, 48, 640), (7, 272, 4224), (11, 96, 1152),
      (12, 64, 3968), (13, 4096, 4096), (16, 160, 8192), (21, 112, 640), (24, 48, 2048),
      (17, 64, 4096), (18, 32, 128), (25, 96, 640), (29, 256, 3968), (19, 1056, 1152),
      (32, 4096, 4096), (23, 512, 4096), (31, 8192, 2048),
      (33, 64, 4096), (40, 192, 640), (48, 512, 3968), (49, 2112, 1152), (64, 4096, 4096),
      (57, 1024, 128), (36, 8192, 2048),
      (8, 8192, 1024), (4, 16384, 512), (16, 16384, 4096), (1, 16384, 128), (3, 16384, 256)]


@pytest.mark.parametrize("fmt", [0, 2, 3])
@pytest.mark.parametrize("M,N,K", RS)
def test_small_m_role_split(M, N, K, fmt):
    assert _role_split(M, N, K)
    x, w, b = _small_inputs(M, N, K, M * 17 + N + K + fmt)
    banner("linear small-M role split", M, N, K, FMTS[fmt])
    _full_check(x, w, fmt, b if (M + K) % 3 else None, name="rs-%d-%d-%d-%d" % (M, N, K, fmt))


@pytest.mark.parametrize("M,N,K", [(9, 128, 1024), (22, 128, 2560), (22, 112, 2560)])
def test_small_m_role_split_inf_block(M, N, K):
    """A block holding Inf: its row of the output is NaN, as in the oracle; the other rows are
    unaffected (one row tile; two row tiles; two 16-row activation tiles in one row tile)."""
    x, w, b = _small_inputs(M, N, K, M + K)
    x[3, 100] = 0x7F80                      # +Inf in row 3
    layer, wq, ws = _layer(w, 0, b)
    banner("linear small-M role split, Inf block", M, N, K)
    y = host_bf16_bits(layer(bf16_dev(x)))
    ref, _, _ = orc.linear_ref(x, wq, ws, 0, b)
    assert np.isnan(tolerance.bf16_to_f64(y)[3]).all() and np.isnan(ref[3]).all()
    keep = np.arange(M) != 3
    ok, rep = tolerance.check(y[keep], ref[keep], name="rs-inf")
    assert ok, rep


@pytest.mark.parametrize("M", [1, 8, 32])
def test_decode_prequant_matches_fused(M):
    d = synth.make("decode%d" % M)
    layer, wq, ws = _layer(d["w"], 0, d["bias"])
    y = layer(bf16_dev(d["x"]))
    xq, xs = orc.quantize(d["x"], orc.E4M3)
    y2 = layer.apply_quantized(u8_dev(xq), u8_dev(xs))
    if _entries_differ(M, 4096, 4096):   # different kernels: each against the oracle
        ref, _, _ = orc.linear_ref(d["x"], wq, ws, 0, d["bias"])
        for yy, nm in ((y, "bf16 entry"), (y2, "pre-quantized entry")):
            ok, rep = tolerance.check(host_bf16_bits(yy), ref, name=nm)
            assert ok, rep
    else:
        assert torch.equal(y.view(torch.int16), y2.view(torch.int16))


@pytest.mark.parametrize("fmt", [0, 2])
@pytest.mark.parametrize("K", [640, 1024])
def test_tiled_kernel_many_tiles(K, fmt):
    """More tiles than CUs (289 tiles of 128 x 128), ragged M and N, K with and without whole
    groups of four K steps."""
    g = np.random.default_rng(K + fmt)
    M, N = 2100, 2080
    x = synth.bf16_bits(g.standard_normal((M, K)).astype(np.float32))
    w = synth.bf16_bits((g.standard_normal((N, K)) * 0.02).astype(np.float32))
    b = synth.bf16_bits((g.standard_normal(N) * 0.01).astype(np.float32))
    banner("tiled many tiles", M, N, K, FMTS[fmt])
    mxfp8.set_tile_config(4, 2)
    try:
        _full_check(x, w, fmt, b, name="many-tiles-%d-%d" % (K, fmt))
    finally:
        mxfp8.set_tile_config(0, 0)


@pytest.mark.parametrize("fmt", [0, 2])
@pytest.mark.parametrize("K,N", [(512, 272), (4224, 272), (544, 272), (512, 256), (4096, 1024)])
def test_batch_invariant_mode(K, N, fmt):
    """Batch-invariant mode: the first rows of a 300-row call (tiled kernel; K % 128 != 0:
    generic kernel) are bit-identical to the same rows called alone at M = 1, 8, 16, 17, 31,
    32, 33, 48 and 64, on both entries, with E4M3 and E2M3 weights; the mode's result is
    checked against the oracle.  The rows called alone run on the role-split kernel with its
    weight waves extending one accumulator chain in K order (the bf16 entry: one row tile up to
    16 rows, K <= 8192; two 16-row activation tiles in one row tile up to 24 rows where
    N % 32 != 0; row tiles from 17 rows where N % 32 == 0 (up to 32 rows) or N % 64 == 0,
    K <= 4096, with two or four weight fragments per workgroup) and on the generic or tiled
    kernel elsewhere (the pre-quantized entry, K % 128 != 0, 31 rows and more at N = 272)."""
    g = np.random.default_rng(K + fmt + N)
    M = 300
    xf = g.standard_normal((M, K)).astype(np.float32)
    xf[:, g.choice(K, 4, replace=False)] *= 50.0                     # outlier channels
    x = synth.bf16_bits(xf)
    w = synth.bf16_bits((g.standard_normal((N, K)) * 0.03).astype(np.float32))
    b = synth.bf16_bits((g.standard_normal(N) * 0.1).astype(np.float32))
    layer, wq, ws = _layer(w, fmt, b)
    xd = bf16_dev(x)
    xq, xs = mxfp8.quantize_act(xd)
    banner("batch invariant", K)
    mxfp8.set_batch_invariant(True)
    try:
        y_all = layer(xd)
        yq_all = layer.apply_quantized(xq, xs)
        assert torch.equal(y_all.view(torch.int16), yq_all.view(torch.int16))
        for m in (1, 8, 16, 17, 31, 32, 33, 48, 64):
            y = layer(xd[:m].contiguous())
            yq = layer.apply_quantized(xq[:m].contiguous(), xs[:m].contiguous())
            assert torch.equal(y.view(torch.int16), y_all[:m].view(torch.int16)), m
            assert torch.equal(yq.view(torch.int16), y_all[:m].view(torch.int16)), m
    finally:
        mxfp8.set_batch_invariant(False)
    ref, _, _ = orc.linear_ref(x, wq, ws, fmt, b)
    ok, rep = tolerance.check(host_bf16_bits(y_all), ref, name="batch-invariant-%d-%d-%d" % (K, N, fmt))
    assert ok, rep


def _tiled_split_k(M, N, K):
    """Whether a single mxfp8_linear call of this layer splits K across workgroups in the tiled
    GEMM (M > 32, at most 96 output tiles of 128 x 128, at least two groups of four K steps)."""
    tiles = -(-N // 128) * -(-M // 128)
    return M > 32 and K % 128 == 0 and N >= 128 and tiles <= 96 and (K // 128 + 3) // 4 >= 2


@pytest.mark.parametrize("M,N,K", [(5, 48, 512), (24, 64, 1024), (9, 8192, 512), (20, 4096, 1024),
                                   (100, 272, 512),
                                   (300, 592, 640), (40, 160, 544)])
def test_batched(M, N, K):
    """Batched layer (bmm_batch_size): every batch equals a separate call bit for bit (same
    kernels: fused small-M, quantizer + small-M, tiled, generic), and batch 1 matches the
    oracle; per-batch bias and the pre-quantized batched entry included.  A layer that a
    separate call splits along K (300 x 592 x 640) runs unsplit in the batched call, as in the
    pre-quantized entry, and is compared with that."""
    Bn = 3
    g = np.random.default_rng(M + N + K)
    xs_ = [synth.bf16_bits(g.standard_normal((M, K)).astype(np.float32)) for _ in range(Bn)]
    ws_ = [synth.bf16_bits((g.standard_normal((N, K)) * 0.03).astype(np.float32)) for _ in range(Bn)]
    bs_ = [synth.bf16_bits((g.standard_normal(N) * 0.1).astype(np.float32)) for _ in range(Bn)]
    banner("batched", Bn, M, N, K)
    layers = [_layer(ws_[b], 0, bs_[b]) for b in range(Bn)]
    packed = torch.cat([l[0].packed for l in layers])
    bias = torch.stack([bf16_dev(bb) for bb in bs_])
    x = torch.stack([bf16_dev(xx) for xx in xs_])
    y = mxfp8.linear_batched(x, packed, N, 0, bias)
    xq, xsc = mxfp8.quantize_act(x.reshape(Bn * M, K))
    yq = mxfp8.linear_prequant_batched(xq.view(Bn, M, K), xsc.view(Bn, M, K // 32), packed, N, 0,
                                       bias)
    split = _tiled_split_k(M, N, K)
    for b in range(Bn):
        y1 = layers[b][0](x[b])
        y1q = layers[b][0].apply_quantized(xq.view(Bn, M, K)[b].contiguous(),
                                           xsc.view(Bn, M, K // 32)[b].contiguous())
        assert torch.equal(y[b].view(torch.int16), (y1q if split else y1).view(torch.int16)), b
        assert torch.equal(yq[b].view(torch.int16), y1q.view(torch.int16)), b
    ref, _, _ = orc.linear_ref(xs_[1], layers[1][1], layers[1][2], 0, bs_[1])
    ok, rep = tolerance.check(host_bf16_bits(y[1]), ref, name="batched-%d-%d-%d" % (M, N, K))
    assert ok, rep
    if split:   # the separate call's split sum meets the same bar
        ok, rep = tolerance.check(host_bf16_bits(layers[1][0](x[1])), ref, name="split-%d" % M)
        assert ok, rep


def test_batch_invariant_mode_per_thread():
    """The per-thread mode, seen through the workspace: at M = 8, K = 8320 the normal path
    (small-M kernel, quantizer fused in) never touches the workspace, while batch-invariant mode
    quantizes into it first and then runs the generic kernel.  A thread with mode on gets the
    quantized rows in its workspace and the 300-row call's bits while the process-wide mode is
    off; a thread with mode off leaves its workspace alone while the process-wide mode is on;
    a thread back at -1 follows the process-wide mode."""
    import threading
    g = np.random.default_rng(3)
    M, N, K, m = 300, 256, 8320, 8
    x = bf16_dev(synth.bf16_bits(g.standard_normal((M, K)).astype(np.float32)))
    w = synth.bf16_bits((g.standard_normal((N, K)) * 0.03).astype(np.float32))
    layer, _, _ = _layer(w, 0, None)
    banner("batch-invariant mode per thread", N, K)
    y_all = layer(x)                                  # tiled: the same bits in either mode
    xm = x[:m].contiguous()
    normal = layer(xm)
    xq, _ = mxfp8.quantize_act(xm)
    need = mxfp8.workspace_bytes(m, N, K)
    torch.cuda.synchronize()
    out, err = {}, []

    def run(name, mode):
        try:
            mxfp8.set_batch_invariant_thread(mode)
            ws = mxfp8.new_workspace(need, DEV)
            ws[65536:].fill_(0xA5)
            y = mxfp8.linear(xm, layer.packed, N, 0, None, workspace=ws)
            torch.cuda.synchronize()
            out[name] = (y, bool(torch.equal(ws[65536:65536 + m * K], xq.view(-1))),
                         bool((ws[65536:] == 0xA5).all()))
        except Exception as e:   # reported by the main thread
            err.append(e)
        finally:
            mxfp8.set_batch_invariant_thread(None)

    try:
        for proc_mode in (False, True):
            mxfp8.set_batch_invariant(proc_mode)
            ts = [threading.Thread(target=run, args=("on", True)),
                  threading.Thread(target=run, args=("off", False)),
                  threading.Thread(target=run, args=("follow", None))]
            for t in ts:
                t.start()
            for t in ts:
                t.join()
            assert not err, err
            for name, on in (("on", True), ("off", False), ("follow", proc_mode)):
                y, quantized_into_ws, untouched = out[name]
                assert quantized_into_ws == on and untouched == (not on), (proc_mode, name)
                want = y_all[:m] if on else normal
                assert torch.equal(y.view(torch.int16), want.view(torch.int16)), (proc_mode, name)
    finally:
        mxfp8.set_batch_invariant(False)


@pytest.mark.parametrize("M", [8, 24, 40])
def test_batched_batch_invariant(M):
    """The batched layer in batch-invariant mode (the role-split kernel's in-order chain, one,
    two and three row tiles; the batch's grid takes four fragments per workgroup from 24 rows):
    every batch equals its rows of a 300-row call of the same layer, bit for bit."""
    Bn, N, K = 3, 256, 1024
    g = np.random.default_rng(M + 5)
    xs_ = [synth.bf16_bits(g.standard_normal((300, K)).astype(np.float32)) for _ in range(Bn)]
    ws_ = [synth.bf16_bits((g.standard_normal((N, K)) * 0.03).astype(np.float32)) for _ in range(Bn)]
    bs_ = [synth.bf16_bits((g.standard_normal(N) * 0.1).astype(np.float32)) for _ in range(Bn)]
    banner("batched, batch-invariant mode", Bn, M, N, K)
    layers = [_layer(ws_[b], 0, bs_[b]) for b in range(Bn)]
    packed = torch.cat([l[0].packed for l in layers])
    bias = torch.stack([bf16_dev(bb) for bb in bs_])
    x_all = [bf16_dev(xx) for xx in xs_]
    x = torch.stack([xx[:M] for xx in x_all])
    mxfp8.set_batch_invariant(True)
    try:
        y = mxfp8.linear_batched(x, packed, N, 0, bias)
        for b in range(Bn):
            y_all = layers[b][0](x_all[b])
            assert torch.equal(y[b].view(torch.int16), y_all[:M].view(torch.int16)), b
    finally:
        mxfp8.set_batch_invariant(False)


@pytest.mark.parametrize("tile", [(7, 36), (6, 36), (7, 4)])
def test_batched_forced_tiles(tile):
    """The batched layer on the ping-pong kernel's tiles (grid y = batch) and on the
    all-waves-in-step kernel's: every batch equals a separate call bit for bit."""
    Bn, M, N, K = 3, 300, 592, 1024
    g = np.random.default_rng(tile[0] * 100 + tile[1])
    xs_ = [synth.bf16_bits(g.standard_normal((M, K)).astype(np.float32)) for _ in range(Bn)]
    ws_ = [synth.bf16_bits((g.standard_normal((N, K)) * 0.03).astype(np.float32)) for _ in range(Bn)]
    bs_ = [synth.bf16_bits((g.standard_normal(N) * 0.1).astype(np.float32)) for _ in range(Bn)]
    banner("batched forced tile", tile, Bn, M, N, K)
    layers = [_layer(ws_[b], 0, bs_[b]) for b in range(Bn)]
    packed = torch.cat([l[0].packed for l in layers])
    bias = torch.stack([bf16_dev(bb) for bb in bs_])
    x = torch.stack([bf16_dev(xx) for xx in xs_])
    mxfp8.set_tile_config(*tile)
    try:
        y = mxfp8.linear_batched(x, packed, N, 0, bias)
        for b in range(Bn):
            y1 = layers[b][0](x[b])
            torch.cuda.synchronize()
            assert torch.equal(y[b].view(torch.int16), y1.view(torch.int16)), b
    finally:
        mxfp8.set_tile_config(0, 0)
    ref, _, _ = orc.linear_ref(xs_[2], layers[2][1], layers[2][2], 0, bs_[2])
    ok, rep = tolerance.check(host_bf16_bits(y[2]), ref, name="batched-tile-%d-%d" % tile)
    assert ok, rep


@pytest.mark.parametrize("M", [5, 24, 300])
def test_bias_at_odd_offset(M):
    """A bias that starts 2 bytes past an 8-byte boundary (a slice of a larger tensor): the
    small-M kernels' 8-byte bias load falls back to element loads."""
    g = np.random.default_rng(M)
    N, K = 144, 512
    x = synth.bf16_bits(g.standard_normal((M, K)).astype(np.float32))
    w = synth.bf16_bits((g.standard_normal((N, K)) * 0.02).astype(np.float32))
    bfull = synth.bf16_bits((g.standard_normal(N + 1) * 0.1).astype(np.float32))
    wq, ws = orc.quantize(w)
    layer = mxfp8.MxLinear(u8_dev(wq), u8_dev(ws), 0)
    bias_t = bf16_dev(bfull)[1:]
    assert bias_t.data_ptr() % 8 == 2
    banner("bias at odd offset", M)
    y = mxfp8.linear(bf16_dev(x), layer.packed, N, 0, bias_t)
    ref, xq, xs = orc.linear_ref(x, wq, ws, 0, bfull[1:])
    ok, rep = tolerance.check(host_bf16_bits(y), ref, name="bias-odd-%d" % M)
    assert ok, rep
    y2 = mxfp8.linear_prequant(u8_dev(xq), u8_dev(xs), layer.packed, N, 0, bias_t)
    ok, rep = tolerance.check(host_bf16_bits(y2), ref, name="bias-odd-prequant-%d" % M)
    assert ok, rep


# one shape per mxfp8_linear path: small-M fused (one, two and four row tiles), split-K decode
# (2 and 4 activation tiles), split-K tiled GEMM with its reduction launch (8 and 2 K parts), tiled
# GEMM, generic GEMM (K % 128 != 0)
PATH_SHAPES = [(8, 1024, 2048), (32, 1024, 4096), (64, 1024, 4096), (32, 1024, 8192),
               (64, 2048, 8192), (100, 2048, 4096), (300, 4096, 4096), (300, 8192, 1024),
               (40, 512, 1120)]


@pytest.mark.parametrize("M,N,K", PATH_SHAPES)
def test_workspace_and_output_bounds_every_path(M, N, K):
    """Each path writes only y [M, N] and the first workspace_bytes(M, N, K) bytes of its
    workspace: guard bands around both keep their fill, the counters are left at zero, and a
    second call into the same buffers repeats the first result bit for bit."""
    g = np.random.default_rng(M + N + K)
    x = bf16_dev(synth.bf16_bits(g.standard_normal((M, K)).astype(np.float32)))
    wb = synth.bf16_bits((g.standard_normal((N, K)) * 0.02).astype(np.float32))
    b = bf16_dev(synth.bf16_bits((g.standard_normal(N) * 0.05).astype(np.float32)))
    wq, wsc = orc.quantize(wb, 0)
    pk = mxfp8.prepack_weight(u8_dev(wq), u8_dev(wsc), 0)
    guard = 8192
    need = mxfp8.workspace_bytes(M, N, K)
    wbig = torch.full((need + 2 * guard,), 0xA5, dtype=torch.uint8, device=DEV)
    wbig[guard:guard + 65536].zero_()                         # counters start at zero
    ws = wbig[guard:guard + need]
    ybig = torch.full((M * N + 2 * guard,), -7777.0, dtype=torch.bfloat16, device=DEV)
    y = ybig[guard:guard + M * N].view(M, N)
    banner("bounds of every path", M, N, K, "workspace", need)
    mxfp8.linear(x, pk, N, 0, b, out=y, workspace=ws)
    y1 = y.clone()
    mxfp8.linear(x, pk, N, 0, b, out=y, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y1.view(torch.int16))
    assert bool((wbig[:guard] == 0xA5).all()) and bool((wbig[guard + need:] == 0xA5).all())
    assert int(ws[:65536].count_nonzero()) == 0
    assert bool((ybig[:guard] == -7777.0).all()) and bool((ybig[guard + M * N:] == -7777.0).all())
    ref, _, _ = orc.linear_ref(host_bf16_bits(x), wq, wsc, 0, host_bf16_bits(b))
    ok, rep = tolerance.check(host_bf16_bits(y), ref, name="bounds-%d-%d-%d" % (M, N, K))
    assert ok, rep


def test_role_split_forms_graph_replay():
    """The role-split kernel's forms captured in one HIP graph (one row tile; two row tiles with
    two fragments; four row tiles with four; a batched call that widens to four fragments;
    batch-invariant mode's in-order chain): every replay, with eager work between replays,
    equals the eager results bit for bit."""
    g = np.random.default_rng(31)
    N, K = 4096, 2048
    wb = synth.bf16_bits((g.standard_normal((N, K)) * 0.02).astype(np.float32))
    wq, wsc = orc.quantize(wb, 0)
    pk = mxfp8.prepack_weight(u8_dev(wq), u8_dev(wsc), 0)
    bias = bf16_dev(synth.bf16_bits((g.standard_normal(N) * 0.1).astype(np.float32)))
    Ms = (8, 32, 64)
    xs = [bf16_dev(synth.bf16_bits(g.standard_normal((M, K)).astype(np.float32))) for M in Ms]
    Bn = 4
    pkb = torch.cat([pk] * Bn)
    xb = bf16_dev(synth.bf16_bits(g.standard_normal((Bn, 12, K)).astype(np.float32)))
    biasb = bias.unsqueeze(0).repeat(Bn, 1).contiguous()
    ys = [torch.empty((x.shape[0], N), dtype=torch.bfloat16, device=DEV) for x in xs]
    yb = torch.empty((Bn, 12, N), dtype=torch.bfloat16, device=DEV)
    ybi = torch.empty((24, N), dtype=torch.bfloat16, device=DEV)
    # explicit workspaces (none of these kernels uses one; the sizes cover every entry)
    ws = mxfp8.new_workspace(max(mxfp8.workspace_bytes(M, N, K) for M in Ms), DEV)
    wsb = mxfp8.new_workspace(mxfp8.workspace_bytes(Bn * 12, N, K), DEV)
    banner("role-split forms, graph replay")

    def calls():
        for x, y in zip(xs, ys):
            mxfp8.linear(x, pk, N, 0, bias, out=y, workspace=ws)
        mxfp8.linear_batched(xb, pkb, N, 0, biasb, out=yb, workspace=wsb)
        mxfp8.set_batch_invariant_thread(True)
        try:
            mxfp8.linear(xs[2][:24].contiguous(), pk, N, 0, bias, out=ybi, workspace=ws)
        finally:
            mxfp8.set_batch_invariant_thread(None)

    calls()
    torch.cuda.synchronize()
    eager = [y.clone() for y in ys] + [yb.clone(), ybi.clone()]
    s = torch.cuda.Stream(DEV)
    s.wait_stream(torch.cuda.current_stream(DEV))
    x24 = xs[2][:24].contiguous()
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gr, stream=s):
        for x, y in zip(xs, ys):
            mxfp8.linear(x, pk, N, 0, bias, out=y, workspace=ws)
        mxfp8.linear_batched(xb, pkb, N, 0, biasb, out=yb, workspace=wsb)
        mxfp8.set_batch_invariant_thread(True)
        try:
            mxfp8.linear(x24, pk, N, 0, bias, out=ybi, workspace=ws)
        finally:
            mxfp8.set_batch_invariant_thread(None)
    for rep in range(3):
        for y in ys + [yb, ybi]:
            y.zero_()
        gr.replay()
        torch.cuda.synchronize()
        for y, e in zip(ys + [yb, ybi], eager):
            assert torch.equal(y.view(torch.int16), e.view(torch.int16)), rep
        calls()                                    # eager work between replays
        torch.cuda.synchronize()


@pytest.mark.parametrize("M", [1, 8, 32])
def test_batched_decode_bench_config(M):
    """The bench's batched decode configuration: eight 4096 x 4096 layers (own activations,
    weights, bias) in one call, M = 1 (one fragment per workgroup), 8 (four fragments) and 32
    (four fragments, two row tiles).  Every batch equals a separate call of its layer bit for
    bit; batches 0 and 7 are checked against the oracle in full."""
    Bn, N, K = 8, 4096, 4096
    g = np.random.default_rng(M + 808)
    xs_ = [synth.bf16_bits(g.standard_normal((M, K)).astype(np.float32)) for _ in range(Bn)]
    ws_ = [synth.bf16_bits((g.standard_normal((N, K)) * 0.02).astype(np.float32)) for _ in range(Bn)]
    bs_ = [synth.bf16_bits((g.standard_normal(N) * 0.01).astype(np.float32)) for _ in range(Bn)]
    banner("batched decode, bench configuration", Bn, M, N, K)
    layers = [_layer(ws_[b], 0, bs_[b]) for b in range(Bn)]
    packed = torch.cat([l[0].packed for l in layers])
    bias = torch.stack([bf16_dev(bb) for bb in bs_])
    x = torch.stack([bf16_dev(xx) for xx in xs_])
    y = mxfp8.linear_batched(x, packed, N, 0, bias)
    for b in range(Bn):
        y1 = layers[b][0](x[b])
        assert torch.equal(y[b].view(torch.int16), y1.view(torch.int16)), b
    for b in (0, Bn - 1):
        ref, _, _ = orc.linear_ref(xs_[b], layers[b][1], layers[b][2], 0, bs_[b])
        ok, rep = tolerance.check(host_bf16_bits(y[b]), ref, name="batched-decode-%d-%d" % (M, b))
        assert ok, rep
