"""GPU parity of the decode path that splits K across workgroups (mxfp8_linear with bf16
activations, N % 64 == 0, K % 128 == 0, 17 <= M <= 64 with K > 4096, and M = 16 with
K > 8192: the shapes whose activation rows the role-split small-M kernel does not hold).

That kernel quantizes the activations itself, in the MFMA operand layout, and adds the K parts
of a column group in a fixed order chosen by the last workgroup to finish (a counter in the
workspace, which every call leaves at zero).  Checked here:
- the layer against the fp64 oracle to the usual bar, for one to eight K parts, ragged parts,
  every weight format, with and without bias, outlier channels and all-zero blocks;
- a block holding Inf: its rows are NaN, as in the oracle, and the other rows are unaffected;
- repeated calls and calls of other shapes and entry points sharing one workspace: results
  repeat bit for bit (the counters come back to zero);
- the calls replayed from a HIP graph, each replay against the eager results.
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

# (M, N, K): K parts = min(ceil(256 / (N / 64)), max(1, K / 1024), 8)
SHAPES = [
    (16, 1024, 16384),  # one activation tile, eight parts of 16 K steps
    (28, 2048, 8192),   # two activation tiles, eight parts of 8 K steps
    (32, 4096, 8192),   # two activation tiles, four parts of 16 K steps
    (17, 4096, 4480),   # 35 K steps in four parts of 8 or 9
    (20, 1024, 8192),   # eight parts
    (20, 16384, 4224),  # 256 column groups: one part of 33 K steps, no cross-workgroup sum
    (26, 640, 5120),    # ten column groups, five parts of 8 K steps on different XCDs
    (33, 4096, 8192),   # three activation tiles, the third with one row
    (48, 2048, 5120),   # three full tiles, five parts of 8 K steps
    (64, 2048, 8192),   # four tiles: each wave finishes two (fragment, tile) pairs
    (57, 2048, 4608),   # four tiles, four parts of 9 K steps
]


def _inputs(M, N, K, seed):
    g = np.random.default_rng(seed)
    x = g.standard_normal((M, K)).astype(np.float32)
    x[:, g.choice(K, max(1, K // 100), replace=False)] *= 60.0       # outlier channels
    xb = x.reshape(M, K // 32, 32)
    xb[g.integers(0, M, 2), g.integers(0, K // 32, 2)] = 0.0          # all-zero blocks
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
def test_decode_split_k_matches_oracle(M, N, K, fmt):
    x, w, b = _inputs(M, N, K, M * 7 + N + K + fmt)
    use_bias = (M + fmt) % 2 == 0
    layer, wq, ws = _layer(w, fmt, b if use_bias else None)
    banner("decode split-K", M, N, K, FMTS[fmt], "bias" if use_bias else "no bias")
    y = layer(bf16_dev(x))
    ref, _, _ = orc.linear_ref(x, wq, ws, fmt, b if use_bias else None)
    ok, rep = tolerance.check(host_bf16_bits(y), ref, name="sk-%d-%d-%d-%d" % (M, N, K, fmt))
    assert ok, rep


def test_decode_split_k_inf_block():
    M, N, K = 27, 2048, 8192
    x, w, b = _inputs(M, N, K, 5)
    x[3, 1000] = 0x7F80                     # +Inf in row 3
    layer, wq, ws = _layer(w, 0, b)
    banner("decode split-K, Inf block", M, N, K)
    y = host_bf16_bits(layer(bf16_dev(x)))
    ref, _, _ = orc.linear_ref(x, wq, ws, 0, b)
    yf = tolerance.bf16_to_f64(y)
    assert np.isnan(yf[3]).all() and np.isnan(ref[3]).all()
    keep = np.arange(M) != 3
    ok, rep = tolerance.check(y[keep], ref[keep], name="sk-inf")
    assert ok, rep


def test_decode_split_k_workspace_reuse():
    """One workspace for a sequence of calls of several shapes and entry points: every call
    repeats its first result bit for bit, so the counters are back at zero after each call."""
    K = 8192
    g = np.random.default_rng(11)
    shapes = [(32, 4096), (16, 1024), (3, 4096), (300, 256), (1, 4096), (20, 640), (64, 4096),
              (100, 4096)]
    ws_bytes = max(mxfp8.workspace_bytes(M, N, K) for M, N in shapes)
    ws = torch.zeros(ws_bytes, dtype=torch.uint8, device=DEV)
    calls = []
    for M, N in shapes:
        x = bf16_dev(synth.bf16_bits(g.standard_normal((M, K)).astype(np.float32)))
        wb = synth.bf16_bits((g.standard_normal((N, K)) * 0.02).astype(np.float32))
        wq, wsc = orc.quantize(wb, 0)
        pk = mxfp8.prepack_weight(u8_dev(wq), u8_dev(wsc), 0)
        calls.append((x, pk, N))
    banner("decode split-K workspace reuse", shapes)
    first = [mxfp8.linear(x, pk, N, 0, workspace=ws).clone() for x, pk, N in calls]
    assert int(ws[:65536].count_nonzero()) == 0
    for rnd in range(3):
        for i in ([0, 1, 2, 3, 4, 5, 6, 7] if rnd != 1 else [5, 3, 7, 0, 6, 0, 2, 1, 4]):
            x, pk, N = calls[i]
            y = mxfp8.linear(x, pk, N, 0, workspace=ws)
            assert torch.equal(y.view(torch.int16), first[i].view(torch.int16)), (rnd, i)
    torch.cuda.synchronize()
    assert int(ws[:65536].count_nonzero()) == 0


def test_decode_split_k_graph_replay():
    """The calls captured in a HIP graph: no memset nodes; every replay, with eager work and
    synchronizations in between, equals the eager results."""
    g = np.random.default_rng(12)
    N, K = 4096, 8192
    wb = synth.bf16_bits((g.standard_normal((N, K)) * 0.02).astype(np.float32))
    wq, wsc = orc.quantize(wb, 0)
    pk = mxfp8.prepack_weight(u8_dev(wq), u8_dev(wsc), 0)
    xs = [bf16_dev(synth.bf16_bits(g.standard_normal((M, K)).astype(np.float32)))
          for M in (32, 16, 2, 64, 100)]
    ws = torch.zeros(max(mxfp8.workspace_bytes(x.shape[0], N, K) for x in xs),
                     dtype=torch.uint8, device=DEV)
    ys = [torch.empty((x.shape[0], N), dtype=torch.bfloat16, device=DEV) for x in xs]
    banner("decode split-K graph replay")
    eager = [mxfp8.linear(x, pk, N, 0, out=torch.empty_like(y), workspace=ws).clone()
             for x, y in zip(xs, ys)]
    s = torch.cuda.Stream(DEV)
    s.wait_stream(torch.cuda.current_stream(DEV))
    with torch.cuda.stream(s):
        for x, y in zip(xs, ys):
            mxfp8.linear(x, pk, N, 0, out=y, workspace=ws)
    torch.cuda.current_stream(DEV).wait_stream(s)
    torch.cuda.synchronize()
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gr, stream=s):
        for x, y in zip(xs, ys):
            mxfp8.linear(x, pk, N, 0, out=y, workspace=ws)
    for rep in range(4):
        for y in ys:
            y.zero_()
        gr.replay()
        torch.cuda.synchronize()
        for y, e in zip(ys, eager):
            assert torch.equal(y.view(torch.int16), e.view(torch.int16)), rep
        # eager work between replays, on the same workspace
        mxfp8.linear(xs[1], pk, N, 0, workspace=ws)
        torch.cuda.synchronize()


@pytest.mark.parametrize("bi", [False, True])
@pytest.mark.parametrize("M,K", [(1, 2048), (2, 2048), (8, 2048), (12, 2048), (16, 2048),
                                 (20, 2048), (24, 2048), (32, 2048), (50, 2048), (64, 2048),
                                 (100, 2048), (32, 4224), (50, 4224)])
def test_fused_quantizers_bit_exact_through_identity_weight(M, K, bi):
    """With W = I (E4M3 1.0 on the diagonal, scale 2^0) every output is one dequantized
    activation, exact in fp32 and in bf16, so the layer's output equals the oracle's
    dequantize(quantize(x)) bit for bit: a bit-level check of the quantizer each path fuses
    (role-split small-M kernel at M = 1 .. 16 with each of its row counts in one row tile, at
    20, 24 and 32 in two row tiles, at 50 and 64 in four; split-K decode kernel at 32 and 50
    with K = 4224; quantizer launch + tiled GEMM at 100; in batch-invariant mode the
    role-split kernel's in-order form up to 64 rows with K = 2048, and the quantizer launch +
    generic or tiled GEMM otherwise).  Inputs hold outlier channels, all-zero blocks, values
    that saturate at 448 after scaling, bf16 subnormals and exact rounding ties."""
    N = K
    g = np.random.default_rng(M + 77)
    x = g.standard_normal((M, K)).astype(np.float32)
    x[:, g.choice(K, 20, replace=False)] *= 200.0
    xb = x.reshape(M, K // 32, 32)
    xb[g.integers(0, M, 3), g.integers(0, K // 32, 3)] = 0.0
    xb[:, 5, :] = g.standard_normal((M, 32)).astype(np.float32) * 1e-39      # bf16 subnormals
    xb[:, 7, 0] = 480.0                  # block max 480: scale 2^0, 480 saturates to 448
    xb[:, 7, 1:5] = [12.5, 13.5, 17.0, 19.0]   # halfway between E4M3 neighbours: even wins
    x_bits = synth.bf16_bits(x)
    w = np.eye(N, K, dtype=np.float32)
    layer, wq, ws = _layer(synth.bf16_bits(w), 0, None)
    banner("identity weight, bit-exact quantizer", M, N, K, "batch-invariant" if bi else "")
    mxfp8.set_batch_invariant(bi)
    try:
        y = host_bf16_bits(layer(bf16_dev(x_bits)))
    finally:
        mxfp8.set_batch_invariant(False)
    xq, xs = orc.quantize(x_bits, orc.E4M3)
    expect = orc.f64_to_bf16(orc.dequantize(xq, xs, orc.E4M3))
    # the layer's output is a sum started at +0, so a code of -0 comes out as +0
    expect[expect == 0x8000] = 0
    assert np.array_equal(y, expect), np.argwhere(y != expect)[:8]


def test_fused_quantizer_two_activation_tiles_bit_exact_through_identity_weight():
    """The role-split kernel's one-row-tile form with two 16-row activation tiles (24 rows,
    N % 32 != 0): W = [I; 0], so the first K outputs of a row are its dequantized activations,
    bit for bit, and the last 16 are zero."""
    M, N, K = 24, 2064, 2048
    g = np.random.default_rng(5)
    x = g.standard_normal((M, K)).astype(np.float32)
    x[:, g.choice(K, 20, replace=False)] *= 200.0
    xb = x.reshape(M, K // 32, 32)
    xb[g.integers(0, M, 3), g.integers(0, K // 32, 3)] = 0.0
    xb[:, 5, :] = g.standard_normal((M, 32)).astype(np.float32) * 1e-39
    xb[:, 7, 0] = 480.0
    xb[:, 7, 1:5] = [12.5, 13.5, 17.0, 19.0]
    x_bits = synth.bf16_bits(x)
    layer, wq, ws = _layer(synth.bf16_bits(np.eye(N, K, dtype=np.float32)), 0, None)
    banner("identity weight, two activation tiles in one row tile", M, N, K)
    y = host_bf16_bits(layer(bf16_dev(x_bits)))
    xq, xs = orc.quantize(x_bits, orc.E4M3)
    expect = orc.f64_to_bf16(orc.dequantize(xq, xs, orc.E4M3))
    expect[expect == 0x8000] = 0
    assert np.array_equal(y[:, :K], expect), np.argwhere(y[:, :K] != expect)[:8]
    assert not y[:, K:].any()


@pytest.mark.parametrize("M", [8, 100])
@pytest.mark.parametrize("fmt", [2, 3])
def test_fp6_activations_bit_exact_through_identity_weight(M, fmt):
    """W6A6 through the identity weight (the format's 1.0 on the diagonal): every output is one
    dequantized FP6 activation, so the layer equals the oracle's dequantize(quantize(x, fmt)) bit
    for bit, which pins the FP6 operand reads of the generic (M = 8) and tiled (M = 100)
    kernels as well as the FP6 quantizer."""
    K = N = 1024
    g = np.random.default_rng(M + fmt)
    x = g.standard_normal((M, K)).astype(np.float32)
    x[:, g.choice(K, 10, replace=False)] *= 50.0
    x.reshape(M, K // 32, 32)[g.integers(0, M, 2), g.integers(0, K // 32, 2)] = 0.0
    x_bits = synth.bf16_bits(x)
    layer, wq, ws = _layer(synth.bf16_bits(np.eye(N, K, dtype=np.float32)), fmt, None)
    banner("identity weight, W6A6", M, N, K, FMTS[fmt])
    ws_t = mxfp8.new_workspace(mxfp8.workspace_bytes_fmt(M, N, K, fmt, fmt), DEV)
    y = host_bf16_bits(mxfp8.linear_fmt(bf16_dev(x_bits), layer.packed, N, fmt, fmt,
                                        workspace=ws_t))
    xq, xs = orc.quantize(x_bits, fmt)
    expect = orc.f64_to_bf16(orc.dequantize(xq, xs, fmt))
    expect[expect == 0x8000] = 0
    assert np.array_equal(y, expect), np.argwhere(y != expect)[:8]


def test_concurrent_streams_with_own_workspaces():
    """Calls on two streams at once, each stream with its own workspace (split-K decode kernel,
    tiled GEMM with K split, small-M kernel): every result equals the same call made alone,
    bit for bit, so workspaces that are not shared never interfere."""
    g = np.random.default_rng(21)
    N, K = 4096, 8192
    wb = synth.bf16_bits((g.standard_normal((N, K)) * 0.02).astype(np.float32))
    wq, wsc = orc.quantize(wb, 0)
    pk = mxfp8.prepack_weight(u8_dev(wq), u8_dev(wsc), 0)
    Ms = (32, 100, 48, 8)
    xs = [bf16_dev(synth.bf16_bits(g.standard_normal((M, K)).astype(np.float32))) for M in Ms]
    alone = [mxfp8.linear(x, pk, N, 0).clone() for x in xs]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(DEV), torch.cuda.Stream(DEV)]
    wss = [mxfp8.new_workspace(max(mxfp8.workspace_bytes(M, N, K) for M in Ms), DEV) for _ in streams]
    ys = [[torch.empty((x.shape[0], N), dtype=torch.bfloat16, device=DEV) for x in xs] for _ in streams]
    banner("two streams, own workspaces", Ms)
    for s in streams:
        s.wait_stream(torch.cuda.current_stream(DEV))
    for rep in range(4):
        for i, x in enumerate(xs):
            for si, s in enumerate(streams):
                with torch.cuda.stream(s):
                    mxfp8.linear(xs[(i + si) % len(xs)], pk, N, 0, out=ys[si][(i + si) % len(xs)],
                                 workspace=wss[si])
    torch.cuda.synchronize()
    for si in range(len(streams)):
        for i in range(len(xs)):
            assert torch.equal(ys[si][i].view(torch.int16), alone[i].view(torch.int16)), (si, i)
        assert int(wss[si][:65536].count_nonzero()) == 0
