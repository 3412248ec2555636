"""mxfp8_linear_noalloc: the allocation-free variant of mxfp8_linear (its workspace is the
library's static per-GPU scratch array).  Called through the C ABI; its output must equal
mxfp8_linear's with a caller workspace bit for bit (same kernels, same order) and meet the
oracle tolerance, on consecutive calls that leave the shared array in different states."""
import ctypes

import numpy as np
import pytest
import torch

import oracle as orc
from mx_block_scaled_amd import mxfp8, synth
from tests import tolerance

MX_OK, MX_EWORKSPACE = 0, -4


def _lib():
    return mxfp8.lib()


def test_scratch_limit_is_refused_before_any_gpu_call():
    """A shape whose workspace exceeds the array is refused with MX_EWORKSPACE, and so is any
    bad argument, before the library touches HIP (this runs without a GPU)."""
    L = _lib()
    A = ctypes.c_void_p(1 << 20)           # aligned dummies; never dereferenced
    M, N, K = 8192, 1024, 8192
    assert mxfp8.workspace_bytes(M, N, K) > mxfp8.NOALLOC_SCRATCH_BYTES
    assert L.mxfp8_linear_noalloc(A, M, K, A, N, 0, None, A, None) == MX_EWORKSPACE
    assert b"scratch" in L.mxfp8_last_error()
    assert L.mxfp8_linear_noalloc(None, 4, 512, A, 256, 0, None, A, None) == -1
    assert L.mxfp8_linear_noalloc(A, 4, 500, A, 256, 0, None, A, None) == -2
    assert L.mxfp8_linear_noalloc(None, 0, 512, A, 256, 0, None, A, None) == MX_OK


def _case(M, N, K, seed, fmt=0, with_bias=True):
    g = np.random.default_rng(seed)
    x = synth.bf16_bits(g.standard_normal((M, K)).astype(np.float32))
    w = synth.bf16_bits((g.standard_normal((N, K)) * 0.02).astype(np.float32))
    b = synth.bf16_bits((g.standard_normal(N) * 0.05).astype(np.float32)) if with_bias else None
    wq, ws = orc.quantize(w, fmt)
    return x, wq, ws, b


def _dev(bits, dtype):
    a = np.ascontiguousarray(bits)
    if dtype == torch.bfloat16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(a).cuda()


@pytest.mark.gpu
def test_noalloc_equals_linear_on_consecutive_calls():
    L = _lib()
    st = torch.cuda.current_stream().cuda_stream
    # the second and third calls are smaller than the first; each leaves the shared array in a
    # different state (quantized activations + split-K parts, then the decode kernel's counters
    # and partial sums, then a path without scratch)
    for i, (M, N, K) in enumerate([(300, 1024, 2048), (24, 1024, 2048), (4, 512, 1024),
                                   (32, 4096, 4096)]):
        print("[gpu-case] noalloc", i, M, N, K, flush=True)
        x, wq, ws, b = _case(M, N, K, 100 + i)
        xd, bd = _dev(x, torch.bfloat16), _dev(b, torch.bfloat16)
        pk = mxfp8.prepack_weight(_dev(wq, torch.uint8), _dev(ws, torch.uint8), 0)
        y0 = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        y1 = torch.full((M, N), -7.0, dtype=torch.bfloat16, device="cuda")
        wsp = mxfp8.new_workspace(mxfp8.workspace_bytes(M, N, K))
        rc = L.mxfp8_linear(xd.data_ptr(), M, K, pk.data_ptr(), N, 0, bd.data_ptr(),
                            y0.data_ptr(), wsp.data_ptr(), wsp.numel(), st)
        assert rc == MX_OK, L.mxfp8_last_error()
        rc = L.mxfp8_linear_noalloc(xd.data_ptr(), M, K, pk.data_ptr(), N, 0, bd.data_ptr(),
                                    y1.data_ptr(), st)
        assert rc == MX_OK, L.mxfp8_last_error()
        torch.cuda.synchronize()
        assert torch.equal(y0.view(torch.int16), y1.view(torch.int16)), (M, N, K)
        ref, _, _ = orc.linear_ref(x, wq, ws, 0, b)
        yb = y1.view(torch.int16).cpu().numpy().view(np.uint16)
        ok, rep = tolerance.check(yb, ref, name="noalloc-%d-%d-%d" % (M, N, K))
        assert ok, rep
        # the same call again reuses the array as the previous call left it
        y2 = torch.empty_like(y1)
        assert L.mxfp8_linear_noalloc(xd.data_ptr(), M, K, pk.data_ptr(), N, 0, bd.data_ptr(),
                                      y2.data_ptr(), st) == MX_OK
        torch.cuda.synchronize()
        assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))


@pytest.mark.gpu
def test_noalloc_binding_and_graph_replay():
    """The binding's linear_noalloc captured in a HIP graph: every replay equals the eager call
    (the scratch array's address is fixed, so the captured kernels need no workspace)."""
    M, N, K = 20, 2048, 4096
    x, wq, ws, b = _case(M, N, K, 7)
    xd, bd = _dev(x, torch.bfloat16), _dev(b, torch.bfloat16)
    pk = mxfp8.prepack_weight(_dev(wq, torch.uint8), _dev(ws, torch.uint8), 0)
    eager = mxfp8.linear_noalloc(xd, pk, N, 0, bd).clone()
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        mxfp8.linear_noalloc(xd, pk, N, 0, bd, out=y)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        mxfp8.linear_noalloc(xd, pk, N, 0, bd, out=y)
    for _ in range(3):
        y.fill_(0)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), eager.view(torch.int16))
        mxfp8.linear_noalloc(xd, pk, N, 0, bd)          # eager work between replays
        torch.cuda.synchronize()
