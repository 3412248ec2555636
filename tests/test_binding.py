"""The Python binding's argument checks (CPU only: every case raises before any GPU call).

A wrong ``out``, ``bias``, ``packed`` or ``workspace`` would make the kernels read or write out of
bounds, so the binding rejects each before it reaches the library; the shape checks run before
the device check, so CPU tensors exercise them here.
"""
import pytest
import torch

from mx_block_scaled_amd import mxfp8

M, N, K = 8, 256, 512


def _x():
    return torch.zeros((M, K), dtype=torch.bfloat16)


def _packed(n=N, k=K, fmt=0, extra=0):
    return torch.zeros(mxfp8.prepacked_bytes(n, k, fmt) + extra, dtype=torch.uint8)


def test_cpu_tensors_are_refused_after_the_shape_checks():
    with pytest.raises(ValueError, match="CUDA tensor"):
        mxfp8.linear(_x(), _packed(), N)
    with pytest.raises(ValueError, match="CUDA tensor"):
        mxfp8.quantize_act(_x())


@pytest.mark.parametrize("shape", [(M, N + 16), (M + 1, N), (M * N,), (N, M)])
def test_out_of_the_wrong_shape(shape):
    out = torch.zeros(shape, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="out has shape"):
        mxfp8.linear(_x(), _packed(), N, out=out)
    xq = torch.zeros((M, K), dtype=torch.uint8)
    xs = torch.zeros((M, K // 32), dtype=torch.uint8)
    with pytest.raises(ValueError, match="out has shape"):
        mxfp8.linear_prequant(xq, xs, _packed(), N, out=out)


def test_out_of_the_wrong_dtype_or_layout():
    with pytest.raises(TypeError):
        mxfp8.linear(_x(), _packed(), N, out=torch.zeros((M, N), dtype=torch.float32))
    with pytest.raises(ValueError, match="contiguous"):
        mxfp8.linear(_x(), _packed(), N, out=torch.zeros((N, M), dtype=torch.bfloat16).t())


@pytest.mark.parametrize("n", [N - 16, N + 1, 1])
def test_bias_of_the_wrong_size(n):
    bias = torch.zeros(n, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="bias has shape"):
        mxfp8.linear(_x(), _packed(), N, bias=bias)
    with pytest.raises(ValueError, match="bias has shape"):
        mxfp8.linear_fmt(_x(), _packed(fmt=2), N, "e2m3", "e2m3", bias=bias)


@pytest.mark.parametrize("delta", [-1, 1, 4096])
def test_packed_of_the_wrong_size(delta):
    with pytest.raises(ValueError, match="packed holds"):
        mxfp8.linear(_x(), _packed(extra=delta), N)
    with pytest.raises(ValueError, match="packed holds"):
        mxfp8.unpack_weight(_packed(extra=delta), N, K)
    # a weight prepacked for another N or format is refused too
    with pytest.raises(ValueError, match="packed holds"):
        mxfp8.linear(_x(), _packed(n=N + 16), N)
    with pytest.raises(ValueError, match="packed holds"):
        mxfp8.linear(_x(), _packed(fmt=2), N, "e4m3")


def test_workspace_too_small_or_wrong_type():
    need = mxfp8.workspace_bytes(M, N, K)
    with pytest.raises(ValueError, match="workspace holds"):
        mxfp8.linear(_x(), _packed(), N, workspace=torch.zeros(need - 1, dtype=torch.uint8))
    with pytest.raises(ValueError, match="workspace must be"):
        mxfp8.linear(_x(), _packed(), N, workspace=torch.zeros(need, dtype=torch.int32))


def test_prequant_scale_and_code_shapes():
    xq = torch.zeros((M, K), dtype=torch.uint8)
    for xs_shape in [(M, K // 32 + 1), (K // 32, M), (M * K // 32,)]:
        with pytest.raises(ValueError, match="do not match"):
            mxfp8.linear_prequant(xq, torch.zeros(xs_shape, dtype=torch.uint8), _packed(), N)
    # FP6 codes are 3K/4 bytes per row
    with pytest.raises(ValueError, match="do not match"):
        mxfp8.linear_prequant_fmt(xq, torch.zeros((M, K // 32), dtype=torch.uint8),
                                  _packed(fmt=2), N, K, "e2m3", "e2m3")


def test_batched_shapes():
    B = 3
    x = torch.zeros((B, M, K), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="packed holds"):
        mxfp8.linear_batched(x, _packed(), N)                    # one weight for three layers
    pk = torch.cat([_packed()] * B)
    with pytest.raises(ValueError, match="bias has shape"):
        mxfp8.linear_batched(x, pk, N, bias=torch.zeros(N, dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="out has shape"):
        mxfp8.linear_batched(x, pk, N, out=torch.zeros((B, M, N - 16), dtype=torch.bfloat16))
    xq = torch.zeros((B, M, K), dtype=torch.uint8)
    with pytest.raises(ValueError, match="do not match"):
        mxfp8.linear_prequant_batched(xq, torch.zeros((B, M, K // 16), dtype=torch.uint8), pk, N)


def test_prepack_source_shapes():
    wq = torch.zeros((N, K), dtype=torch.uint8)
    with pytest.raises(ValueError, match="smaller than"):
        mxfp8.prepack_weight(wq, torch.zeros((N - 1, K // 32), dtype=torch.uint8))
    with pytest.raises(ValueError, match="smaller than"):
        mxfp8.prepack_weight(wq, torch.zeros((N, K // 32 - 1), dtype=torch.uint8))
    with pytest.raises(ValueError, match="K = "):
        mxfp8.prepack_weight(wq, torch.zeros((N, K // 16), dtype=torch.uint8), K=2 * K)
