"""GPU parity of the fused producer of pre-quantized activations: RMS norm + MXFP8 quantization
(the Mxfp8LinearKernel page's input_quant_key; the norm is the reading in the oracle,
orc_rmsnorm) against the CPU oracle.

Bit-exact: the normalized bf16 rows y, the E4M3 codes and the E8M0 scales.  The one place
where the two sides may differ is fp32(r): the fp64 sum of squares is added in a different
order, so a row whose r lies within 2^-45 (relative) of an fp32 rounding tie is exempt (such
rows are counted and must be absent from these seeded inputs).  The fused codes equal the GPU
quantizer applied to the kernel's own y, bit for bit.  Then the layer on the fused output.
"""
import numpy as np
import pytest
import torch

import oracle as orc
from mx_block_scaled_amd import mxfp8, synth
from tests import tolerance
from tests.gpu_helpers import banner, bf16_dev, host_bf16_bits, host_u8, u8_dev

pytestmark = pytest.mark.gpu


def _r32_ambiguous(x_bits, eps):
    """rows whose r = 1 / sqrt(mean(x^2) + eps) is within 2^-45 of an fp32 rounding tie"""
    xd = tolerance.bf16_to_f64(x_bits)
    r = 1.0 / np.sqrt((xd * xd).sum(axis=1) / xd.shape[1] + eps)
    e = np.floor(np.log2(r))
    q = r / np.exp2(e - 23)
    return np.abs(q - np.floor(q) - 0.5) < 2.0 ** -22


def _inputs(M, K, seed, outliers=False):
    g = np.random.default_rng(seed)
    x = g.standard_normal((M, K)).astype(np.float32)
    if outliers:
        x[:, g.choice(K, max(1, K // 100), replace=False)] *= 100.0
        x[g.integers(0, M, 3), :] *= 1e-3
    gamma = (g.uniform(0.25, 2.0, K) * np.where(g.random(K) < 0.1, -1, 1)).astype(np.float32)
    return synth.bf16_bits(x), synth.bf16_bits(gamma)


@pytest.mark.parametrize("M,K,eps,outliers", [(64, 4096, 1e-6, False), (37, 608, 1e-5, True),
                                              (5, 32, 0.0, False), (300, 1024, 1e-6, True),
                                              (4096, 4096, 1e-6, False), (33, 8192, 1e-6, True),
                                              (6, 5120, 1e-6, False), (3, 12320, 1e-5, True)])
def test_rmsnorm_quantize(M, K, eps, outliers):
    x, gamma = _inputs(M, K, M + K, outliers)
    banner("rmsnorm+quant", M, K, eps, outliers)
    xq, xs, y = mxfp8.rmsnorm_quantize_act(bf16_dev(x), bf16_dev(gamma), eps, return_y=True)
    y_ref, _ = orc.rmsnorm(x, gamma, np.float32(eps))
    q_ref, s_ref = orc.quantize(y_ref)
    amb = _r32_ambiguous(x, float(np.float32(eps)))
    assert amb.sum() == 0, np.nonzero(amb)
    assert np.array_equal(host_bf16_bits(y), y_ref)
    assert np.array_equal(host_u8(xs), s_ref)
    assert np.array_equal(host_u8(xq), q_ref)
    # the fused codes are the GPU quantizer's codes for the kernel's own y
    q2, s2 = mxfp8.quantize_act(y)
    assert torch.equal(q2, xq) and torch.equal(s2, xs)


def test_producer_feeds_the_layer():
    """RMS norm + quantization, then the pre-quantized layer entry, against the oracle."""
    M, N, K = 512, 1024, 4096
    x, gamma = _inputs(M, K, 7, outliers=True)
    g = np.random.default_rng(8)
    w = synth.bf16_bits((g.standard_normal((N, K)) * 0.02).astype(np.float32))
    wq, ws = orc.quantize(w)
    layer = mxfp8.MxLinear(u8_dev(wq), u8_dev(ws), 0)
    banner("producer -> layer", M, N, K)
    xq, xs = mxfp8.rmsnorm_quantize_act(bf16_dev(x), bf16_dev(gamma), 1e-6)
    y = layer.apply_quantized(xq, xs)
    y_ref, _ = orc.rmsnorm(x, gamma, np.float32(1e-6))
    ref, _, _ = orc.linear_ref(y_ref, wq, ws)
    ok, rep = tolerance.check(host_bf16_bits(y), ref, name="producer-layer")
    assert ok, rep
