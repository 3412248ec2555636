"""Seeded synthetic inputs for the MX linear layer workloads (host side, numpy only).

This module draws random bf16 tensors and nothing else: it holds none of the layer's arithmetic
(no quantization, no scaling rule, no GEMM), so the HIP path and the CPU oracle can both take
their inputs from it without sharing any of the method.

Recipe (one ``numpy.random.Generator(PCG64(seed + t))`` per tensor, t = 0 activations,
1 weights, 2 bias, 3 outlier-channel choice, 4 zero-block choice; values drawn in float32,
scaled, then rounded to bf16 with round-to-nearest-even):

==========  ==============================================================================
tiny        x [16, 512] ~ N(0, 1); W [256, 512] ~ N(0, 0.02); no bias
decode      x [M, 4096] ~ N(0, 1), M in {1, 8, 32}; W [4096, 4096] ~ N(0, 0.02);
            bias [4096] ~ N(0, 0.01)
prefill     x [4096, 4096] ~ N(0, 1); W [14336, 4096] ~ N(0, 0.02); no bias
outlier     x [2048, 4096] ~ N(0, 1), 41 random K-channels (1 % of 4096, rounded) x 100,
            262 random (row, 32-block) blocks (0.1 % of 2048 * 128, rounded) set to zero;
            W [6144, 4096] ~ N(0, 0.02); no bias
mxfp6       x [512, 8192] ~ Laplace(0, 1); W [8192, 8192] ~ N(0, 0.02); no bias
==========  ==============================================================================

bf16 tensors are returned as ``uint16`` bit patterns.
"""
import numpy as np

__all__ = ["CONFIGS", "bf16_bits", "normal_bf16", "laplace_bf16", "outlier_x", "make"]

# name -> (M, N, K, bias?, activation kind)
CONFIGS = {
    "tiny": dict(M=16, N=256, K=512, bias=False, act="normal"),
    "decode1": dict(M=1, N=4096, K=4096, bias=True, act="normal"),
    "decode8": dict(M=8, N=4096, K=4096, bias=True, act="normal"),
    "decode32": dict(M=32, N=4096, K=4096, bias=True, act="normal"),
    "prefill": dict(M=4096, N=14336, K=4096, bias=False, act="normal"),
    "outlier": dict(M=2048, N=6144, K=4096, bias=False, act="outlier"),
    "mxfp6": dict(M=512, N=8192, K=8192, bias=False, act="laplace"),
}

W_STD, BIAS_STD = 0.02, 0.01
OUTLIER_FRAC_CHANNELS, OUTLIER_GAIN, ZERO_BLOCK_FRAC = 0.01, 100.0, 0.001


def _rng(seed, t):
    return np.random.Generator(np.random.PCG64(int(seed) + int(t)))


def bf16_bits(f32):
    """float32 array -> bf16 bit patterns (uint16), round to nearest even; NaN stays NaN."""
    u = np.ascontiguousarray(f32, dtype=np.float32).view(np.uint32)
    r = ((u + np.uint32(0x7FFF) + ((u >> 16) & np.uint32(1))) >> 16).astype(np.uint16)
    nan = (u & np.uint32(0x7FFFFFFF)) > np.uint32(0x7F800000)
    return np.where(nan, np.uint16(0x7FC0), r)


def normal_bf16(shape, std, seed, t):
    g = _rng(seed, t)
    return bf16_bits(g.standard_normal(shape, dtype=np.float32) * np.float32(std))


def laplace_bf16(shape, seed, t):
    g = _rng(seed, t)
    return bf16_bits(g.laplace(0.0, 1.0, size=shape).astype(np.float32))


def outlier_x(M, K, seed):
    """N(0,1) activations with 1 % of K-channels x100 and 0.1 % of 32-blocks zeroed."""
    x = _rng(seed, 0).standard_normal((M, K), dtype=np.float32)
    n_ch = int(round(OUTLIER_FRAC_CHANNELS * K))
    ch = _rng(seed, 3).choice(K, size=n_ch, replace=False)
    x[:, ch] *= np.float32(OUTLIER_GAIN)
    KB = K // 32
    n_blk = int(round(ZERO_BLOCK_FRAC * M * KB))
    blk = _rng(seed, 4).choice(M * KB, size=n_blk, replace=False)
    xv = x.reshape(M, KB, 32)
    xv[blk // KB, blk % KB, :] = 0.0
    return bf16_bits(x), np.sort(ch), np.sort(blk)


def make(name, seed=0, M=None, N=None, with_w=True):
    """Inputs of a named workload: dict(x, w, bias (or None), M, N, K).  ``M`` / ``N`` override
    the row counts (reduced-size parity cases drawn from the same distributions: the first
    rows of the full-size tensors are not reproduced, only their distribution)."""
    cfg = dict(CONFIGS[name])
    if M is not None:
        cfg["M"] = int(M)
    if N is not None:
        cfg["N"] = int(N)
    Mr, N, K = cfg["M"], cfg["N"], cfg["K"]
    if cfg["act"] == "normal":
        x = normal_bf16((Mr, K), 1.0, seed, 0)
    elif cfg["act"] == "laplace":
        x = laplace_bf16((Mr, K), seed, 0)
    else:
        x = outlier_x(Mr, K, seed)[0]
    w = normal_bf16((N, K), W_STD, seed, 1) if with_w else None
    bias = normal_bf16((N,), BIAS_STD, seed, 2) if cfg["bias"] else None
    return dict(x=x, w=w, bias=bias, M=Mr, N=N, K=K)
