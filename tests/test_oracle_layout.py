"""Pins for the oracle's FP6 storage and the pages' (16, 16) weight shuffle (CPU only)."""
import numpy as np
import torch


def test_fp6_pack_closed_forms(orc):
    # four 6-bit codes per three bytes, little-endian along K
    cases = {
        (1, 0, 0, 0): [1, 0, 0],
        (0, 1, 0, 0): [64, 0, 0],
        (0, 0, 1, 0): [0, 16, 0],
        (0, 0, 0, 1): [0, 0, 4],
        (63, 63, 63, 63): [255, 255, 255],
        (0x2A, 0x15, 0x3F, 0x00): [0x2A | (0x15 & 3) << 6, (0x15 >> 2) | (0x3F & 15) << 4, 0x3F >> 4],
    }
    for c, b in cases.items():
        got = orc.fp6_pack(np.array([c], np.uint8))
        assert got[0].tolist() == b, (c, got)


def test_fp6_pack_roundtrip(orc):
    g = np.random.default_rng(0)
    c = g.integers(0, 64, (9, 128)).astype(np.uint8)
    p = orc.fp6_pack(c)
    assert p.shape == (9, 96)
    assert np.array_equal(orc.fp6_unpack(p, 128), c)
    # a 32-element MX block is exactly 24 packed bytes
    assert np.array_equal(orc.fp6_pack(c[:, 32:64]), p[:, 24:48])


def test_shuffle16_against_pages_inverse(orc):
    """aiter_flydsl page, row_major_weight: the stored [N/16, K/32, 2, 16, 16] array is turned back
    into row-major W by view(n/16, k/32, 2, 16, 16).permute(0, 3, 1, 2, 4).reshape(n, k)."""
    g = np.random.default_rng(1)
    for N, K in [(16, 32), (32, 64), (48, 256), (256, 512)]:
        w = g.integers(0, 256, (N, K)).astype(np.uint8)
        s = orc.shuffle16(w)
        t = torch.from_numpy(s.copy())
        back = t.view(N // 16, K // 32, 2, 16, 16).permute(0, 3, 1, 2, 4).reshape(N, K).numpy()
        assert np.array_equal(back, w)
        assert np.array_equal(orc.unshuffle16(s, N, K), w)
        # and the inverse-then-forward direction
        assert np.array_equal(orc.shuffle16(orc.unshuffle16(s, N, K)), s)


def test_shuffle16_index_matrix(orc):
    """Byte offset of W[n, k] in the stored order is ((n0*KB + k0)*2 + k1)*256 + n1*16 + k2."""
    N, K = 32, 64
    idx = np.arange(N * K).reshape(N, K)
    lo = (idx % 256).astype(np.uint8)
    hi = (idx // 256).astype(np.uint8)
    s = orc.shuffle16(lo).astype(np.int64) + 256 * orc.shuffle16(hi).astype(np.int64)
    for n in range(N):
        for k in range(K):
            off = (((n // 16) * (K // 32) + k // 32) * 2 + (k % 32) // 16) * 256 + (n % 16) * 16 + k % 16
            assert s[off] == n * K + k
