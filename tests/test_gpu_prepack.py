"""GPU: the load-time weight prepack has an exact inverse (aiter_flydsl page, row_major_weight:
the rearranged weight can always be read back as row-major [N, K]), for every format, ragged K,
and weight-scale tensors larger than [N, K/32] (process_weights_after_loading slices them)."""
import numpy as np
import pytest
import torch

from mx_block_scaled_amd import mxfp8
from tests.gpu_helpers import DEV, banner, host_u8, u8_dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("fmt", [0, 2, 3])
@pytest.mark.parametrize("N,K", [(16, 32), (48, 160), (256, 544), (4096, 4096), (128, 8192)])
def test_roundtrip(fmt, N, K):
    g = np.random.default_rng(N + K + fmt)
    row = K if fmt == 0 else K // 4 * 3
    wq = g.integers(0, 256, (N, row)).astype(np.uint8)
    ws = g.integers(0, 255, (N, K // 32)).astype(np.uint8)
    banner("prepack roundtrip", fmt, N, K)
    p = mxfp8.prepack_weight(u8_dev(wq), u8_dev(ws), fmt, K=K)
    assert p.numel() == mxfp8.prepacked_bytes(N, K, fmt)
    wq2, ws2 = mxfp8.unpack_weight(p, N, K, fmt)
    assert np.array_equal(host_u8(wq2), wq)
    assert np.array_equal(host_u8(ws2), ws)


def test_strided_sources():
    g = np.random.default_rng(9)
    N, K = 64, 256
    wq_big = g.integers(0, 256, (N, K + 32)).astype(np.uint8)     # row stride > K
    ws_big = g.integers(0, 255, (N + 16, K // 32 + 3)).astype(np.uint8)   # padded scale tensor
    t = u8_dev(wq_big)
    s = u8_dev(ws_big)
    p = torch.empty(mxfp8.prepacked_bytes(N, K, 0), dtype=torch.uint8, device=DEV)
    rc = mxfp8.lib().mxfp8_prepack_weight(t.data_ptr(), K + 32, s.data_ptr(), K // 32 + 3, N, K, 0,
                                          p.data_ptr(), None)
    assert rc == 0
    wq2, ws2 = mxfp8.unpack_weight(p, N, K, 0)
    assert np.array_equal(host_u8(wq2), wq_big[:, :K])
    assert np.array_equal(host_u8(ws2), ws_big[:N, :K // 32])


@pytest.mark.parametrize("N,K", [(16, 32), (48, 160), (256, 544), (4096, 4096)])
def test_shuffled16_import_export(N, K):
    """Weights in the aiter_flydsl page's (16, 16) preshuffled order (produced here by the
    oracle's shuffle, itself pinned to the page's row_major_weight inverse) prepack to exactly
    the bytes of the row-major prepack, and export back to that order."""
    import oracle as orc
    g = np.random.default_rng(3 * N + K)
    wq = g.integers(0, 256, (N, K)).astype(np.uint8)
    ws = g.integers(0, 255, (N, K // 32)).astype(np.uint8)
    w16 = orc.shuffle16(wq)
    banner("shuffled16 import/export", N, K)
    p_row = mxfp8.prepack_weight(u8_dev(wq), u8_dev(ws), 0)
    p_shuf = mxfp8.prepack_weight_shuffled16(u8_dev(w16.reshape(-1)), u8_dev(ws), N, K)
    assert torch.equal(p_row, p_shuf)
    w16b, ws2 = mxfp8.unpack_weight_shuffled16(p_row, N, K)
    assert np.array_equal(host_u8(w16b), w16.reshape(-1))
    assert np.array_equal(host_u8(ws2), ws)
