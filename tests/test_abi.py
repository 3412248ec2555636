"""The C-ABI library loads, exports every entry point include/mxfp8.h declares, and rejects bad
arguments before touching HIP (so these run without a GPU)."""
import ctypes
import os
import re

import pytest

from mx_block_scaled_amd import mxfp8

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mxfp8.h")
MX_OK, MX_EINVAL, MX_ESHAPE, MX_EALIGN, MX_EWORKSPACE = 0, -1, -2, -3, -4


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(mxfp8_\w+)\s*\(", src)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(mxfp8.library_path):
        import __graft_entry__
        __graft_entry__.build()
    return mxfp8.lib()


def test_exports_every_declared_symbol(L):
    names = _declared()
    assert len(names) >= 10, names
    raw = ctypes.CDLL(mxfp8.library_path)
    for n in names:
        assert hasattr(raw, n), n


def test_binding_covers_header(L):
    # the Python binding registers a signature for each declared entry point
    for n in _declared():
        assert getattr(L, n).argtypes is not None or n == "mxfp8_last_error", n


# Fake 16-byte aligned "device" addresses.  Every call below must be rejected by argument
# validation (or be an M == 0 no-op): none may reach a kernel launch, so these tests are safe
# on a GPU machine too.
A = 1 << 20
B = (1 << 20) + 4096


def test_quantize_act_validation(L):
    assert L.mxfp8_quantize_act(A, 4, 48, 48, B, B, None) == MX_ESHAPE       # K % 32
    assert L.mxfp8_quantize_act(A, -1, 64, 64, B, B, None) == MX_ESHAPE
    assert L.mxfp8_quantize_act(None, 4, 64, 64, B, B, None) == MX_EINVAL
    assert L.mxfp8_quantize_act(A, 4, 64, 32, B, B, None) == MX_ESHAPE       # ldx < K
    assert L.mxfp8_quantize_act(A + 2, 4, 64, 64, B, B, None) == MX_EALIGN
    assert L.mxfp8_quantize_act(A, 4, 64, 68, B, B, None) == MX_EALIGN       # ldx % 8
    assert L.mxfp8_quantize_act(None, 0, 64, 64, None, None, None) == MX_OK  # M == 0: no-op
    L.mxfp8_quantize_act(A, 4, 40, 40, B, B, None)
    assert b"multiple of 32" in L.mxfp8_last_error()


def test_linear_validation(L):
    assert L.mxfp8_workspace_bytes(65, 256, 512, 0) == 65536 + 65 * 512 + 65 * 16  # prefix, xq, xs
    # 64 rows, K <= 4096: the role-split small-M kernel (no workspace); the size covers
    # batch-invariant mode's quantized activations
    ws = L.mxfp8_workspace_bytes(64, 256, 512, 0)
    assert ws == 65536 + 64 * 512 + 64 * 16
    # decode shapes with K split across workgroups (N % 64 == 0, 17 <= M <= 64, K > 4096): the
    # prefix, then the partial sums (K parts x N/64 column groups x (fragment, tile) pairs x
    # 1 KiB)
    assert L.mxfp8_workspace_bytes(32, 4096, 8192, 0) == 65536 + 4 * 64 * 8 * 1024
    assert L.mxfp8_workspace_bytes(17, 2048, 8192, 0) == 65536 + 8 * 32 * 8 * 1024
    assert L.mxfp8_workspace_bytes(48, 2048, 5120, 0) == 65536 + 5 * 32 * 12 * 1024
    assert L.mxfp8_workspace_bytes(64, 2048, 8192, 0) == 65536 + 8 * 32 * 16 * 1024
    # up to 16 rows (K <= 8192) and up to 64 (K <= 4096) run on the role-split small-M kernel,
    # which needs no workspace: the size covers batch-invariant mode's quantized activations
    for m in (16, 24, 25, 32, 48, 64):
        assert L.mxfp8_workspace_bytes(m, 4096, 4096, 0) == 65536 + m * 4096 + m * 128
    # above 64 rows, 32 tiles of 128 x 128: the quantized activations, then room for 8 K parts
    # of fp32 sums of the tiled GEMM (E4M3 operands run 4 parts on 64 x 128 tiles; the size
    # covers the 128 x 128 plan)
    q = 65536 + 65 * 4096 + 65 * 128
    need65 = (q + 255) // 256 * 256 + 8 * 65 * 4096 * 4
    assert L.mxfp8_workspace_bytes(65, 4096, 4096, 0) == need65
    # one byte short of the split-K parts: rejected before any launch
    assert L.mxfp8_linear(A, 65, 4096, B, 4096, 0, None, B, B, need65 - 1, None) == MX_EWORKSPACE
    assert b"needed" in L.mxfp8_last_error()
    # FP6 activations: the same split from 33 rows (no split-K decode kernel on that entry);
    # codes in 128-byte slices per K step (K % 128 == 0), so K bytes a row
    q6 = 65536 + 40 * 4096 + 40 * 128
    assert L.mxfp8_workspace_bytes_fmt(40, 4096, 4096, 2, 2) == (q6 + 255) // 256 * 256 + 8 * 40 * 4096 * 4
    assert L.mxfp8_workspace_bytes(8, 4096, 4096, 0) == 65536 + 8 * 4096 + 8 * 128
    assert L.mxfp8_workspace_bytes(1, 4096, 4096, 0) == 65536 + 4096 + 128
    assert L.mxfp8_linear(A, 64, 512, B, 256, 0, None, B, B, ws - 1, None) == MX_EWORKSPACE
    assert L.mxfp8_linear(A, 64, 512, B, 256, 0, None, B, None, ws, None) == MX_EWORKSPACE
    assert L.mxfp8_linear(A, 64, 512, B, 250, 0, None, B, B, ws, None) == MX_ESHAPE   # N % 16
    assert L.mxfp8_linear(A, 64, 500, B, 256, 0, None, B, B, ws, None) == MX_ESHAPE   # K % 32
    assert L.mxfp8_linear(A, 64, 512, B, 256, 1, None, B, B, ws, None) == MX_EINVAL   # E5M2: no
    assert L.mxfp8_linear(A, 64, 512, B, 256, 4, None, B, B, ws, None) == MX_EINVAL
    assert L.mxfp8_linear(A, 64, 512, None, 256, 0, None, B, B, ws, None) == MX_EINVAL
    assert L.mxfp8_linear(A, 64, 512, B, 256, 0, None, B + 8, B, ws, None) == MX_EALIGN
    assert L.mxfp8_linear(None, 0, 512, B, 256, 0, None, B, None, 0, None) == MX_OK
    assert L.mxfp8_linear_prequant(A, B, 64, 512, B, 256, 0, None, None, None) == MX_EINVAL
    assert L.mxfp8_linear_prequant(A, None, 64, 512, B, 256, 0, None, B, None) == MX_EINVAL
    assert L.mxfp8_linear_prequant(A + 1, B, 64, 512, B, 256, 0, None, B, None) == MX_EALIGN
    assert L.mxfp8_linear_prequant(A, B, 0, 512, B, 256, 0, None, B, None) == MX_OK


def test_weight_validation(L):
    assert L.mxfp8_prepack_weight(A, 500, B, 16, 256, 512, 0, B, None) == MX_ESHAPE   # ldw < K
    assert L.mxfp8_prepack_weight(A, 512, B, 8, 256, 512, 0, B, None) == MX_ESHAPE    # ld_ws
    assert L.mxfp8_prepack_weight(A, 520, B, 16, 256, 512, 0, B + 8, None) == MX_EALIGN  # packed
    # an FP6 row of 3K/4 = 384 bytes passes the shape check (then fails on the odd pointer)
    assert L.mxfp8_prepack_weight(A, 384, B, 16, 256, 512, 2, B + 1, None) == MX_EALIGN
    assert L.mxfp8_prepack_weight(A, 383, B, 16, 256, 512, 2, B, None) == MX_ESHAPE
    assert L.mxfp8_prepack_weight(A, 512, B, 16, 256, 512, 7, B, None) == MX_EINVAL
    assert L.mxfp8_unpack_weight(None, 256, 512, 0, B, B, None) == MX_EINVAL
    assert L.mxfp8_quantize_weight(A, 256, 512, 512, 5, B, B, None) == MX_EINVAL
    assert L.mxfp8_quantize_weight(A, 255, 512, 512, 0, B, B, None) == MX_ESHAPE


def test_sizes(L):
    # prepacked: K padded to 128 per 16-row fragment (2048 B E4M3, 1536 B FP6) + scale words
    assert L.mxfp8_prepacked_bytes(256, 512, 0) == 4 * 16 * 2048 + 1 * 16 * 256
    assert L.mxfp8_prepacked_bytes(256, 544, 0) == 5 * 16 * 2048 + 2 * 16 * 256
    assert L.mxfp8_prepacked_bytes(8192, 8192, 2) == 64 * 512 * 1536 + 16 * 512 * 256
    assert L.mxfp8_prepacked_bytes(250, 512, 0) == 0
    assert L.mxfp8_prepacked_bytes(256, 512, 9) == 0
    assert L.mxfp8_workspace_bytes(0, 256, 512, 0) == 0
    assert L.mxfp8_device_supported(-1) == MX_EINVAL


def test_binding_raises_without_library(monkeypatch, tmp_path):
    import importlib
    m = importlib.reload(mxfp8)
    monkeypatch.setattr(m, "library_path", str(tmp_path / "missing.so"))
    monkeypatch.setattr(m, "_lib", None)
    with pytest.raises(RuntimeError, match="not built"):
        m.lib()
    importlib.reload(mxfp8)


def test_shuffled16_and_mode_validation(L):
    assert L.mxfp8_prepack_weight_shuffled16(A, B, 16, 250, 512, B, None) == MX_ESHAPE   # N % 16
    assert L.mxfp8_prepack_weight_shuffled16(A, B, 8, 256, 512, B, None) == MX_ESHAPE    # ld_ws
    assert L.mxfp8_prepack_weight_shuffled16(None, B, 16, 256, 512, B, None) == MX_EINVAL
    assert L.mxfp8_prepack_weight_shuffled16(A, B, 16, 256, 512, B + 4, None) == MX_EALIGN
    assert L.mxfp8_unpack_weight_shuffled16(B, 256, 500, A, A, None) == MX_ESHAPE         # K % 32
    assert L.mxfp8_unpack_weight_shuffled16(B + 8, 256, 512, A, A, None) == MX_EALIGN
    assert L.mxfp8_set_batch_invariant(1) == MX_OK
    assert L.mxfp8_set_batch_invariant(0) == MX_OK
    for mode in (1, 0, -1):
        assert L.mxfp8_set_batch_invariant_thread(mode) == MX_OK
    assert L.mxfp8_set_batch_invariant_thread(2) == MX_EINVAL
    assert L.mxfp8_set_batch_invariant_thread(-2) == MX_EINVAL


def test_batched_validation(L):
    ws = L.mxfp8_workspace_bytes(3 * 64, 256, 512, 0)
    assert L.mxfp8_linear_batched(A, -1, 64, 512, B, 256, 0, None, B, B, ws, None) == MX_ESHAPE
    assert L.mxfp8_linear_batched(None, 3, 64, 512, B, 256, 0, None, B, B, ws, None) == MX_EINVAL
    assert L.mxfp8_linear_batched(A, 3, 64, 512, B, 256, 0, None, B, B, ws - 1, None) == MX_EWORKSPACE
    assert L.mxfp8_linear_batched(A, 3, 64, 500, B, 256, 0, None, B, B, ws, None) == MX_ESHAPE
    assert L.mxfp8_linear_batched(None, 0, 64, 512, B, 256, 0, None, B, None, 0, None) == MX_OK
    assert L.mxfp8_linear_prequant_batched(A, None, 3, 64, 512, B, 256, 0, None, B, None) == MX_EINVAL
    assert L.mxfp8_linear_prequant_batched(A, B, 70000, 1, 512, B, 256, 0, None, B, None) == MX_ESHAPE
    assert L.mxfp8_linear_prequant_batched(A, B, 3, 0, 512, B, 256, 0, None, B, None) == MX_OK


def test_tile_config_hook(L):
    assert L.mxfp8_set_tile_config(3, 3) == MX_EINVAL
    assert L.mxfp8_set_tile_config(0, 0) == MX_OK


def test_fp6_activation_validation(L):
    """MXFP6 activations (mxfp6 page, activation_quant_key): format pairs, shapes, workspace."""
    q = L.mxfp8_quantize_act_fmt
    assert q(A, 4, 64, 64, 1, B, B, None) == MX_EINVAL          # no E5M2
    assert q(A, 4, 48, 48, 2, B, B, None) == MX_ESHAPE          # K % 32
    assert q(A, 4, 64, 32, 3, B, B, None) == MX_ESHAPE          # ldx < K
    assert q(A + 2, 4, 64, 64, 3, B, B, None) == MX_EALIGN
    assert q(None, 4, 64, 64, 2, B, B, None) == MX_EINVAL
    assert q(None, 0, 64, 64, 2, None, None, None) == MX_OK      # M == 0: no-op
    # workspace: the 64 KiB counter prefix, the FP6 codes (K % 128 == 0: every K step's 96 bytes
    # in a 128-byte slice, K bytes a row; else packed, 3K/4 bytes a row), then the scales at a
    # 256-byte boundary
    assert L.mxfp8_workspace_bytes_fmt(64, 256, 512, 2, 2) == 65536 + 64 * 512 + 64 * 16
    assert L.mxfp8_workspace_bytes_fmt(3, 256, 160, 3, 2) == 65536 + 512 + 3 * 5
    assert L.mxfp8_workspace_bytes_fmt(64, 256, 512, 0, 2) == 0   # FP6 activations: FP6 weights
    assert L.mxfp8_workspace_bytes_fmt(64, 256, 512, 2, 0) == L.mxfp8_workspace_bytes(64, 256, 512, 2)
    ws = L.mxfp8_workspace_bytes_fmt(64, 256, 512, 2, 3)
    f = L.mxfp8_linear_fmt
    assert f(A, 64, 512, B, 256, 0, 2, None, B, B, ws, None) == MX_EINVAL     # E4M3 weight
    assert f(A, 64, 512, B, 256, 2, 1, None, B, B, ws, None) == MX_EINVAL
    assert f(A, 64, 512, B, 256, 2, 3, None, B, B, ws - 1, None) == MX_EWORKSPACE
    assert f(A, 64, 500, B, 256, 2, 3, None, B, B, ws, None) == MX_ESHAPE
    assert f(A, 64, 512, B, 250, 2, 3, None, B, B, ws, None) == MX_ESHAPE
    assert f(A, 64, 512, B, 256, 2, 3, None, B + 8, B, ws, None) == MX_EALIGN
    assert f(None, 0, 512, B, 256, 3, 3, None, B, None, 0, None) == MX_OK
    p = L.mxfp8_linear_prequant_fmt
    assert p(A, B, 64, 512, 2, B, 256, 0, None, B, None) == MX_EINVAL        # E4M3 weight
    assert p(A, None, 64, 512, 2, B, 256, 2, None, B, None) == MX_EINVAL
    assert p(A + 8, B, 64, 512, 2, B, 256, 2, None, B, None) == MX_EALIGN
    assert p(A, B, 64, 512, 3, B, 256, 3, None, None, None) == MX_EINVAL     # y
    assert p(A, B, 0, 512, 3, B, 256, 2, None, B, None) == MX_OK


def test_rmsnorm_quantize_validation(L):
    f = L.mxfp8_rmsnorm_quantize_act
    assert f(A, 4, 64, 64, B, -1.0, B, B, None, None) == MX_EINVAL           # eps < 0
    assert f(A, 4, 64, 64, B, float("nan"), B, B, None, None) == MX_EINVAL
    assert f(A, 4, 64, 64, B, float("inf"), B, B, None, None) == MX_EINVAL
    assert f(A, 4, 64, 64, None, 1e-6, B, B, None, None) == MX_EINVAL        # gamma
    assert f(A, 4, 48, 48, B, 1e-6, B, B, None, None) == MX_ESHAPE           # K % 32
    assert f(A, 4, 64, 32, B, 1e-6, B, B, None, None) == MX_ESHAPE           # ldx < K
    assert f(A, 4, 64, 64, B + 2, 1e-6, B, B, None, None) == MX_EALIGN
    assert f(A, 4, 64, 64, B, 1e-6, B, B, A + 8, None) == MX_EALIGN          # y
    assert f(None, 0, 64, 64, None, 1e-6, None, None, None, None) == MX_OK   # M == 0
