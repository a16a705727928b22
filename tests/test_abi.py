"""The C ABI library loads, exports what include/kq.h declares, and rejects
bad arguments before touching the GPU.  No compute call is made here."""
import ctypes
import os
import re

import pytest

from conftest import ROOT

HEADER = os.path.join(ROOT, "include", "kq.h")


@pytest.fixture(scope="module")
def kq():
    import q6_q8_matmul_amd as kq
    from q6_q8_matmul_amd import build

    if not os.path.exists(kq.LIB_PATH):
        build.build()
    kq.lib()
    return kq


def declared_functions():
    with open(HEADER) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kq_\w+)\s*\(", text)))


def test_header_declares_the_boundary():
    assert declared_functions() == sorted([
        "kq_quantize_q8_1", "kq_gemv_q4k", "kq_gemv_q6k", "kq_mmq_q4k", "kq_mmq_q6k",
        "kq_q6k_split_bytes", "kq_repack_q6k", "kq_gemv_q6k_split", "kq_mmq_q6k_split",
        "kq_rmsnorm_q8_1", "kq_swiglu_q8_1", "kq_gemv_q4k_seg", "kq_last_error",
        "kq_abi_version", "kq_read_probe", "kq_read_probe_words", "kq_mmq_q6k_ws",
        "kq_mmq_q6k_workspace_bytes", "kq_mmq_q6k_noalloc", "kq_mmq_q4k_ws",
        "kq_mmq_q4k_workspace_bytes"])


def test_library_exports_every_declared_symbol(kq):
    lib = ctypes.CDLL(kq.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), f"{name} not exported"


def test_abi_version(kq):
    assert kq.kq_abi_version() == 2


# Fake, aligned, never-dereferenced addresses: every call below fails argument
# validation, which runs before any HIP call.
W = 0x10000
X = 0x20000
Y = 0x40000
R = 0x80000


def _rc(fn, *args):
    return fn(*args)


@pytest.mark.parametrize("args,needle", [
    ((None, X, 1, 256, None), "null pointer"),
    ((W, None, 1, 256, None), "null pointer"),
    ((W, X, 1, 0, None), "k=0"),
    ((W, X, 1, 48, None), "k=48"),
    ((W, X, 1, 65536 + 32, None), "k=65568"),
    ((W, X, -1, 256, None), "rows=-1"),
    ((W + 4, X, 1, 256, None), "misaligned"),
    ((W, X + 2, 1, 256, None), "misaligned"),
    ((W, W + 64, 1, 256, None), "overlaps"),
])
def test_quantize_rejects(kq, args, needle):
    rc = kq.lib().kq_quantize_q8_1(*args)
    assert rc == kq.KQ_ERR_ARG
    assert needle in kq.kq_last_error()
    assert "kq_quantize_q8_1" in kq.kq_last_error()


@pytest.mark.parametrize("fn", ["kq_gemv_q4k", "kq_gemv_q6k", "kq_gemv_q6k_split"])
@pytest.mark.parametrize("args,needle", [
    ((None, X, Y, None, 8, 256, 1, None), "null pointer"),
    ((W, X, None, None, 8, 256, 1, None), "null pointer"),
    ((W, X, Y, None, 8, 128, 1, None), "k=128"),
    ((W, X, Y, None, 8, 256 * 257, 1, None), "k="),
    ((W, X, Y, None, -3, 256, 1, None), "m=-3"),
    ((W, X, Y, None, 8, 256, 0, None), "batch=0"),
    ((W, X, Y, None, 8, 256, 9, None), "batch=9"),
    ((W + 8, X, Y, None, 8, 256, 1, None), "misaligned"),
    ((W, X + 1, Y, None, 8, 256, 1, None), "misaligned"),
    ((W, X + 4, Y, None, 8, 256, 1, None), "misaligned"),
    ((W, X, Y + 2, None, 8, 256, 1, None), "misaligned"),
    ((W, X, Y, R + 2, 8, 256, 1, None), "misaligned"),
    ((W, X, W + 16, None, 8, 256, 1, None), "overlaps"),
    ((W, X, X, None, 8, 256, 1, None), "overlaps"),
    ((W, X, Y, Y + 4, 8, 256, 1, None), "partially overlaps"),
])
def test_gemv_rejects(kq, fn, args, needle):
    rc = getattr(kq.lib(), fn)(*args)
    assert rc == kq.KQ_ERR_ARG, kq.kq_last_error()
    assert needle in kq.kq_last_error()
    assert fn in kq.kq_last_error()


@pytest.mark.parametrize("fn", ["kq_mmq_q4k", "kq_mmq_q6k", "kq_mmq_q6k_split", "kq_mmq_q6k_noalloc"])
@pytest.mark.parametrize("args,needle", [
    ((None, X, Y, 8, 8, 256, None), "null pointer"),
    ((W, X, Y, 8, 8, 100, None), "k=100"),
    ((W, X, Y, -1, 8, 256, None), "m=-1"),
    ((W, X, Y, 8, -1, 256, None), "n=-1"),
    ((W, X, Y, 8, 65535 * 128 + 1, 256, None), "out of range"),
    ((W + 4, X, Y, 8, 8, 256, None), "misaligned"),
    ((W, X + 4, Y, 8, 8, 256, None), "misaligned"),
    ((W, X, W, 8, 8, 256, None), "overlaps"),
    ((W, X, Y, 1 << 24, 8, 65536, None), "4 GiB"),
    ((W, X, Y, 8, 1 << 20, 65536, None), "4 GiB"),
])
def test_mmq_rejects(kq, fn, args, needle):
    rc = getattr(kq.lib(), fn)(*args)
    assert rc == kq.KQ_ERR_ARG, kq.kq_last_error()
    assert needle in kq.kq_last_error()
    assert fn in kq.kq_last_error()


@pytest.mark.parametrize("args,needle", [
    ((None, X, Y, 8, 8, 256, R, 64, None), "null pointer"),
    ((W, X, Y, 8, 8, 100, R, 64, None), "k=100"),
    ((W, X, W, 8, 8, 256, R, 64, None), "overlaps"),
    ((W, X, Y, 8, 8, 256, R, -16, None), "ws_bytes=-16"),
    ((W, X, Y, 8, 8, 256, None, 64, None), "ws_bytes=64"),
])
@pytest.mark.parametrize("fn", ["kq_mmq_q4k_ws", "kq_mmq_q6k_ws"])
def test_mmq_ws_rejects(kq, fn, args, needle):
    rc = getattr(kq.lib(), fn)(*args)
    assert rc == kq.KQ_ERR_ARG, kq.kq_last_error()
    assert needle in kq.kq_last_error() and fn in kq.kq_last_error()
    assert getattr(kq.lib(), fn)(W, X, Y, 0, 8, 256, None, 0, None) == kq.KQ_OK


@pytest.mark.parametrize("m,n,k", [(-1, 8, 256), (8, -1, 256), (8, 8, 100), (8, 8, 0),
                                   (8, 65535 * 128 + 1, 256), (8, 8, 65536 + 256)])
@pytest.mark.parametrize("fn", ["kq_mmq_q4k_workspace_bytes", "kq_mmq_q6k_workspace_bytes"])
def test_mmq_workspace_bytes_rejects(kq, fn, m, n, k):
    assert getattr(kq.lib(), fn)(m, n, k) == -1
    assert fn in kq.kq_last_error()
    assert getattr(kq.lib(), fn)(0, 8, 256) == 0


@pytest.mark.parametrize("m,k", [(0, 256), (1, 256), (3, 1280), (7, 4096), (128256, 4096), (5, 18944)])
def test_split_bytes_match_the_oracle(kq, m, k):
    import oracle

    assert kq.kq_q6k_split_bytes(m, k) == oracle.q6k_split_bytes(m, k)


@pytest.mark.parametrize("m,k", [(-1, 256), (1, 0), (1, 100), (1, 65536 + 256), (1 << 31, 256)])
def test_split_bytes_rejects(kq, m, k):
    assert kq.kq_q6k_split_bytes(m, k) == -1


@pytest.mark.parametrize("args,needle", [
    ((None, X, 8, 256, None), "null pointer"),
    ((W, None, 8, 256, None), "null pointer"),
    ((W, X, 8, 100, None), "k=100"),
    ((W, X, -2, 256, None), "m=-2"),
    ((W + 2, X, 8, 256, None), "misaligned"),
    ((W, X + 8, 8, 256, None), "misaligned"),
    ((W, W + 1024, 8, 256, None), "overlaps"),
    ((W + 1024, W, 8, 256, None), "overlaps"),
])
def test_repack_rejects(kq, args, needle):
    rc = kq.lib().kq_repack_q6k(*args)
    assert rc == kq.KQ_ERR_ARG, kq.kq_last_error()
    assert needle in kq.kq_last_error() and "kq_repack_q6k" in kq.kq_last_error()


def test_split_overlap_uses_the_split_size(kq):
    # 1 x 512: 420 raw bytes, 432 in the split layout; y at W + 420 lies past
    # the raw size but inside the split buffer
    assert kq.kq_q6k_split_bytes(1, 512) == 432
    rc = kq.lib().kq_gemv_q6k_split(W, X, W + 420, None, 1, 512, 1, None)
    assert rc == kq.KQ_ERR_ARG and "overlaps" in kq.kq_last_error()
    rc = kq.lib().kq_mmq_q6k_split(W, X, W + 420, 1, 1, 512, None)
    assert rc == kq.KQ_ERR_ARG and "overlaps" in kq.kq_last_error()


def test_mmq_q6k_size_guard_uses_its_block_size(kq):
    # 100000 rows x 65536: 4.9e9 bytes of Q6_K (rejected), 3.4e9 of Q4_K
    rc = kq.lib().kq_mmq_q6k(W, X, Y, 100000, 8, 65536, None)
    assert rc == kq.KQ_ERR_ARG and "4 GiB" in kq.kq_last_error()


def test_empty_inputs_launch_nothing(kq):
    # zero rows / tokens are valid and return before any device access
    L = kq.lib()
    assert L.kq_quantize_q8_1(W, X, 0, 256, None) == kq.KQ_OK
    assert L.kq_gemv_q4k(W, X, Y, None, 0, 256, 1, None) == kq.KQ_OK
    assert L.kq_gemv_q6k(W, X, Y, None, 0, 256, 4, None) == kq.KQ_OK
    assert L.kq_mmq_q4k(W, X, Y, 0, 16, 256, None) == kq.KQ_OK
    assert L.kq_mmq_q4k(W, X, Y, 16, 0, 256, None) == kq.KQ_OK
    assert L.kq_mmq_q6k(W, X, Y, 0, 16, 256, None) == kq.KQ_OK
    assert L.kq_mmq_q6k(W, X, Y, 16, 0, 256, None) == kq.KQ_OK
    assert L.kq_mmq_q6k_split(W, X, Y, 0, 16, 256, None) == kq.KQ_OK
    assert L.kq_gemv_q6k_split(W, X, Y, None, 0, 256, 2, None) == kq.KQ_OK
    assert L.kq_repack_q6k(W, X, 0, 256, None) == kq.KQ_OK


def test_binding_raises_with_message(kq):
    with pytest.raises(kq.KQError, match="batch=9"):
        kq.kq_gemv_q4k(W, X, Y, None, 8, 256, 9, stream=0)


def test_no_gpu_means_unsupported(kq):
    """Valid arguments on a host without a gfx950 device: KQ_ERR_UNSUPPORTED,
    nothing launched.  Only meaningful where no GPU is visible."""
    import torch

    if torch.cuda.device_count() > 0:
        pytest.skip("a GPU is visible")
    rc = kq.lib().kq_gemv_q4k(W, X, Y, None, 8, 256, 1, None)
    assert rc == kq.KQ_ERR_UNSUPPORTED
    assert "kq_gemv_q4k" in kq.kq_last_error()


G = 0x100000
Q = 0x200000


@pytest.mark.parametrize("args,needle", [
    ((None, None, G, 1e-5, Y, Q, 1, 256, None), "null pointer"),
    ((X, None, None, 1e-5, Y, Q, 1, 256, None), "null pointer"),
    ((X, None, G, 1e-5, Y, None, 1, 256, None), "null pointer"),
    ((X, None, G, 1e-5, Y, Q, 1, 288, None), "n=288"),
    ((X, None, G, 1e-5, Y, Q, 1, 0, None), "n=0"),
    ((X, None, G, 1e-5, Y, Q, -1, 256, None), "rows=-1"),
    ((X + 4, None, G, 1e-5, Y, Q, 1, 256, None), "misaligned"),
    ((X, R + 4, G, 1e-5, Y, Q, 1, 256, None), "misaligned"),
    ((X, None, G, 1e-5, Y + 8, Q, 1, 256, None), "misaligned"),
    ((X, None, G, 1e-5, Y, Q + 2, 1, 256, None), "misaligned"),
    ((X, None, G, 1e-5, X, Q, 1, 256, None), "overlaps"),
    ((X, R, G, 1e-5, R, Q, 1, 256, None), "overlaps"),
    ((X, None, G, 1e-5, Y, X, 1, 256, None), "overlaps"),
    ((X, None, G, 1e-5, Y, Y + 512, 1, 256, None), "overlaps"),
])
def test_rmsnorm_rejects(kq, args, needle):
    rc = kq.lib().kq_rmsnorm_q8_1(*args)
    assert rc == kq.KQ_ERR_ARG, kq.kq_last_error()
    assert needle in kq.kq_last_error()
    assert "kq_rmsnorm_q8_1" in kq.kq_last_error()


@pytest.mark.parametrize("args,needle", [
    ((None, X, Y, Q, 1, 256, None), "null pointer"),
    ((X, None, Y, Q, 1, 256, None), "null pointer"),
    ((X, R, Y, None, 1, 256, None), "null pointer"),
    ((X, R, Y, Q, 1, 32, None), "n=32"),
    ((X, R, Y, Q, -2, 256, None), "rows=-2"),
    ((X, R, Y, Q, 1 << 24, 65536, None), "too large"),
    ((X + 4, R, Y, Q, 1, 256, None), "misaligned"),
    ((X, R, Y + 4, Q, 1, 256, None), "misaligned"),
    ((X, R, X, Q, 1, 256, None), "overlaps"),
    ((X, R, Y, R + 16, 1, 256, None), "overlaps"),
])
def test_swiglu_rejects(kq, args, needle):
    rc = kq.lib().kq_swiglu_q8_1(*args)
    assert rc == kq.KQ_ERR_ARG, kq.kq_last_error()
    assert needle in kq.kq_last_error()
    assert "kq_swiglu_q8_1" in kq.kq_last_error()


def test_producers_empty_and_no_fused_output(kq):
    L = kq.lib()
    assert L.kq_rmsnorm_q8_1(X, None, G, 1e-5, None, Q, 0, 4096, None) == kq.KQ_OK
    assert L.kq_swiglu_q8_1(X, R, None, Q, 0, 14336, None) == kq.KQ_OK


def _seg(kq, nseg, w, m, y, res, xq=X, k=256, batch=1):
    import ctypes
    n = len(w)
    W = (ctypes.c_void_p * n)(*w)
    M = (ctypes.c_int64 * n)(*m)
    Y = (ctypes.c_void_p * n)(*y)
    R = None if res is None else (ctypes.c_void_p * n)(*res)
    return kq.lib().kq_gemv_q4k_seg(nseg, W, M, Y, R, xq, k, batch, None)


@pytest.mark.parametrize("case,needle", [
    ((0, [W], [8], [Y], None), "nseg=0"),
    ((9, [W] * 9, [8] * 9, [Y + 4096 * i for i in range(9)], None), "nseg=9"),
    ((2, [W, 0], [8, 8], [Y, Y + 4096], None), "null pointer"),
    ((2, [W, W + 4], [8, 8], [Y, Y + 4096], None), "misaligned"),
    ((2, [W, W + 16 * 4096], [8, -1], [Y, Y + 4096], None), "m=-1"),
    ((2, [W, W + 16 * 4096], [8, 8], [Y, Y + 16], None), "overlaps"),
    ((2, [W, W + 16 * 4096], [8, 8], [Y, W], None), "overlaps"),
    ((2, [W, W + 16 * 4096], [8, 8], [Y, Y + 4096], [Y + 4096, 0]), "overlaps"),
])
def test_gemv_seg_rejects(kq, case, needle):
    rc = _seg(kq, *case)
    assert rc == kq.KQ_ERR_ARG, kq.kq_last_error()
    assert needle in kq.kq_last_error()


def test_gemv_seg_empty_and_null_arrays(kq):
    assert _seg(kq, 2, [W, W + 16 * 4096], [0, 0], [Y, Y + 4096], None) == kq.KQ_OK
    assert _seg(kq, 2, [0, 0], [0, 0], [0, 0], None) == kq.KQ_OK
    rc = _seg(kq, 1, [W], [0], [Y], None, k=100)
    assert rc == kq.KQ_ERR_ARG and "k=100" in kq.kq_last_error()
    rc = kq.lib().kq_gemv_q4k_seg(1, None, None, None, None, X, 256, 1, None)
    assert rc == kq.KQ_ERR_ARG and "null array" in kq.kq_last_error()


@pytest.mark.parametrize("nbytes,grid,loads,words", [
    (16, 0, 8, 4), (32768, 0, 8, 4), (32784, 0, 8, 8), (2 << 30, 0, 8, 4 * 65536),
    (2 << 30, 512, 16, 4 * 512), (2 << 30, 0, 32, 4 * 16384), (32784, 100, 4, 4 * 3),
    (16, 7, 32, 4)])
def test_read_probe_words(kq, nbytes, grid, loads, words):
    assert kq.kq_read_probe_words(nbytes, grid, loads) == words


@pytest.mark.parametrize("nbytes,grid,loads", [(0, 0, 8), (-16, 0, 8), (8, 0, 8), (1 << 40, 0, 8),
                                               (4096, -1, 8), (4096, 0, 12), (4096, 1 << 31, 8)])
def test_read_probe_words_rejects(kq, nbytes, grid, loads):
    assert kq.kq_read_probe_words(nbytes, grid, loads) == -1


@pytest.mark.parametrize("args,needle", [
    ((None, 4096, Y, 0, 8, None), "null pointer"),
    ((W, 4096, None, 0, 8, None), "null pointer"),
    ((W, 0, Y, 0, 8, None), "nbytes=0"),
    ((W, 4100, Y, 0, 8, None), "nbytes=4100"),
    ((W, 4096, Y, 0, 7, None), "loads=7"),
    ((W, 4096, Y, -2, 8, None), "grid=-2"),
    ((W + 8, 4096, Y, 0, 8, None), "misaligned"),
    ((W, 4096, Y + 2, 0, 8, None), "misaligned"),
    ((W, 4096, W + 64, 0, 8, None), "overlaps"),
])
def test_read_probe_rejects(kq, args, needle):
    rc = kq.lib().kq_read_probe(*args)
    assert rc == kq.KQ_ERR_ARG, kq.kq_last_error()
    assert needle in kq.kq_last_error() and "kq_read_probe" in kq.kq_last_error()
