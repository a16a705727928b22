"""Python binding of libkq, the k-quant matmul for AMD MI355X (gfx950).

Thin ``ctypes`` marshalling over the C ABI declared in ``include/kq.h``:
every function below has the name of a C entry point, turns tensors into
device pointers and the current torch stream into a ``hipStream_t``, calls
the library and raises :class:`KQError` on a non-zero status.  All
arithmetic runs in the library's gfx950 kernels; there is no other path.

PyTorch (ROCm build) supplies device memory and streams only.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkq.so")

KQ_OK = 0
KQ_ERR_ARG = -1
KQ_ERR_UNSUPPORTED = -2
KQ_ERR_HIP = -3

Q4K_BYTES = 144
Q6K_BYTES = 210
Q81_BYTES = 36


class KQError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"[status {status}] {message}")
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libkq.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is missing: build it with `python -m q6_q8_matmul_amd.build` "
                "(there is no fallback implementation)")
        L = ctypes.CDLL(LIB_PATH)
        p, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
        L.kq_quantize_q8_1.argtypes = [p, p, i64, i64, p]
        L.kq_gemv_q4k.argtypes = [p, p, p, p, i64, i64, i32, p]
        L.kq_gemv_q6k.argtypes = [p, p, p, p, i64, i64, i32, p]
        L.kq_mmq_q4k.argtypes = [p, p, p, i64, i64, i64, p]
        L.kq_mmq_q6k.argtypes = [p, p, p, i64, i64, i64, p]
        L.kq_mmq_q6k_split.argtypes = [p, p, p, i64, i64, i64, p]
        L.kq_mmq_q6k_ws.argtypes = [p, p, p, i64, i64, i64, p, i64, p]
        L.kq_mmq_q4k_ws.argtypes = [p, p, p, i64, i64, i64, p, i64, p]
        L.kq_mmq_q4k_workspace_bytes.argtypes = [i64, i64, i64]
        L.kq_mmq_q4k_workspace_bytes.restype = i64
        L.kq_mmq_q6k_noalloc.argtypes = [p, p, p, i64, i64, i64, p]
        L.kq_mmq_q6k_workspace_bytes.argtypes = [i64, i64, i64]
        L.kq_mmq_q6k_workspace_bytes.restype = i64
        L.kq_gemv_q6k_split.argtypes = [p, p, p, p, i64, i64, i32, p]
        L.kq_repack_q6k.argtypes = [p, p, i64, i64, p]
        L.kq_q6k_split_bytes.argtypes = [i64, i64]
        L.kq_q6k_split_bytes.restype = i64
        L.kq_rmsnorm_q8_1.argtypes = [p, p, p, ctypes.c_float, p, p, i64, i64, p]
        L.kq_swiglu_q8_1.argtypes = [p, p, p, p, i64, i64, p]
        L.kq_gemv_q4k_seg.argtypes = [i32, p, p, p, p, p, i64, i32, p]
        L.kq_read_probe.argtypes = [p, i64, p, i64, i32, p]
        L.kq_read_probe_words.argtypes = [i64, i64, i32]
        L.kq_read_probe_words.restype = i64
        for fn in (L.kq_quantize_q8_1, L.kq_gemv_q4k, L.kq_gemv_q6k, L.kq_mmq_q4k,
                   L.kq_mmq_q6k, L.kq_mmq_q6k_split, L.kq_mmq_q6k_ws, L.kq_mmq_q4k_ws, L.kq_mmq_q6k_noalloc, L.kq_gemv_q6k_split, L.kq_repack_q6k,
                   L.kq_rmsnorm_q8_1, L.kq_swiglu_q8_1, L.kq_gemv_q4k_seg, L.kq_read_probe):
            fn.restype = ctypes.c_int
        L.kq_last_error.argtypes = []
        L.kq_last_error.restype = ctypes.c_char_p
        L.kq_abi_version.argtypes = []
        L.kq_abi_version.restype = ctypes.c_int
        _lib = L
    return _lib


def _ptr(t):
    """Device address of a tensor (or pass an int/None through)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        import torch

        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(rc: int) -> None:
    if rc != KQ_OK:
        raise KQError(rc, kq_last_error())


# ------------------------------------------------------------- the C ABI ----

def kq_last_error() -> str:
    return lib().kq_last_error().decode()


def kq_abi_version() -> int:
    return int(lib().kq_abi_version())


def kq_quantize_q8_1(x, xq, rows: int, k: int, stream=None) -> None:
    _check(lib().kq_quantize_q8_1(_ptr(x), _ptr(xq), rows, k, _stream(stream)))


def kq_gemv_q4k(w, xq, y, residual, m: int, k: int, batch: int, stream=None) -> None:
    _check(lib().kq_gemv_q4k(_ptr(w), _ptr(xq), _ptr(y), _ptr(residual), m, k, batch,
                             _stream(stream)))


def kq_gemv_q6k(w, xq, y, residual, m: int, k: int, batch: int, stream=None) -> None:
    _check(lib().kq_gemv_q6k(_ptr(w), _ptr(xq), _ptr(y), _ptr(residual), m, k, batch,
                             _stream(stream)))


def kq_mmq_q4k(w, xq, y, m: int, n: int, k: int, stream=None) -> None:
    _check(lib().kq_mmq_q4k(_ptr(w), _ptr(xq), _ptr(y), m, n, k, _stream(stream)))


def kq_mmq_q6k(w, xq, y, m: int, n: int, k: int, stream=None) -> None:
    _check(lib().kq_mmq_q6k(_ptr(w), _ptr(xq), _ptr(y), m, n, k, _stream(stream)))


def kq_mmq_q4k_workspace_bytes(m: int, n: int, k: int) -> int:
    v = int(lib().kq_mmq_q4k_workspace_bytes(m, n, k))
    if v < 0:
        raise KQError(KQ_ERR_ARG, kq_last_error())
    return v


def kq_mmq_q4k_ws(w, xq, y, m: int, n: int, k: int, ws, ws_bytes: int, stream=None) -> None:
    _check(lib().kq_mmq_q4k_ws(_ptr(w), _ptr(xq), _ptr(y), m, n, k, _ptr(ws), ws_bytes,
                               _stream(stream)))


def kq_mmq_q6k_workspace_bytes(m: int, n: int, k: int) -> int:
    v = int(lib().kq_mmq_q6k_workspace_bytes(m, n, k))
    if v < 0:
        raise KQError(KQ_ERR_ARG, kq_last_error())
    return v


def kq_mmq_q6k_ws(w, xq, y, m: int, n: int, k: int, ws, ws_bytes: int, stream=None) -> None:
    _check(lib().kq_mmq_q6k_ws(_ptr(w), _ptr(xq), _ptr(y), m, n, k, _ptr(ws), ws_bytes,
                               _stream(stream)))


def kq_mmq_q6k_noalloc(w, xq, y, m: int, n: int, k: int, stream=None) -> None:
    _check(lib().kq_mmq_q6k_noalloc(_ptr(w), _ptr(xq), _ptr(y), m, n, k, _stream(stream)))


def kq_mmq_q6k_split(wr, xq, y, m: int, n: int, k: int, stream=None) -> None:
    _check(lib().kq_mmq_q6k_split(_ptr(wr), _ptr(xq), _ptr(y), m, n, k, _stream(stream)))


def kq_gemv_q6k_split(wr, xq, y, residual, m: int, k: int, batch: int, stream=None) -> None:
    _check(lib().kq_gemv_q6k_split(_ptr(wr), _ptr(xq), _ptr(y), _ptr(residual), m, k, batch,
                                   _stream(stream)))


def kq_repack_q6k(w, wr, m: int, k: int, stream=None) -> None:
    _check(lib().kq_repack_q6k(_ptr(w), _ptr(wr), m, k, _stream(stream)))


def kq_q6k_split_bytes(m: int, k: int) -> int:
    return int(lib().kq_q6k_split_bytes(m, k))


def kq_read_probe_words(nbytes: int, grid: int = 0, loads: int = 8) -> int:
    return int(lib().kq_read_probe_words(nbytes, grid, loads))


def kq_read_probe(p, nbytes: int, out, grid: int = 0, loads: int = 8, stream=None) -> None:
    _check(lib().kq_read_probe(_ptr(p), nbytes, _ptr(out), grid, loads, _stream(stream)))


def kq_gemv_q4k_seg(w, m, y, residual, xq, k: int, batch: int, stream=None) -> None:
    """Segmented Q4_K GEMV: w, m, y (and residual, or None) are sequences of
    equal length; their entries are tensors / device addresses / row counts."""
    n = len(w)
    W = (ctypes.c_void_p * n)(*[_ptr(t) for t in w])
    M = (ctypes.c_int64 * n)(*[int(v) for v in m])
    Y = (ctypes.c_void_p * n)(*[_ptr(t) for t in y])
    R = None if residual is None else (ctypes.c_void_p * n)(*[_ptr(t) for t in residual])
    _check(lib().kq_gemv_q4k_seg(n, W, M, Y, R, _ptr(xq), k, batch, _stream(stream)))


def kq_rmsnorm_q8_1(x, res, g, eps: float, y, xq, rows: int, n: int, stream=None) -> None:
    _check(lib().kq_rmsnorm_q8_1(_ptr(x), _ptr(res), _ptr(g), ctypes.c_float(eps), _ptr(y),
                                 _ptr(xq), rows, n, _stream(stream)))


def kq_swiglu_q8_1(gate, up, y, xq, rows: int, n: int, stream=None) -> None:
    _check(lib().kq_swiglu_q8_1(_ptr(gate), _ptr(up), _ptr(y), _ptr(xq), rows, n,
                                _stream(stream)))


# ------------------------------------------- allocating conveniences -------
# These allocate the output with torch and call the entry point above.

def _require_cuda(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("tensors must live on the GPU")


def quantize_q8_1(x, stream=None):
    """f32 ``[rows, k]`` -> uint8 ``[rows, k/32*36]`` q8_1 tensor."""
    import torch

    _require_cuda(x)
    if x.dtype != torch.float32 or not x.is_contiguous():
        raise ValueError("x must be a contiguous float32 tensor")
    rows, k = x.shape
    xq = torch.empty((rows, (k // 32) * Q81_BYTES), dtype=torch.uint8, device=x.device)
    kq_quantize_q8_1(x, xq, rows, k, stream)
    return xq


def gemv_q4k(w, xq, m: int, k: int, batch: int, residual=None, out=None, stream=None):
    import torch

    _require_cuda(w, xq, residual)
    y = out if out is not None else torch.empty((batch, m), dtype=torch.float32, device=w.device)
    kq_gemv_q4k(w, xq, y, residual, m, k, batch, stream)
    return y


def gemv_q6k(w, xq, m: int, k: int, batch: int, residual=None, out=None, stream=None):
    import torch

    _require_cuda(w, xq, residual)
    y = out if out is not None else torch.empty((batch, m), dtype=torch.float32, device=w.device)
    kq_gemv_q6k(w, xq, y, residual, m, k, batch, stream)
    return y


def mmq_q4k(w, xq, m: int, n: int, k: int, out=None, stream=None):
    import torch

    _require_cuda(w, xq)
    y = out if out is not None else torch.empty((n, m), dtype=torch.float32, device=w.device)
    kq_mmq_q4k(w, xq, y, m, n, k, stream)
    return y


def repack_q6k(w, m: int, k: int, stream=None):
    """Raw Q6_K weight (uint8 device tensor) -> a new tensor in the split layout."""
    import torch

    _require_cuda(w)
    nbytes = kq_q6k_split_bytes(m, k)
    if nbytes < 0:
        raise KQError(f"repack_q6k: invalid m={m} or k={k}")
    wr = torch.empty(nbytes, dtype=torch.uint8, device=w.device)
    kq_repack_q6k(w, wr, m, k, stream)
    return wr


def gemv_q6k_split(wr, xq, m: int, k: int, batch: int, residual=None, out=None, stream=None):
    import torch

    _require_cuda(wr, xq, residual)
    y = out if out is not None else torch.empty((batch, m), dtype=torch.float32, device=wr.device)
    kq_gemv_q6k_split(wr, xq, y, residual, m, k, batch, stream)
    return y


def mmq_q6k_split(wr, xq, m: int, n: int, k: int, out=None, stream=None):
    import torch

    _require_cuda(wr, xq)
    y = out if out is not None else torch.empty((n, m), dtype=torch.float32, device=wr.device)
    kq_mmq_q6k_split(wr, xq, y, m, n, k, stream)
    return y


def mmq_q4k_ws(w, xq, m: int, n: int, k: int, ws=None, out=None, stream=None):
    """kq_mmq_q4k_ws with a workspace tensor of the size the split needs
    (allocated here by torch when `ws` is None)."""
    import torch

    _require_cuda(w, xq)
    y = out if out is not None else torch.empty((n, m), dtype=torch.float32, device=w.device)
    if ws is None:
        nb = kq_mmq_q4k_workspace_bytes(m, n, k)
        ws = torch.empty(max(nb, 16), dtype=torch.uint8, device=w.device)
    kq_mmq_q4k_ws(w, xq, y, m, n, k, ws, ws.numel() * ws.element_size(), stream)
    return y


def mmq_q6k_ws(w, xq, m: int, n: int, k: int, ws=None, out=None, stream=None):
    """kq_mmq_q6k_ws with a workspace tensor of the size the split needs
    (allocated here by torch when `ws` is None)."""
    import torch

    _require_cuda(w, xq)
    y = out if out is not None else torch.empty((n, m), dtype=torch.float32, device=w.device)
    if ws is None:
        nb = kq_mmq_q6k_workspace_bytes(m, n, k)
        ws = torch.empty(max(nb, 16), dtype=torch.uint8, device=w.device)
    kq_mmq_q6k_ws(w, xq, y, m, n, k, ws, ws.numel() * ws.element_size(), stream)
    return y


def mmq_q6k(w, xq, m: int, n: int, k: int, out=None, stream=None):
    import torch

    _require_cuda(w, xq)
    y = out if out is not None else torch.empty((n, m), dtype=torch.float32, device=w.device)
    kq_mmq_q6k(w, xq, y, m, n, k, stream)
    return y


def rmsnorm_q8_1(x, g, eps: float, residual=None, want_y: bool = True, stream=None):
    """RMSNorm(x [+ residual]) * g -> (y f32 [rows, n] or None, q8_1 uint8)."""
    import torch

    _require_cuda(x, g, residual)
    rows, n = x.shape
    xq = torch.empty((rows, (n // 32) * Q81_BYTES), dtype=torch.uint8, device=x.device)
    y = torch.empty((rows, n), dtype=torch.float32, device=x.device) if want_y else None
    kq_rmsnorm_q8_1(x, residual, g, eps, y, xq, rows, n, stream)
    return y, xq


def swiglu_q8_1(gate, up, want_y: bool = True, stream=None):
    """silu(gate) * up -> (y f32 [rows, n] or None, q8_1 uint8)."""
    import torch

    _require_cuda(gate, up)
    rows, n = gate.shape
    xq = torch.empty((rows, (n // 32) * Q81_BYTES), dtype=torch.uint8, device=gate.device)
    y = torch.empty((rows, n), dtype=torch.float32, device=gate.device) if want_y else None
    kq_swiglu_q8_1(gate, up, y, xq, rows, n, stream)
    return y, xq


def gemv_q4k_seg(ws, ms, xq, k: int, batch: int, residuals=None, outs=None, stream=None):
    """Several Q4_K GEMVs sharing one q8_1 activation in one launch; returns
    the list of outputs f32 [batch, m[s]]."""
    import torch

    _require_cuda(xq, *ws)
    ys = outs if outs is not None else [
        torch.empty((batch, int(m)), dtype=torch.float32, device=xq.device) for m in ms]
    kq_gemv_q4k_seg(ws, ms, ys, residuals, xq, k, batch, stream)
    return ys
