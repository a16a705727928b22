"""CPU oracle for the k-quant matmul -- TEST INFRASTRUCTURE ONLY.

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The HIP library never calls it and
shares no code with it.

``kq_oracle.c`` holds the arithmetic (see its header for what each routine
computes and which passage it follows); this module builds it with ``gcc``
and wraps it with ``ctypes``.  ``exact.py`` is an independent exact-rational
checker for tiny inputs.

Parity status: every function here is pinned by tests under ``tests/``
(hand-worked values in ``tests/golden``, closed forms, the exact-rational
checker, ``numpy``'s binary16 conversion).  The Q4_K/Q6_K *bit positions* are
the public GGUF layout; the pages give only block sizes and field lists, so
compatibility with real GGUF files is parity unpinned by the pages.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kq_oracle.c")
_LIB = os.path.join(_HERE, "libkq_oracle.so")

WT_Q4K = 0
WT_Q6K = 1
_WT = {"q4k": WT_Q4K, "q6k": WT_Q6K}

CFLAGS = ["-O2", "-fno-fast-math", "-ffp-contract=off", "-fopenmp", "-shared", "-fPIC",
          "-Wall", "-Wextra"]


def build(force: bool = True) -> str:
    """Compile ``kq_oracle.c`` into ``libkq_oracle.so`` (always, when force)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", *CFLAGS, "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _bind(L: ctypes.CDLL) -> ctypes.CDLL:
    p, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    sig = {
        "kqo_quantize_q8_1": ([p, p, i64, i64], None),
        "kqo_dequant_q8_1": ([p, p, i64, i64], None),
        "kqo_dequant": ([i32, p, p, i64, i64], i32),
        "kqo_matmul": ([i32, p, p, p, i64, i64, i64, p, p], i32),
        "kqo_matmul_pairs": ([i32, p, p, p, i64, i64, i64, p, p, i64, p, p], i32),
        "kqo_matmul_factored": ([i32, p, p, p, i64, i64, i64, p], i32),
        "kqo_f32_to_f16_array": ([p, p, i64], None),
        "kqo_f16_to_f32_array": ([p, p, i64], None),
        "kqo_exp_array": ([p, p, i64], None),
        "kqo_silu_array": ([p, p, i64], None),
        "kqo_rms_sumsq": ([p, i64], ctypes.c_float),
        "kqo_rmsnorm_q8_1": ([p, p, p, ctypes.c_float, p, p, i64, i64], None),
        "kqo_swiglu_q8_1": ([p, p, p, p, i64, i64], None),
        "kqo_set_threads": ([i32], None),
        "kqo_max_threads": ([], i32),
    }
    for name, (args, res) in sig.items():
        fn = getattr(L, name)
        fn.argtypes = args
        fn.restype = res
    return L


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=True)
        _lib = _bind(ctypes.CDLL(_LIB))
    return _lib


class using_library:
    """Temporarily route every wrapper below through another build of the
    oracle source (the mutation tests compile deliberately broken copies)."""

    def __init__(self, path: str):
        self.path = path

    def __enter__(self):
        global _lib
        self.saved = _lib
        _lib = _bind(ctypes.CDLL(self.path))
        return self

    def __exit__(self, *exc):
        global _lib
        _lib = self.saved
        return False


def _ptr(a: np.ndarray | None):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def set_threads(n: int) -> None:
    lib().kqo_set_threads(int(n))


def max_threads() -> int:
    return int(lib().kqo_max_threads())


# ------------------------------------------------------------------ f16 ----

def f32_to_f16_bits(x) -> np.ndarray:
    a = np.ascontiguousarray(np.asarray(x, dtype=np.float32).ravel())
    out = np.empty(a.size, dtype=np.uint16)
    lib().kqo_f32_to_f16_array(_ptr(a), _ptr(out), a.size)
    return out


def f16_bits_to_f32(h) -> np.ndarray:
    a = np.ascontiguousarray(np.asarray(h, dtype=np.uint16).ravel())
    out = np.empty(a.size, dtype=np.float32)
    lib().kqo_f16_to_f32_array(_ptr(a), _ptr(out), a.size)
    return out


# ----------------------------------------------------------------- q8_1 ----

def quantize_q8_1(x: np.ndarray) -> np.ndarray:
    """f32 ``[rows, k]`` -> ``uint8[rows, (k/32)*36]`` q8_1 blocks."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if x.ndim == 1:
        x = x[None, :]
    rows, k = x.shape
    if k % 32:
        raise ValueError("k must be a multiple of 32")
    out = np.empty((rows, (k // 32) * 36), dtype=np.uint8)
    lib().kqo_quantize_q8_1(_ptr(x), _ptr(out), rows, k)
    return out


def dequant_q8_1(xq: np.ndarray, rows: int, k: int) -> np.ndarray:
    xq = np.ascontiguousarray(xq, dtype=np.uint8)
    assert xq.size == rows * (k // 32) * 36
    out = np.empty((rows, k), dtype=np.float32)
    lib().kqo_dequant_q8_1(_ptr(xq), _ptr(out), rows, k)
    return out


# ------------------------------------------------------------ producers ----

def exp_f32(a) -> np.ndarray:
    """The producers' exponential e(a) (Cody-Waite reduction, degree-7 Taylor)."""
    a = np.ascontiguousarray(np.asarray(a, dtype=np.float32).ravel())
    out = np.empty_like(a)
    lib().kqo_exp_array(_ptr(a), _ptr(out), a.size)
    return out


def silu_f32(t) -> np.ndarray:
    t = np.ascontiguousarray(np.asarray(t, dtype=np.float32).ravel())
    out = np.empty_like(t)
    lib().kqo_silu_array(_ptr(t), _ptr(out), t.size)
    return out


def rms_sumsq(h) -> float:
    """Sum of squares of one row in the RMSNorm reduction order (n % 256 == 0)."""
    h = np.ascontiguousarray(np.asarray(h, dtype=np.float32).ravel())
    if h.size % 256:
        raise ValueError("n must be a multiple of 256")
    return float(lib().kqo_rms_sumsq(_ptr(h), h.size))


def _rows2(a):
    a = np.ascontiguousarray(a, dtype=np.float32)
    return a[None, :] if a.ndim == 1 else a


def rmsnorm_q8_1(x, g, eps: float, residual=None):
    """RMSNorm (of x + residual when given) times g, and its q8_1 blocks.
    Returns (y f32 [rows, n], xq uint8 [rows, n/32*36])."""
    x = _rows2(x)
    rows, n = x.shape
    if n % 256:
        raise ValueError("n must be a multiple of 256")
    g = np.ascontiguousarray(g, dtype=np.float32).ravel()
    assert g.size == n
    res = None if residual is None else _rows2(residual)
    if res is not None:
        assert res.shape == x.shape
    y = np.empty((rows, n), dtype=np.float32)
    xq = np.empty((rows, (n // 32) * 36), dtype=np.uint8)
    lib().kqo_rmsnorm_q8_1(_ptr(x), _ptr(res), _ptr(g), ctypes.c_float(eps), _ptr(y), _ptr(xq),
                           rows, n)
    return y, xq


def swiglu_q8_1(gate, up):
    """silu(gate) * up and its q8_1 blocks.  Returns (y, xq)."""
    gate, up = _rows2(gate), _rows2(up)
    assert gate.shape == up.shape
    rows, n = gate.shape
    if n % 32:
        raise ValueError("n must be a multiple of 32")
    y = np.empty((rows, n), dtype=np.float32)
    xq = np.empty((rows, (n // 32) * 36), dtype=np.uint8)
    lib().kqo_swiglu_q8_1(_ptr(gate), _ptr(up), _ptr(y), _ptr(xq), rows, n)
    return y, xq


# -------------------------------------------------------------- weights ----

def dequant(kind: str, w: np.ndarray, m: int, k: int) -> np.ndarray:
    """GGUF-order f32 dequantisation of a Q4_K / Q6_K matrix -> f32 ``[m, k]``."""
    w = np.ascontiguousarray(w, dtype=np.uint8)
    out = np.empty((m, k), dtype=np.float32)
    rc = lib().kqo_dequant(_WT[kind], _ptr(w), _ptr(out), m, k)
    if rc:
        raise ValueError(f"kqo_dequant rc={rc}")
    return out


# Split Q6_K layout (cajeta "One model, start to last token" 2, residency
# step 3: a Q6_K weight is split into a scale prefix and 208-byte bodies so the
# kernels read it with aligned 16-byte loads).  Reading: the prefix is the
# f16 super-scale d of every superblock g = row * S + s, in that order, zero
# padded to a multiple of 16 bytes; body g is the superblock's bytes 0..207
# (ql, qh and the 16 int8 scales) unchanged.  A byte permutation: no value
# changes.

def q6k_split_bytes(m: int, k: int) -> int:
    """Size of the split layout of an ``m x k`` Q6_K matrix."""
    g = m * (k // 256)
    return (2 * g + 15) // 16 * 16 + 208 * g


def q6k_split(w: np.ndarray, m: int, k: int) -> np.ndarray:
    """Raw Q6_K ``uint8[m, (k/256)*210]`` -> the split layout (flat uint8)."""
    g = m * (k // 256)
    raw = np.ascontiguousarray(w, dtype=np.uint8).reshape(g, 210)
    prefix = (2 * g + 15) // 16 * 16
    out = np.zeros(prefix + 208 * g, dtype=np.uint8)
    out[: 2 * g] = raw[:, 208:210].reshape(-1)
    out[prefix:] = raw[:, :208].reshape(-1)
    return out


def q6k_unsplit(wr: np.ndarray, m: int, k: int) -> np.ndarray:
    """The split layout -> raw Q6_K ``uint8[m, (k/256)*210]``."""
    g = m * (k // 256)
    wr = np.ascontiguousarray(wr, dtype=np.uint8).reshape(-1)
    prefix = (2 * g + 15) // 16 * 16
    raw = np.empty((g, 210), dtype=np.uint8)
    raw[:, 208:210] = wr[: 2 * g].reshape(g, 2)
    raw[:, :208] = wr[prefix: prefix + 208 * g].reshape(g, 208)
    return raw.reshape(m, (k // 256) * 210)


# --------------------------------------------------------------- matmul ----

def matmul(kind: str, w: np.ndarray, xq: np.ndarray, m: int, n: int, k: int,
           residual: np.ndarray | None = None):
    """Oracle ``y[n, m]`` (f64) and tolerance denominators ``den[n, m]``."""
    w = np.ascontiguousarray(w, dtype=np.uint8)
    xq = np.ascontiguousarray(xq, dtype=np.uint8)
    res = None if residual is None else np.ascontiguousarray(residual, dtype=np.float32)
    if res is not None:
        assert res.shape == (n, m)
    y = np.empty((n, m), dtype=np.float64)
    den = np.empty((n, m), dtype=np.float64)
    rc = lib().kqo_matmul(_WT[kind], _ptr(w), _ptr(xq), _ptr(res), m, n, k, _ptr(y), _ptr(den))
    if rc:
        raise RuntimeError(f"kqo_matmul rc={rc}")
    return y, den


def matmul_pairs(kind: str, w: np.ndarray, xq: np.ndarray, m: int, n: int, k: int,
                 tok, row, residual: np.ndarray | None = None):
    """The same definition for the (tok[p], row[p]) outputs only."""
    w = np.ascontiguousarray(w, dtype=np.uint8)
    xq = np.ascontiguousarray(xq, dtype=np.uint8)
    tok = np.ascontiguousarray(tok, dtype=np.int64)
    row = np.ascontiguousarray(row, dtype=np.int64)
    res = None if residual is None else np.ascontiguousarray(residual, dtype=np.float32)
    y = np.empty(tok.size, dtype=np.float64)
    den = np.empty(tok.size, dtype=np.float64)
    rc = lib().kqo_matmul_pairs(_WT[kind], _ptr(w), _ptr(xq), _ptr(res), m, n, k,
                                _ptr(tok), _ptr(row), tok.size, _ptr(y), _ptr(den))
    if rc:
        raise RuntimeError(f"kqo_matmul_pairs rc={rc}")
    return y, den


def matmul_factored(kind: str, w: np.ndarray, xq: np.ndarray, m: int, n: int, k: int,
                    residual: np.ndarray | None = None) -> np.ndarray:
    """Integer-factored second form of the same output (identity check)."""
    w = np.ascontiguousarray(w, dtype=np.uint8)
    xq = np.ascontiguousarray(xq, dtype=np.uint8)
    res = None if residual is None else np.ascontiguousarray(residual, dtype=np.float32)
    y = np.empty((n, m), dtype=np.float64)
    rc = lib().kqo_matmul_factored(_WT[kind], _ptr(w), _ptr(xq), _ptr(res), m, n, k, _ptr(y))
    if rc:
        raise RuntimeError(f"kqo_matmul_factored rc={rc}")
    return y


def tolerance_ok(y_test: np.ndarray, y_ref: np.ndarray, den: np.ndarray, rtol: float = 1e-5):
    """The pass rule |y_test - y_ref| <= rtol * den, elementwise.

    Returns (all_ok, max_ratio) where max_ratio = max |y_test - y_ref| / den
    (an output with den == 0 must match exactly).
    """
    y_test = np.asarray(y_test, dtype=np.float64)
    diff = np.abs(y_test - y_ref)
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = np.where(den > 0, diff / np.where(den > 0, den, 1.0),
                         np.where(diff == 0, 0.0, np.inf))
    ok = bool(np.all(diff <= rtol * den))
    return ok, float(ratio.max()) if ratio.size else 0.0
