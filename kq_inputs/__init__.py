"""Seeded synthetic inputs for the k-quant matmul workloads.

This module only draws random numbers and places them at the byte offsets of
the block formats.  It performs none of the method's arithmetic (no unpacking,
no dequantisation, no quantisation), so both the CPU oracle and the HIP path
can take their inputs from it without sharing any computation.

Formats (byte layouts of one block, little-endian):

* Q4_K superblock, 256 values, 144 bytes: f16 ``d`` at 0, f16 ``dmin`` at 2,
  12 bytes of packed 6-bit scales and mins at 4..15, 128 bytes of 4-bit codes
  at 16..143 (leone-cuda "CUDA kernel design": Q4_K repack paragraph; minfer
  "The CUDA backend" section 2.3).
* Q6_K superblock, 256 values, 210 bytes: ``ql`` 128 bytes at 0, ``qh`` 64
  bytes at 128, 16 int8 scales at 192, f16 ``d`` at 208 (minfer "The CUDA
  backend" section 3.2.2 gives the 210-byte size).

Value distributions of the workloads: 4-bit codes uniform in 0..15, six-bit
scales and mins uniform in 0..63, ``d``/``dmin`` = f16(|N(0,1)| * 2^-8),
Q6_K ``ql``/``qh`` uniform bytes, Q6_K scales uniform in -32..31,
activations and residuals N(0,1) in f32, normalisation gains 1 + 0.1 N(0,1).

Uniform random bytes realise the Q4_K code and scale distributions exactly:
every bit of the 128 code bytes belongs to exactly one 4-bit code, and every
bit of the 12 scale bytes belongs to exactly one of the sixteen 6-bit fields,
so independent uniform bytes give independent uniform fields.

Every tensor is drawn from its own stream
``numpy.random.default_rng(SeedSequence([seed, tensor_id]))``.
"""
from __future__ import annotations

import numpy as np

QK_K = 256
Q4K_BYTES = 144
Q6K_BYTES = 210
Q81_BYTES = 36
Q81_VALUES = 32


def _rng(seed: int, tensor_id: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([int(seed), int(tensor_id)]))


def _f16_scale_field(rng: np.random.Generator, shape) -> np.ndarray:
    """f16(|N(0,1)| * 2^-8) as raw little-endian uint16 bit patterns."""
    v = np.abs(rng.standard_normal(shape)) * 2.0 ** -8
    return v.astype(np.float16).view(np.uint16)


def q4k_weights(seed: int, tensor_id: int, m: int, k: int) -> np.ndarray:
    """Random Q4_K matrix, ``uint8[m, (k/256)*144]``, row-major superblocks."""
    assert k % QK_K == 0 and m >= 0
    s = k // QK_K
    rng = _rng(seed, tensor_id)
    w = rng.integers(0, 256, size=(m, s, Q4K_BYTES), dtype=np.uint8)
    d = _f16_scale_field(rng, (m, s))
    dmin = _f16_scale_field(rng, (m, s))
    w[:, :, 0:2] = d.view(np.uint8).reshape(m, s, 2)
    w[:, :, 2:4] = dmin.view(np.uint8).reshape(m, s, 2)
    return w.reshape(m, s * Q4K_BYTES)


def q6k_weights(seed: int, tensor_id: int, m: int, k: int) -> np.ndarray:
    """Random Q6_K matrix, ``uint8[m, (k/256)*210]``, row-major superblocks."""
    assert k % QK_K == 0 and m >= 0
    s = k // QK_K
    rng = _rng(seed, tensor_id)
    w = np.empty((m, s, Q6K_BYTES), dtype=np.uint8)
    w[:, :, 0:192] = rng.integers(0, 256, size=(m, s, 192), dtype=np.uint8)
    w[:, :, 192:208] = rng.integers(-32, 32, size=(m, s, 16), dtype=np.int8).view(np.uint8)
    w[:, :, 208:210] = _f16_scale_field(rng, (m, s)).view(np.uint8).reshape(m, s, 2)
    return w.reshape(m, s * Q6K_BYTES)


def activations(seed: int, tensor_id: int, rows: int, k: int) -> np.ndarray:
    """f32 N(0,1) activations, ``float32[rows, k]``."""
    return _rng(seed, tensor_id).standard_normal((rows, k), dtype=np.float32)


def residual(seed: int, tensor_id: int, rows: int, m: int) -> np.ndarray:
    """f32 N(0,1) residual stream, ``float32[rows, m]``."""
    return _rng(seed, tensor_id).standard_normal((rows, m), dtype=np.float32)


def gain(seed: int, tensor_id: int, rows: int, n: int) -> np.ndarray:
    """f32 normalisation gain 1 + 0.1*N(0,1), ``float32[rows, n]`` (rows = 1)."""
    v = 1.0 + 0.1 * _rng(seed, tensor_id).standard_normal((rows, n))
    return v.astype(np.float32)


# --------------------------------------------------------------------------
# The five workloads.  Each op names its weight tensor, its activation tensor
# and (optionally) a residual tensor.  Tensor ids are the positions in
# ``tensors``; the seed is the workload index.
# --------------------------------------------------------------------------

WORKLOADS = {
    0: dict(
        name="tiny_q4k_gemv_256x1024_b1",
        tensors=[("w", "q4k", 256, 1024), ("x", "act", 1, 1024)],
        ops=[dict(op="gemv_q4k", label="w", w="w", x="x", m=256, k=1024, batch=1)],
    ),
    1: dict(
        name="llama3_8b_decode_gemv_q4k_b1",
        tensors=[
            ("attn_out", "q4k", 4096, 4096),
            ("gate", "q4k", 14336, 4096),
            ("up", "q4k", 14336, 4096),
            ("down", "q4k", 4096, 14336),
            ("x_attn", "act", 1, 4096),
            ("x_ffn", "act", 1, 4096),
            ("x_down", "act", 1, 14336),
        ],
        ops=[
            dict(op="gemv_q4k", label="attn_out", w="attn_out", x="x_attn", m=4096, k=4096, batch=1),
            dict(op="gemv_q4k", label="gate", w="gate", x="x_ffn", m=14336, k=4096, batch=1),
            dict(op="gemv_q4k", label="up", w="up", x="x_ffn", m=14336, k=4096, batch=1),
            dict(op="gemv_q4k", label="down", w="down", x="x_down", m=4096, k=14336, batch=1),
        ],
        # gate and up share one q8_1 activation; laid out as one contiguous
        # 28672-row matrix they are one launch
        bench_ops=[
            dict(op="gemv_q4k", label="attn_out", w="attn_out", x="x_attn", m=4096, k=4096, batch=1),
            dict(op="gemv_q4k", label="gate|up", w=["gate", "up"], x="x_ffn", m=28672, k=4096, batch=1),
            dict(op="gemv_q4k", label="down", w="down", x="x_down", m=4096, k=14336, batch=1),
        ],
    ),
    2: dict(
        name="llama3_8b_decode_gemv_q4k_b4",
        tensors=[
            ("qkv", "q4k", 6144, 4096),
            ("down", "q4k", 4096, 14336),
            ("x_qkv", "act", 4, 4096),
            ("x_down", "act", 4, 14336),
            ("res_down", "res", 4, 4096),
        ],
        ops=[
            dict(op="gemv_q4k", label="qkv", w="qkv", x="x_qkv", m=6144, k=4096, batch=4),
            dict(op="gemv_q4k", label="down+residual", w="down", x="x_down", m=4096, k=14336,
                 batch=4, residual="res_down"),
        ],
    ),
    3: dict(
        name="llama3_8b_head_gemv_q6k",
        tensors=[
            ("head", "q6k", 128256, 4096),
            ("x_b1", "act", 1, 4096),
            ("x_b4", "act", 4, 4096),
        ],
        ops=[
            dict(op="gemv_q6k", label="head_b1", w="head", x="x_b1", m=128256, k=4096, batch=1),
            dict(op="gemv_q6k", label="head_b4", w="head", x="x_b4", m=128256, k=4096, batch=4),
        ],
    ),
    4: dict(
        name="qwen2_7b_prefill_mmq_q4k_n2048",
        tensors=[
            ("gate", "q4k", 18944, 3584),
            ("up", "q4k", 18944, 3584),
            ("down", "q4k", 3584, 18944),
            ("qkv", "q4k", 4608, 3584),
            ("x_in", "act", 2048, 3584),
            ("x_down", "act", 2048, 18944),
        ],
        ops=[
            dict(op="mmq_q4k", label="gate", w="gate", x="x_in", m=18944, k=3584, n=2048),
            dict(op="mmq_q4k", label="up", w="up", x="x_in", m=18944, k=3584, n=2048),
            dict(op="mmq_q4k", label="down", w="down", x="x_down", m=3584, k=18944, n=2048),
            dict(op="mmq_q4k", label="qkv", w="qkv", x="x_in", m=4608, k=3584, n=2048),
        ],
    ),
    # producers that emit q8_1 directly (RMSNorm of x + residual; SwiGLU),
    # decode sizes of Llama-3-8B and prefill sizes of Qwen2-7B at 2048 tokens
    5: dict(
        name="llama3_8b_decode_producers_q8_1",
        tensors=[
            ("x", "act", 1, 4096),
            ("res", "res", 1, 4096),
            ("g", "gain", 1, 4096),
            ("gate", "act", 1, 14336),
            ("up", "act", 1, 14336),
        ],
        ops=[
            dict(op="rmsnorm_q8_1", label="attn_norm", x="x", res="res", g="g", eps=1e-5, rows=1, n=4096),
            dict(op="swiglu_q8_1", label="ffn_swiglu", gate="gate", up="up", rows=1, n=14336),
        ],
    ),
    6: dict(
        name="qwen2_7b_prefill_producers_q8_1_n2048",
        tensors=[
            ("x", "act", 2048, 3584),
            ("res", "res", 2048, 3584),
            ("g", "gain", 1, 3584),
            ("gate", "act", 2048, 18944),
            ("up", "act", 2048, 18944),
        ],
        ops=[
            dict(op="rmsnorm_q8_1", label="attn_norm", x="x", res="res", g="g", eps=1e-6, rows=2048, n=3584),
            dict(op="swiglu_q8_1", label="ffn_swiglu", gate="gate", up="up", rows=2048, n=18944),
        ],
    ),
    # decode of eight sequences at once (minfer's decode range is 2..8 tokens)
    7: dict(
        name="llama3_8b_decode_gemv_q4k_b8",
        tensors=[
            ("qkv", "q4k", 6144, 4096),
            ("down", "q4k", 4096, 14336),
            ("x_qkv", "act", 8, 4096),
            ("x_down", "act", 8, 14336),
            ("res_down", "res", 8, 4096),
        ],
        ops=[
            dict(op="gemv_q4k", label="qkv", w="qkv", x="x_qkv", m=6144, k=4096, batch=8),
            dict(op="gemv_q4k", label="down+residual", w="down", x="x_down", m=4096, k=14336,
                 batch=8, residual="res_down"),
        ],
    ),
    # separately stored attention projections of Llama-3-8B (GGUF keeps q, k
    # and v as three tensors): three launches, or one segmented launch
    8: dict(
        name="llama3_8b_decode_qkv_separate_b1",
        tensors=[
            ("q", "q4k", 4096, 4096),
            ("k", "q4k", 1024, 4096),
            ("v", "q4k", 1024, 4096),
            ("x", "act", 1, 4096),
        ],
        ops=[
            dict(op="gemv_q4k", label="q", w="q", x="x", m=4096, k=4096, batch=1),
            dict(op="gemv_q4k", label="k", w="k", x="x", m=1024, k=4096, batch=1),
            dict(op="gemv_q4k", label="v", w="v", x="x", m=1024, k=4096, batch=1),
        ],
    ),
    # the Q6_K tensors of the same prefill (a Q4_K_M model keeps the value
    # projection and the down projection of half its layers in Q6_K)
    9: dict(
        name="qwen2_7b_prefill_mmq_q6k_n2048",
        tensors=[
            ("v", "q6k", 512, 3584),
            ("down", "q6k", 3584, 18944),
            ("x_in", "act", 2048, 3584),
            ("x_down", "act", 2048, 18944),
        ],
        ops=[
            dict(op="mmq_q6k", label="v", w="v", x="x_in", m=512, k=3584, n=2048),
            dict(op="mmq_q6k", label="down", w="down", x="x_down", m=3584, k=18944, n=2048),
        ],
    ),
}


def tensor(cfg: int, name: str) -> np.ndarray:
    """Generate one named tensor of workload ``cfg`` (seed = ``cfg``)."""
    wl = WORKLOADS[cfg]
    for tid, (tname, kind, a, b) in enumerate(wl["tensors"]):
        if tname != name:
            continue
        if kind == "q4k":
            return q4k_weights(cfg, tid, a, b)
        if kind == "q6k":
            return q6k_weights(cfg, tid, a, b)
        if kind == "act":
            return activations(cfg, tid, a, b)
        if kind == "res":
            return residual(cfg, tid, a, b)
        if kind == "gain":
            return gain(cfg, tid, a, b)
        raise ValueError(kind)
    raise KeyError(f"workload {cfg} has no tensor {name!r}")


def random_case(seed: int, kind: str, m: int, k: int, rows: int, with_residual: bool = False):
    """A free-standing random case (weights, activations, optional residual)
    with the workloads' value distributions, for parity tests at other sizes."""
    if kind == "q4k":
        w = q4k_weights(seed, 100, m, k)
    elif kind == "q6k":
        w = q6k_weights(seed, 100, m, k)
    else:
        raise ValueError(kind)
    x = activations(seed, 101, rows, k)
    r = residual(seed, 102, rows, m) if with_residual else None
    return w, x, r
