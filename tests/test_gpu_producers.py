"""Parity of the fused producers (RMSNorm -> q8_1, SwiGLU -> q8_1) with the
CPU oracle, through the C ABI.

Both producers are defined step by step in IEEE f32 (the oracle's header and
include/kq.h state the reduction order and the exponential), so the f32
output y and the q8_1 blocks must match the oracle bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle
from kq_inputs import WORKLOADS, activations, gain, residual, tensor

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def kq():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    import q6_q8_matmul_amd as kq

    kq.lib()
    oracle.build(force=False)
    return kq


def say(msg):
    print(f"\n[case] {msg}", flush=True)


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def check_rmsnorm(kq, x, g, eps, res=None, want_y=True, label=""):
    y_ref, q_ref = oracle.rmsnorm_q8_1(x, g, eps, residual=res)
    y, xq = kq.rmsnorm_q8_1(dev(x), dev(g), eps, residual=None if res is None else dev(res),
                            want_y=want_y)
    q = host(xq)
    assert np.array_equal(q, q_ref), f"{label}: q8_1 blocks differ"
    if want_y:
        yy = host(y)
        same = (yy == y_ref) | (np.isnan(yy) & np.isnan(y_ref))
        assert same.all(), f"{label}: {np.count_nonzero(~same)} y values differ"


def check_swiglu(kq, gate, up, want_y=True, label=""):
    y_ref, q_ref = oracle.swiglu_q8_1(gate, up)
    y, xq = kq.swiglu_q8_1(dev(gate), dev(up), want_y=want_y)
    q = host(xq)
    assert np.array_equal(q, q_ref), f"{label}: q8_1 blocks differ"
    if want_y:
        yy = host(y)
        same = (yy == y_ref) | (np.isnan(yy) & np.isnan(y_ref))
        assert same.all(), f"{label}: {np.count_nonzero(~same)} y values differ"


RMS_SHAPES = [(1, 256), (1, 4096), (3, 14336), (2, 65536), (17, 1280), (64, 512), (70, 16384),
              (300, 3584), (80, 16128)]


@pytest.mark.parametrize("rows,n", RMS_SHAPES, ids=[f"r{r}-n{n}" for r, n in RMS_SHAPES])
@pytest.mark.parametrize("with_res", [False, True], ids=["plain", "residual"])
def test_rmsnorm_bitexact(kq, rows, n, with_res):
    say(f"rmsnorm rows={rows} n={n} residual={with_res}")
    x = activations(rows * 7 + n, 0, rows, n)
    res = residual(rows * 7 + n, 1, rows, n) if with_res else None
    g = gain(rows * 7 + n, 2, 1, n)[0]
    check_rmsnorm(kq, x, g, 1e-5, res, label=f"r{rows} n{n}")


def test_rmsnorm_skip_write_and_eps(kq):
    say("rmsnorm q8_1 only; eps 0 and 1e-2; tiny and huge rows")
    n = 1024
    x = activations(91, 0, 4, n)
    g = gain(91, 1, 1, n)[0]
    check_rmsnorm(kq, x, g, 1e-5, want_y=False, label="skip y")
    check_rmsnorm(kq, x, g, 0.0, label="eps 0")
    check_rmsnorm(kq, x * np.float32(1e-3), g, 1e-2, label="eps dominates")
    check_rmsnorm(kq, x * np.float32(1e-21), g, 0.0, label="subnormal squares")
    check_rmsnorm(kq, x * np.float32(1e19), g, 1e-5, label="squares overflow")


def test_rmsnorm_edge_rows(kq):
    say("rmsnorm zero row, constant row, reduction-order row")
    n = 512
    x = np.zeros((3, n), dtype=np.float32)
    x[1, :] = -8.0
    x[2, 0], x[2, 1], x[2, 257] = 4096.0, 1.0, 1.0
    g = gain(92, 0, 1, n)[0]
    check_rmsnorm(kq, x, g, 1e-6, label="edge rows")


SW_SHAPES = [(1, 256), (1, 14336), (3, 18944), (2, 65536), (33, 768)]


@pytest.mark.parametrize("rows,n", SW_SHAPES, ids=[f"r{r}-n{n}" for r, n in SW_SHAPES])
def test_swiglu_bitexact(kq, rows, n):
    say(f"swiglu rows={rows} n={n}")
    gate = activations(rows * 11 + n, 0, rows, n) * np.float32(4.0)
    up = activations(rows * 11 + n, 1, rows, n)
    check_swiglu(kq, gate, up, label=f"r{rows} n{n}")


def test_swiglu_special_gates(kq):
    say("swiglu saturated, overflowing and exact gates")
    vals = np.array([0.0, -0.0, 30.0, -30.0, 87.0, -87.0, 88.5, -88.5, 100.0, -100.0, 100.5,
                     -100.5, 110.0, -110.0, 111.0, -111.0, 1e30, -1e30, 1e-30, -1e-30,
                     0.5, -0.5, 17.0, -17.0], dtype=np.float32)
    gate = np.resize(vals, (2, 256)).astype(np.float32)
    up = np.resize(np.array([2.0, -1.0, 0.25, 3.0], dtype=np.float32), (2, 256)).astype(np.float32)
    check_swiglu(kq, gate, up, label="special gates")
    sweep = np.linspace(-120.0, 120.0, 65536, dtype=np.float32).reshape(4, 16384)
    check_swiglu(kq, sweep, np.ones_like(sweep), label="gate sweep")
    check_swiglu(kq, sweep, np.ones_like(sweep), want_y=False, label="gate sweep, q8_1 only")


@pytest.mark.parametrize("cfg", [5, 6])
def test_producer_workloads(kq, cfg):
    wl = WORKLOADS[cfg]
    for op in wl["ops"]:
        say(f"{wl['name']} {op['label']}")
        if op["op"] == "rmsnorm_q8_1":
            check_rmsnorm(kq, tensor(cfg, op["x"]), tensor(cfg, op["g"])[0], op["eps"],
                          tensor(cfg, op["res"]), label=op["label"])
        else:
            check_swiglu(kq, tensor(cfg, op["gate"]), tensor(cfg, op["up"]), label=op["label"])


def test_fused_producer_feeds_the_gemv(kq):
    """The q8_1 blocks of the fused producer are those of the separate
    quantiser applied to its f32 output, so the GEMV sees the same input."""
    say("rmsnorm_q8_1 -> gemv_q4k vs rmsnorm -> quantize -> gemv_q4k")
    from kq_inputs import q4k_weights

    n, m = 4096, 512
    x = activations(93, 0, 1, n)
    g = gain(93, 1, 1, n)[0]
    w = dev(q4k_weights(93, 2, m, n))
    y, xq = kq.rmsnorm_q8_1(dev(x), dev(g), 1e-5)
    xq2 = kq.quantize_q8_1(y)
    assert torch.equal(xq, xq2)
    a = kq.gemv_q4k(w, xq, m, n, 1)
    b = kq.gemv_q4k(w, xq2, m, n, 1)
    assert torch.equal(a, b)
