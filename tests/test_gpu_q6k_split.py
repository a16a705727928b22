"""The split Q6_K layout on the GPU, through the C ABI.

* kq_repack_q6k: byte-exact against the oracle's split layout (f16 d prefix
  padded to 16 bytes, 208-byte bodies), including the full output head.
* kq_gemv_q6k_split / kq_mmq_q6k_split: bitwise equal to kq_gemv_q6k /
  kq_mmq_q6k on the raw bytes (the same arithmetic in the same order), and
  within 1e-5 x (sum of |per-32-block terms|) of the oracle on the raw weights.
"""
import numpy as np
import pytest
import torch

import oracle
from kq_inputs import WORKLOADS, activations, q6k_weights, random_case, residual, tensor

pytestmark = pytest.mark.gpu
RTOL = 1e-5


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


def check_close(y_gpu, y_ref, den, label):
    ok, ratio = oracle.tolerance_ok(y_gpu, y_ref, den, RTOL)
    say(f"{label}: max |gpu-oracle|/den = {ratio:.3e}")
    assert ok, f"{label}: tolerance exceeded, max ratio {ratio:.3e} > {RTOL}"


REPACK_SHAPES = [(1, 256), (2, 512), (3, 1280), (7, 4096), (33, 768), (129, 18944)]


@pytest.mark.parametrize("m,k", REPACK_SHAPES, ids=[f"m{m}-k{k}" for m, k in REPACK_SHAPES])
def test_repack_bytes(kq, m, k):
    say(f"repack m={m} k={k}")
    w = q6k_weights(11, m, m, k)
    wr = kq.repack_q6k(dev(w), m, k)
    assert np.array_equal(host(wr), oracle.q6k_split(w, m, k))


def test_repack_output_head(kq):
    op = WORKLOADS[3]["ops"][0]
    m, k = op["m"], op["k"]
    say(f"repack output head m={m} k={k}")
    w = tensor(3, op["w"])
    wr = kq.repack_q6k(dev(w), m, k)
    assert np.array_equal(host(wr), oracle.q6k_split(w, m, k))


GEMV_CASES = [(m, k, b, r) for (m, k) in [(1, 256), (37, 768), (300, 4096), (130, 14336), (37, 65536)]
              for b in (1, 2, 4, 8) for r in (False, True)]


@pytest.mark.parametrize("m,k,batch,res_on", GEMV_CASES,
                         ids=[f"m{m}-k{k}-b{b}-{'res' if r else 'nores'}" for m, k, b, r in GEMV_CASES])
def test_gemv_split_matches_raw(kq, m, k, batch, res_on):
    say(f"gemv q6k split m={m} k={k} batch={batch} residual={res_on}")
    w, x, rh = random_case(m + k + batch, "q6k", m, k, batch, with_residual=res_on)
    xq_h = oracle.quantize_q8_1(x)
    wd, xq = dev(w), dev(xq_h)
    rd = dev(rh) if res_on else None
    wr = kq.repack_q6k(wd, m, k)
    y_split = kq.gemv_q6k_split(wr, xq, m, k, batch, residual=rd)
    y_raw = kq.gemv_q6k(wd, xq, m, k, batch, residual=rd)
    assert torch.equal(y_split, y_raw), "split layout differs from the raw layout"
    y_ref, den = oracle.matmul("q6k", w, xq_h, m, batch, k, residual=rh)
    check_close(host(y_split), y_ref, den, f"gemv split m{m} k{k} b{batch}")


def test_gemv_split_in_place_residual(kq):
    m, k, batch = 200, 2048, 3
    say(f"gemv q6k split in place m={m} k={k} batch={batch}")
    w, x, rh = random_case(77, "q6k", m, k, batch, with_residual=True)
    xq_h = oracle.quantize_q8_1(x)
    wr = kq.repack_q6k(dev(w), m, k)
    y = dev(rh)
    kq.gemv_q6k_split(wr, dev(xq_h), m, k, batch, residual=y, out=y)
    y_ref, den = oracle.matmul("q6k", w, xq_h, m, batch, k, residual=rh)
    check_close(host(y), y_ref, den, "gemv split in place")


def test_gemv_split_output_head(kq):
    cfg = 3
    for op in WORKLOADS[cfg]["ops"]:
        m, k, b = op["m"], op["k"], op["batch"]
        say(f"gemv q6k split cfg3 {op['label']} m={m} k={k} batch={b}")
        w = tensor(cfg, op["w"])
        x = tensor(cfg, op["x"])
        xq_h = oracle.quantize_q8_1(x)
        wd, xq = dev(w), dev(xq_h)
        wr = kq.repack_q6k(wd, m, k)
        y_split = kq.gemv_q6k_split(wr, xq, m, k, b)
        assert torch.equal(y_split, kq.gemv_q6k(wd, xq, m, k, b))
        rows = np.random.default_rng(b).integers(0, m, 3000)
        tok = np.repeat(np.arange(b), rows.size)
        row = np.tile(rows, b)
        y_ref, den = oracle.matmul_pairs("q6k", w, xq_h, m, b, k, tok, row)
        check_close(host(y_split)[tok, row], y_ref, den, f"gemv split head b{b} (sampled)")
        del wd, wr
        torch.cuda.empty_cache()


MMQ_CASES = [(1, 1, 256), (5, 3, 512), (150, 70, 768), (300, 130, 3584), (131, 70, 18944),
             (3584, 640, 256), (4096, 1024, 256), (130, 70, 65536)]


@pytest.mark.parametrize("m,n,k", MMQ_CASES, ids=[f"m{m}-n{n}-k{k}" for m, n, k in MMQ_CASES])
def test_mmq_split_matches_raw(kq, m, n, k):
    say(f"mmq q6k split m={m} n={n} k={k}")
    w, x, _ = random_case(m * 3 + n + k, "q6k", m, k, n)
    xq_h = oracle.quantize_q8_1(x)
    wd, xq = dev(w), dev(xq_h)
    wr = kq.repack_q6k(wd, m, k)
    y_split = kq.mmq_q6k_split(wr, xq, m, n, k)
    assert torch.equal(y_split, kq.mmq_q6k(wd, xq, m, n, k)), "split layout differs from raw"
    y_ref, den = oracle.matmul("q6k", w, xq_h, m, n, k)
    check_close(host(y_split), y_ref, den, f"mmq split m{m} n{n} k{k}")


def test_split_bad_arguments_launch_nothing(kq):
    say("split entry points: argument errors on real buffers")
    m, k = 64, 512
    w = dev(q6k_weights(5, 0, m, k))
    wr = kq.repack_q6k(w, m, k)
    xq = dev(oracle.quantize_q8_1(activations(5, 1, 2, k)))
    y = torch.full((2, m), 7.0, device="cuda")
    for call in (
        lambda: kq.kq_gemv_q6k_split(wr, xq, y, None, m, 500, 2),
        lambda: kq.kq_gemv_q6k_split(wr, xq, y, None, m, k, 9),
        lambda: kq.kq_mmq_q6k_split(wr, xq, wr, m, 2, k),
        lambda: kq.kq_repack_q6k(w, w, m, k),
    ):
        with pytest.raises(kq.KQError):
            call()
    assert torch.all(y == 7.0).item()
    assert np.array_equal(host(wr), oracle.q6k_split(w.cpu().numpy(), m, k))
