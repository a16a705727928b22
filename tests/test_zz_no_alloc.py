"""kq_mmq_q6k_noalloc -- the K-split Q6_K product whose workspace is the
library's static device scratch -- through the C ABI: the same bits as
kq_mmq_q6k_ws with a workspace, on consecutive calls (the second smaller,
so it runs over what the first left in the scratch), within the oracle's
bound, and a clear error for a product whose split needs more scratch than
the array holds."""
import numpy as np
import pytest
import torch

import oracle
from kq_inputs import random_case

pytestmark = pytest.mark.gpu
RTOL = 1e-5
SCRATCH = 32 << 20     # KQ_NOALLOC_SCRATCH_BYTES


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


def test_noalloc_matches_the_workspace_form(kq):
    for m, n, k in ((512, 2048, 3584), (300, 100, 2048), (33, 5, 1280)):
        say(f"mmq q6k no-alloc m={m} n={n} k={k}")
        nb = kq.kq_mmq_q6k_workspace_bytes(m, n, k)
        assert 0 < nb <= SCRATCH
        w, x, _ = random_case(m + 5 * n + k, "q6k", m, k, n)
        xq = oracle.quantize_q8_1(x)
        wd, xd = dev(w), dev(xq)
        y_ws = kq.mmq_q6k_ws(wd, xd, m, n, k)
        y = torch.full((n, m), float("nan"), device="cuda")
        rc = kq.lib().kq_mmq_q6k_noalloc(wd.data_ptr(), xd.data_ptr(), y.data_ptr(), m, n, k,
                                         torch.cuda.current_stream().cuda_stream)
        assert rc == kq.KQ_OK, kq.kq_last_error()
        torch.cuda.synchronize()
        assert torch.equal(y, y_ws), "differs from kq_mmq_q6k_ws"
        if m * n * k <= 1 << 31:
            y_ref, den = oracle.matmul("q6k", w, xq, m, n, k)
            ok, ratio = oracle.tolerance_ok(y.cpu().numpy(), y_ref, den, RTOL)
            say(f"max |gpu-oracle|/den = {ratio:.3e}")
            assert ok


def test_noalloc_without_a_split(kq):
    m, n, k = 4096, 1024, 512
    say(f"mmq q6k no-alloc, no split m={m} n={n} k={k}")
    assert kq.kq_mmq_q6k_workspace_bytes(m, n, k) == 0
    w, x, _ = random_case(77, "q6k", m, k, n)
    wd, xd = dev(w), dev(oracle.quantize_q8_1(x))
    y = torch.empty((n, m), device="cuda")
    kq.kq_mmq_q6k_noalloc(wd, xd, y, m, n, k)
    assert torch.equal(y, kq.mmq_q6k(wd, xd, m, n, k))


def test_noalloc_rejects_a_split_beyond_the_scratch(kq):
    m, n, k = 3584, 2048, 18944          # split in four: 88 MB of ranges
    say(f"mmq q6k no-alloc beyond the scratch m={m} n={n} k={k}")
    assert kq.kq_mmq_q6k_workspace_bytes(m, n, k) > SCRATCH
    w = torch.zeros(m * (k // 256) * 210, dtype=torch.uint8, device="cuda")
    xq = torch.zeros(n * (k // 32) * 36, dtype=torch.uint8, device="cuda")
    y = torch.full((n, m), 7.0, device="cuda")
    with pytest.raises(kq.KQError, match="bytes of scratch"):
        kq.kq_mmq_q6k_noalloc(w, xq, y, m, n, k)
    torch.cuda.synchronize()
    assert torch.all(y == 7.0).item()
