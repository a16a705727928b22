"""HIP-graph capture of a decode step (what bench.py replays): every replay,
interleaved with eager work and synchronisations, must reproduce the eager
outputs bit for bit."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu


def test_graph_replay_matches_eager():
    import q6_q8_matmul_amd as kq
    from kq_inputs import random_case

    print("\n[case] graph replay: quantize + gemv_q4k + gemv_q6k(residual) + mmq_q4k", flush=True)
    w4, x4, _ = random_case(1, "q4k", 1000, 4096, 4)
    w6, _, res = random_case(2, "q6k", 700, 4096, 4, with_residual=True)
    wm, xm, _ = random_case(3, "q4k", 300, 1024, 200)
    d = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    w4d, x4d, w6d, resd, wmd, xmd = d(w4), d(x4), d(w6), d(res), d(wm), d(xm)
    xq = torch.empty((4, 4096 // 32 * 36), dtype=torch.uint8, device="cuda")
    xqm = torch.empty((200, 1024 // 32 * 36), dtype=torch.uint8, device="cuda")
    y4 = torch.empty((4, 1000), device="cuda")
    y6 = torch.empty((4, 700), device="cuda")
    ym = torch.empty((200, 300), device="cuda")

    def step():
        kq.kq_quantize_q8_1(x4d, xq, 4, 4096)
        kq.kq_gemv_q4k(w4d, xq, y4, None, 1000, 4096, 4)
        kq.kq_gemv_q6k(w6d, xq, y6, resd, 700, 4096, 4)
        kq.kq_quantize_q8_1(xmd, xqm, 200, 1024)
        kq.kq_mmq_q4k(wmd, xqm, ym, 300, 200, 1024)

    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (xq, y4, y6, ym)]

    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    with torch.cuda.graph(g, stream=side):
        step()
    for rep in range(4):
        for t in (xq, y4, y6, ym):
            t.zero_()                       # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(ref, (xq, y4, y6, ym)):
            assert torch.equal(a, b), f"replay {rep} differs from the eager step"
        step()                              # eager again, still identical
        torch.cuda.synchronize()
        for a, b in zip(ref, (xq, y4, y6, ym)):
            assert torch.equal(a, b)


def test_multi_step_graph_over_copies_matches_eager():
    """What bench.py replays: one graph holding several steps that rotate over
    weight copies, here with the segmented GEMV and the K-split MMQ (whose
    fixed-order sum is a second launch inside the graph).  Every replay, with
    eager work in between, must give each copy's eager outputs bit for bit."""
    import q6_q8_matmul_amd as kq
    from kq_inputs import random_case

    print("\n[case] multi-step graph: seg GEMV + K-split MMQ over 2 weight copies", flush=True)
    d = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    m_q, m_k, k, batch = 512, 256, 2048, 2
    mm, nn, kk = 384, 256, 2048
    nb = kq.kq_mmq_q4k_workspace_bytes(mm, nn, kk)
    assert nb > 0, "the MMQ shape must take the K split"
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
    copies = []
    for c in range(2):
        wq, x, _ = random_case(10 + c, "q4k", m_q, k, batch)
        wk, _, _ = random_case(20 + c, "q4k", m_k, k, batch)
        wm, xm, _ = random_case(30 + c, "q4k", mm, kk, nn)
        copies.append({"wq": d(wq), "wk": d(wk), "wm": d(wm), "x": d(x), "xm": d(xm),
                       "xq": torch.empty((batch, k // 32 * 36), dtype=torch.uint8, device="cuda"),
                       "xqm": torch.empty((nn, kk // 32 * 36), dtype=torch.uint8, device="cuda"),
                       "yq": torch.empty((batch, m_q), device="cuda"),
                       "yk": torch.empty((batch, m_k), device="cuda"),
                       "ym": torch.empty((nn, mm), device="cuda")})

    def step(c):
        t = copies[c]
        kq.kq_quantize_q8_1(t["x"], t["xq"], batch, k)
        kq.kq_gemv_q4k_seg([t["wq"], t["wk"]], [m_q, m_k], [t["yq"], t["yk"]], None, t["xq"], k, batch)
        kq.kq_quantize_q8_1(t["xm"], t["xqm"], nn, kk)
        kq.kq_mmq_q4k_ws(t["wm"], t["xqm"], t["ym"], mm, nn, kk, ws, nb)

    outs = ("xq", "yq", "yk", "xqm", "ym")
    ref = []
    for c in range(2):
        step(c)
        torch.cuda.synchronize()
        ref.append({n: copies[c][n].clone() for n in outs})
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    with torch.cuda.graph(g, stream=side):
        for i in range(6):
            step(i % 2)
    for rep in range(3):
        for c in range(2):
            for n in outs:
                copies[c][n].zero_()        # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for c in range(2):
            for n in outs:
                assert torch.equal(ref[c][n], copies[c][n]), f"replay {rep}, copy {c}: {n} differs"
        step(rep % 2)                       # eager again, still identical
        torch.cuda.synchronize()
        for n in outs:
            assert torch.equal(ref[rep % 2][n], copies[rep % 2][n])
