"""Parity of the gfx950 kernels with the CPU oracle, through the C ABI.

* q8_1 quantisation: bit-exact (codes, f16 scale, f16 source sum).
* matmuls: |y_gpu - y_oracle| <= 1e-5 * (sum_j |T_j| + |residual|) for every
  output checked, T_j being the oracle's per-32-block term (f64).
GEMVs are checked on every output at the workloads' full sizes; the prefill
MMQ is checked on every output at sizes spanning several tiles with ragged
edges, and on sampled outputs (tile corners plus random picks) at the
prefill workload's full size.
"""
import numpy as np
import pytest
import torch

import oracle
from kq_inputs import WORKLOADS, activations, random_case, residual, tensor
from oracle_pins import _adversarial_blocks, _distinguishing_blocks

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


# ------------------------------------------------------------ quantiser ----

ACTS = [(c, name) for c, wl in WORKLOADS.items() for (name, kind, *_r) in wl["tensors"]
        if kind == "act"]


@pytest.mark.parametrize("cfg,name", ACTS, ids=[f"cfg{c}-{n}" for c, n in ACTS])
def test_quantize_bitexact_workloads(kq, cfg, name):
    x = tensor(cfg, name)
    say(f"quantize cfg{cfg} {name} {x.shape}")
    ref = oracle.quantize_q8_1(x)
    got = host(kq.quantize_q8_1(dev(x)))
    assert np.array_equal(got, ref), f"{np.count_nonzero(got != ref)} bytes differ"


def test_quantize_bitexact_adversarial(kq):
    blocks = np.concatenate([_adversarial_blocks(), _distinguishing_blocks()]).astype(np.float32)
    rng = np.random.default_rng(3)
    extra = [
        (rng.standard_normal((64, 32)) * 2.0 ** -20).astype(np.float32),  # f16-subnormal d
        (rng.standard_normal((64, 32)) * 6e4).astype(np.float32),         # large values
        np.full((2, 32), -0.0, dtype=np.float32),
    ]
    x = np.concatenate([blocks] + extra)
    n = (x.shape[0] // 8) * 8
    x = x[:n].reshape(-1, 256)
    say(f"quantize adversarial {x.shape}")
    ref = oracle.quantize_q8_1(x)
    got = host(kq.quantize_q8_1(dev(x)))
    bad = np.nonzero((got != ref).any(axis=1))[0]
    assert bad.size == 0, f"rows {bad[:5]} differ"


@pytest.mark.parametrize("rows,k", [(1, 32), (3, 96), (5, 256), (7, 4128), (1000, 64), (3, 65536)])
def test_quantize_ragged(kq, rows, k):
    x = np.random.default_rng(rows * 7 + k).standard_normal((rows, k)).astype(np.float32)
    say(f"quantize ragged rows={rows} k={k}")
    assert np.array_equal(host(kq.quantize_q8_1(dev(x))), oracle.quantize_q8_1(x))


def test_quantize_tiny_scale_blocks(kq):
    """Blocks whose 1/d overflows (amax < 127 * 2^-128): zeros code 0,
    nonzero values +-127, f16 d = 0 -- bit-exact with the oracle."""
    say("quantize tiny-scale blocks")
    rng = np.random.default_rng(17)
    x = np.zeros((4, 256), dtype=np.float32)
    x[0, :] = rng.standard_normal(256).astype(np.float32) * np.float32(1e-38)
    x[1, ::3] = np.float32(-(2.0 ** -122))
    x[1, 1::7] = np.float32(2.0 ** -140)
    x[2, :] = np.float32(2.0 ** -149) * rng.integers(-3, 4, 256).astype(np.float32)
    x[3, :] = rng.standard_normal(256).astype(np.float32) * np.float32(3e-37)
    xq = host(kq.quantize_q8_1(dev(x)))
    assert np.array_equal(xq, oracle.quantize_q8_1(x))


# --------------------------------------------------------------- GEMVs -----

def run_gemv(kq, kind, w, xq, m, k, batch, res=None, inplace=False):
    wd, xd = dev(w), dev(xq)
    rd = dev(res) if res is not None else None
    fn = kq.gemv_q4k if kind == "q4k" else kq.gemv_q6k
    if inplace:
        y = fn(wd, xd, m, k, batch, residual=rd, out=rd)
    else:
        y = fn(wd, xd, m, k, batch, residual=rd)
    return host(y)


GEMV_OPS = [(c, i) for c in (0, 1, 2, 3, 7) for i in range(len(WORKLOADS[c]["ops"]))]


@pytest.mark.parametrize("cfg,i", GEMV_OPS,
                         ids=[f"cfg{c}-{WORKLOADS[c]['ops'][i]['label']}" for c, i in GEMV_OPS])
def test_gemv_workloads_full(kq, cfg, i):
    op = WORKLOADS[cfg]["ops"][i]
    kind = "q4k" if op["op"] == "gemv_q4k" else "q6k"
    m, k, b = op["m"], op["k"], op["batch"]
    say(f"gemv {kind} cfg{cfg} {op['label']} m={m} k={k} batch={b}")
    w = tensor(cfg, op["w"])
    x = tensor(cfg, op["x"])
    res = tensor(cfg, op["residual"]) if "residual" in op else None
    xq = oracle.quantize_q8_1(x)
    y_ref, den = oracle.matmul(kind, w, xq, m, b, k, residual=res)
    y = run_gemv(kq, kind, w, xq, m, k, b, res)
    check_close(y, y_ref, den, f"cfg{cfg} {op['label']}")


SHAPES = [
    # kind, m, k, batch, residual -- ragged rows, one superblock, odd superblock
    # counts (Q6_K superblocks at 2 mod 4), several LDS chunks (k*batch large)
    ("q4k", 1, 256, 1, False), ("q4k", 7, 768, 3, True), ("q4k", 13, 2304, 2, False),
    ("q4k", 1000, 1024, 4, True), ("q4k", 37, 14336, 4, True), ("q4k", 9, 32768, 4, False),
    ("q4k", 300, 4352, 1, False),
    ("q6k", 1, 256, 1, False), ("q6k", 7, 768, 3, True), ("q6k", 13, 2304, 2, False),
    ("q6k", 1001, 1280, 4, True), ("q6k", 37, 14336, 4, True), ("q6k", 9, 32768, 4, False),
    ("q6k", 300, 4352, 1, False), ("q6k", 20001, 512, 3, True),
    # batches 5..8: persistent (activation fits) and chunked (it does not)
    ("q4k", 1000, 4096, 8, True), ("q4k", 513, 2048, 5, False), ("q4k", 37, 14336, 6, True),
    ("q4k", 130, 28672, 7, False), ("q6k", 1001, 4096, 8, True), ("q6k", 77, 768, 5, False),
    ("q6k", 9, 32768, 8, False), ("q6k", 2000, 1024, 6, True),
    # the largest k the calls accept (KQ_MAX_K): the activation in many LDS chunks
    ("q4k", 37, 65536, 1, True), ("q4k", 37, 65536, 4, False), ("q4k", 19, 65536, 8, True),
    ("q6k", 37, 65536, 1, False), ("q6k", 37, 65536, 4, True), ("q6k", 19, 65536, 8, False),
]


@pytest.mark.parametrize("kind,m,k,batch,with_res", SHAPES,
                         ids=[f"{s[0]}-m{s[1]}-k{s[2]}-b{s[3]}{'-res' if s[4] else ''}" for s in SHAPES])
def test_gemv_shapes(kq, kind, m, k, batch, with_res):
    say(f"gemv {kind} m={m} k={k} batch={batch} residual={with_res}")
    w, x, res = random_case(m * 131 + k + batch, kind, m, k, batch, with_residual=with_res)
    xq = oracle.quantize_q8_1(x)
    y_ref, den = oracle.matmul(kind, w, xq, m, batch, k, residual=res)
    check_close(run_gemv(kq, kind, w, xq, m, k, batch, res), y_ref, den, f"{kind} m{m} k{k} b{batch}")


@pytest.mark.parametrize("kind", ["q4k", "q6k"])
@pytest.mark.parametrize("k", [4096, 14336])   # 14336 at batch 4: the Q4_K K split
def test_gemv_in_place_residual(kq, kind, k):
    m, b = 333, 4
    say(f"gemv {kind} in place m={m} k={k} batch={b}")
    w, x, res = random_case(77, kind, m, k, b, with_residual=True)
    xq = oracle.quantize_q8_1(x)
    y_ref, den = oracle.matmul(kind, w, xq, m, b, k, residual=res)
    check_close(run_gemv(kq, kind, w, xq, m, k, b, res, inplace=True), y_ref, den, "in place")


@pytest.mark.parametrize("kind", ["q4k", "q6k"])
@pytest.mark.parametrize("k", [4096, 14336])
def test_gemv_batch_columns(kq, kind, k):
    """Column b of a batch-4 call against the batch-1 call on x_b: bitwise
    where both stage the activation in one piece, else within tolerance."""
    m = 515
    say(f"gemv {kind} batch columns m={m} k={k}")
    w, x, _ = random_case(88 + k, kind, m, k, 4)
    xq = oracle.quantize_q8_1(x)
    y4 = run_gemv(kq, kind, w, xq, m, k, 4)
    y_ref, den = oracle.matmul(kind, w, xq, m, 4, k)
    for b in range(4):
        y1 = run_gemv(kq, kind, w, xq[b:b + 1], m, k, 1)[0]
        if k == 4096:
            assert np.array_equal(y1, y4[b]), f"column {b} differs bitwise"
        check_close(y1, y_ref[b], den[b], f"column {b} batch-1")


@pytest.mark.parametrize("kind", ["q4k", "q6k"])
def test_gemv_deterministic(kq, kind):
    m, k, b = 4096, 4096, 4
    say(f"gemv {kind} determinism m={m} k={k} batch={b}")
    w, x, _ = random_case(5, kind, m, k, b)
    xq = oracle.quantize_q8_1(x)
    wd, xd = dev(w), dev(xq)
    fn = kq.gemv_q4k if kind == "q4k" else kq.gemv_q6k
    a = host(fn(wd, xd, m, k, b))
    for _ in range(3):
        assert np.array_equal(a, host(fn(wd, xd, m, k, b)))


# ----------------------------------------------------------------- MMQ -----

# Workgroup tiles on a 256-CU MI355X.  Q6_K: the small shapes take 32
# tokens; 3584 x 640 and 4096 x 1024 are the first grids of 64 and 128
# tokens to give every CU a workgroup.  Q4_K: 192 rows x 128 tokens, with a
# clamped form for problems smaller than one tile in either direction
# (m < 192 or n < 128); 7168 x 2048 is 608 tiles, more than two rounds of
# one workgroup per CU, with ragged last row tiles.
MMQ_SHAPES = [(1, 1, 256), (5, 3, 512), (128, 128, 256), (200, 150, 1024), (129, 257, 768),
              (300, 64, 3584), (64, 300, 2048), (131, 70, 18944), (3584, 640, 256),
              (4096, 1024, 256), (3584, 2048, 256), (130, 70, 65536), (7168, 2048, 256),
              (191, 127, 512), (193, 129, 512)]
MMQ_CASES = [(kind, *shape) for kind in ("q4k", "q6k") for shape in MMQ_SHAPES]


def mmq(kq, kind):
    return kq.mmq_q4k if kind == "q4k" else kq.mmq_q6k


@pytest.mark.parametrize("kind,m,n,k", MMQ_CASES, ids=[f"{c[0]}-m{c[1]}-n{c[2]}-k{c[3]}" for c in MMQ_CASES])
def test_mmq_full(kq, kind, m, n, k):
    say(f"mmq {kind} m={m} n={n} k={k}")
    w, x, _ = random_case(m + 3 * n + k, kind, m, k, n)
    xq = oracle.quantize_q8_1(x)
    y_ref, den = oracle.matmul(kind, w, xq, m, n, k)
    y = host(mmq(kq, kind)(dev(w), dev(xq), m, n, k))
    check_close(y, y_ref, den, f"mmq {kind} m{m} n{n} k{k}")


@pytest.mark.parametrize("kind", ["q4k", "q6k"])
def test_mmq_token_grid_limit(kq, kind):
    """More tokens than 65535 workgroups of 64 cover (n = 2^22 + 64, a ragged
    last tile): the launch must take 128-token tiles.  The q8_1 rows repeat
    with period 4096, so every token's outputs must equal those of its base
    token bit for bit, and the base tokens are checked against the oracle."""
    m, k, period, n = 3, 256, 4096, (1 << 22) + 64
    say(f"mmq {kind} token-grid limit m={m} n={n} k={k}")
    w, x, _ = random_case(9001, kind, m, k, period)
    xq_base = oracle.quantize_q8_1(x)
    reps = -(-n // period)
    xq = np.tile(xq_base, (reps, 1))[:n]
    y = mmq(kq, kind)(dev(w), dev(xq), m, n, k)
    del xq
    torch.cuda.synchronize()
    yb = y[:period].clone()
    full = y[: (n // period) * period].view(n // period, period, m)
    assert torch.equal(full, yb.expand_as(full)), "a repeated token's outputs differ"
    assert torch.equal(y[(n // period) * period:], yb[: n % period]), "ragged tail differs"
    y_ref, den = oracle.matmul(kind, w, xq_base, m, period, k)
    check_close(host(yb), y_ref, den, f"mmq {kind} token-grid limit (base tokens)")
    del y, full, yb
    torch.cuda.empty_cache()


def _q6k_extreme(m, k, rng, scale_choice, code_choice):
    """Q6_K bytes with chosen int8 scales and 6-bit codes (placed at the
    format's byte offsets: ql nibbles and qh bit pairs of every code equal)."""
    s = k // 256
    w = np.zeros((m, s, 210), dtype=np.uint8)
    q = rng.choice(np.array(code_choice, dtype=np.uint8), size=(m, s, 1))
    w[:, :, 0:128] = (q & 15) * 17                                  # both nibbles
    w[:, :, 128:192] = ((q >> 4) & 3) * 0x55                        # all four bit pairs
    w[:, :, 192:208] = rng.choice(np.array(scale_choice, dtype=np.int16), size=(m, s, 16)).astype(np.int8).view(np.uint8)
    w[:, :, 208:210] = np.frombuffer(np.float16(0.25).tobytes(), dtype=np.uint8)
    return w.reshape(m, s * 210)


@pytest.mark.parametrize("case", ["max_product", "min_product", "full_range"])
def test_mmq_q6k_extreme_scales(kq, case):
    """Scales at the ends of the int8 range with the extreme codes: the
    products sc*(q-32) reach 4096 and -4064, and the 32-value integer dots
    reach 2^24 - 2^17 (every q8 code at +-127)."""
    m, n, k = 160, 40, 1024
    rng = np.random.default_rng({"max_product": 1, "min_product": 2, "full_range": 3}[case])
    if case == "max_product":       # sc = -128, q = 0: (q-32)*sc = 4096
        w = _q6k_extreme(m, k, rng, [-128], [0])
    elif case == "min_product":     # sc = 127, q = 0: -4064; sc = -128, q = 63: -3968
        w = _q6k_extreme(m, k, rng, [127, -128], [0, 63])
    else:
        w = _q6k_extreme(m, k, rng, list(range(-128, 128)), list(range(64)))
        w.reshape(m, k // 256, 210)[:, :, 0:192] = rng.integers(0, 256, (m, k // 256, 192), dtype=np.uint8)
    say(f"mmq q6k extreme scales ({case}) m={m} n={n} k={k}")
    x = np.where(rng.random((n, k)) < 0.5, 1.0, -1.0).astype(np.float32)
    x[0], x[1] = 1.0, -1.0   # every code +127 / -127: the largest dots
    if case == "full_range":
        x[2: n // 2] *= rng.standard_normal((n // 2 - 2, k)).astype(np.float32)
    xq = oracle.quantize_q8_1(x)
    y_ref, den = oracle.matmul("q6k", w, xq, m, n, k)
    y = host(kq.mmq_q6k(dev(w), dev(xq), m, n, k))
    check_close(y, y_ref, den, f"mmq q6k {case}")
    g = host(kq.gemv_q6k(dev(w), dev(xq[:4]), m, k, 4))
    check_close(g, y_ref[:4], den[:4], f"gemv q6k {case}")


def _sample_pairs(m, n, rng, nrand=1500):
    edge_r = sorted({0, 1, 31, 32, 63, 64, 127, 128, 129, m // 2, m - 129, m - 128, m - 2, m - 1})
    edge_t = sorted({0, 1, 31, 32, 64, 127, 128, n // 2, n - 129, n - 1})
    edge_r = [r for r in edge_r if 0 <= r < m]
    edge_t = [t for t in edge_t if 0 <= t < n]
    tok = [t for t in edge_t for _ in edge_r] + list(rng.integers(0, n, nrand))
    row = [r for _ in edge_t for r in edge_r] + list(rng.integers(0, m, nrand))
    return np.array(tok, dtype=np.int64), np.array(row, dtype=np.int64)


MMQ_OPS = list(range(len(WORKLOADS[4]["ops"])))


PREFILL_OPS = [(c, i) for c in (4, 9) for i in range(len(WORKLOADS[c]["ops"]))]


@pytest.mark.parametrize("cfg,i", PREFILL_OPS,
                         ids=[f"cfg{c}-{WORKLOADS[c]['ops'][i]['label']}" for c, i in PREFILL_OPS])
def test_mmq_prefill_sampled(kq, cfg, i):
    op = WORKLOADS[cfg]["ops"][i]
    kind = op["op"][-3:]
    m, n, k = op["m"], op["n"], op["k"]
    say(f"mmq {kind} cfg{cfg} {op['label']} m={m} n={n} k={k} (sampled)")
    w = tensor(cfg, op["w"])
    x = tensor(cfg, op["x"])
    xq_ref = oracle.quantize_q8_1(x)
    xd = dev(x)
    xq = kq.quantize_q8_1(xd)              # the path as the bench runs it
    assert np.array_equal(host(xq), xq_ref)
    y = host(mmq(kq, kind)(dev(w), xq, m, n, k))
    tok, row = _sample_pairs(m, n, np.random.default_rng(i))
    y_ref, den = oracle.matmul_pairs(kind, w, xq_ref, m, n, k, tok, row)
    check_close(y[tok, row], y_ref, den, f"cfg{cfg} {op['label']} ({tok.size} outputs)")
    assert np.all(np.isfinite(y))


PREFILL_FULL = [(4, i) for i, op in enumerate(WORKLOADS[4]["ops"]) if op["label"] in ("down", "qkv")]


@pytest.mark.parametrize("cfg,i", PREFILL_FULL,
                         ids=[f"cfg{c}-{WORKLOADS[c]['ops'][i]['label']}" for c, i in PREFILL_FULL])
def test_mmq_prefill_full(kq, cfg, i):
    """Every output of a full-size prefill launch against the oracle: down
    3584 x 18944 x 2048 (19 x 16 tiles, more than one round) and qkv
    4608 x 3584 x 2048 (24 x 16 tiles)."""
    op = WORKLOADS[cfg]["ops"][i]
    kind = op["op"][-3:]
    m, n, k = op["m"], op["n"], op["k"]
    say(f"mmq {kind} cfg{cfg} {op['label']} m={m} n={n} k={k} (every output)")
    w = tensor(cfg, op["w"])
    x = tensor(cfg, op["x"])
    xq = kq.quantize_q8_1(dev(x))
    xq_h = host(xq)
    y = host(mmq(kq, kind)(dev(w), xq, m, n, k))
    y_ref, den = oracle.matmul(kind, w, xq_h, m, n, k)
    check_close(y, y_ref, den, f"cfg{cfg} {op['label']} ({m * n} outputs)")


# Activations scaled so that every q8_1 scale d8 = amax/127 lands in the f16
# subnormal range [2^-24, 2^-14) or rounds to zero: N(0,1) values (amax about
# 2.5 to 4.5) times 2^e, with e from -10 down to -24 by row unless given.
def _subnormal_acts(seed, rows, k, exps=None):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((rows, k)).astype(np.float32)
    e = -10 - (np.arange(rows) % 15) if exps is None else np.asarray(exps)
    return (x * np.exp2(e.astype(np.float64))[:, None]).astype(np.float32)


def _d8_values(xq):
    blk = xq.reshape(-1, 36)
    return oracle.f16_bits_to_f32(blk[:, 0:2].copy().view(np.uint16).ravel())


SUBNORMAL_MMQ = [("q4k", 400, 300, 1024), ("q4k", 150, 100, 768),      # full and clamped tiles
                 ("q6k", 300, 40, 1024), ("q6k", 3584, 640, 256), ("q6k", 4096, 1024, 256)]


@pytest.mark.parametrize("kind,m,n,k", SUBNORMAL_MMQ, ids=[f"{c[0]}-m{c[1]}-n{c[2]}" for c in SUBNORMAL_MMQ])
def test_mmq_subnormal_d8(kq, kind, m, n, k):
    say(f"mmq {kind} subnormal d8 m={m} n={n} k={k}")
    w, _, _ = random_case(m + n + 5, kind, m, k, 1)
    xq = oracle.quantize_q8_1(_subnormal_acts(m + n, n, k))
    d8 = _d8_values(xq)
    assert np.all(d8 < 2.0 ** -14) and np.any((d8 > 0) & (d8 < 2.0 ** -20)) and np.any(d8 == 0)
    y_ref, den = oracle.matmul(kind, w, xq, m, n, k)
    y = host(mmq(kq, kind)(dev(w), dev(xq), m, n, k))
    check_close(y, y_ref, den, f"mmq {kind} subnormal d8")


@pytest.mark.parametrize("kind", ["q4k", "q6k"])
@pytest.mark.parametrize("batch", [1, 4])
def test_gemv_subnormal_d8(kq, kind, batch):
    m, k = 1000, 4096
    say(f"gemv {kind} subnormal d8 m={m} k={k} batch={batch}")
    w, _, res = random_case(batch + 40, kind, m, k, batch, with_residual=True)
    exps = [-17] if batch == 1 else [-10, -13, -16, -18]
    xq = oracle.quantize_q8_1(_subnormal_acts(batch, batch, k, exps))
    d8 = _d8_values(xq)
    assert np.all(d8 < 2.0 ** -14) and np.all(d8 > 0)
    res = (res * np.float32(2.0 ** -20)).astype(np.float32)
    y_ref, den = oracle.matmul(kind, w, xq, m, batch, k, residual=res)
    check_close(run_gemv(kq, kind, w, xq, m, k, batch, res), y_ref, den, f"gemv {kind} subnormal d8")


@pytest.mark.parametrize("kind", ["q4k", "q6k"])
def test_nonfinite_scale_confined(kq, kind):
    """An f16 inf scale in one weight row (d of its first superblock) and in
    one token (a q8_1 block whose values exceed 65504*127) leaves every other
    output of the GEMV and of both MMQ forms within the oracle bound."""
    m, n, k, bad_row, bad_tok = 300, 260, 1024, 11, 7
    say(f"{kind} non-finite scales confined m={m} n={n} k={k}")
    w, x, _ = random_case(4242, kind, m, k, n)
    x[bad_tok, 64] = np.float32(1e7)
    sb = w.reshape(m, k // 256, -1)
    off = 0 if kind == "q4k" else 208
    sb[bad_row, 0, off:off + 2] = np.array([0x7C00], dtype=np.uint16).view(np.uint8)
    xq = oracle.quantize_q8_1(x)
    assert _d8_values(xq[bad_tok])[2] == np.inf
    y_ref, den = oracle.matmul(kind, w, xq, m, n, k)
    keep = np.ones((n, m), dtype=bool)
    keep[bad_tok, :] = False
    keep[:, bad_row] = False
    for nn, mm in ((n, m), (100, 150)):           # full and (q4k) clamped tiles
        y = host(mmq(kq, kind)(dev(w[:mm]), dev(xq[:nn]), mm, nn, k))
        kp = keep[:nn, :mm]
        check_close(y[kp], y_ref[:nn, :mm][kp], den[:nn, :mm][kp], f"mmq {kind} n{nn} m{mm}")
    g = run_gemv(kq, kind, w, xq[5:9], m, k, 4)
    kp = keep[5:9]
    check_close(g[kp], y_ref[5:9][kp], den[5:9][kp], f"gemv {kind} batch 4")


@pytest.mark.parametrize("kind", ["q4k", "q6k"])
def test_mmq_matches_gemv_columns(kq, kind):
    m, n, k = 777, 5, 4096
    say(f"mmq {kind} vs gemv m={m} n={n} k={k}")
    w, x, _ = random_case(99, kind, m, k, n)
    xq = oracle.quantize_q8_1(x)
    wd, xd = dev(w), dev(xq)
    y = host(mmq(kq, kind)(wd, xd, m, n, k))
    y_ref, den = oracle.matmul(kind, w, xq, m, n, k)
    gemv = kq.gemv_q4k if kind == "q4k" else kq.gemv_q6k
    for t in range(n):
        g = host(gemv(wd, xd[t:t + 1], m, k, 1))[0]
        check_close(g, y_ref[t], den[t], f"gemv token {t}")
        check_close(y[t], y_ref[t], den[t], f"mmq token {t}")


@pytest.mark.parametrize("kind", ["q4k", "q6k"])
def test_mmq_deterministic(kq, kind):
    m, n, k = 512, 256, 3584
    say(f"mmq {kind} determinism m={m} n={n} k={k}")
    w, x, _ = random_case(6, kind, m, k, n)
    xq = oracle.quantize_q8_1(x)
    wd, xd = dev(w), dev(xq)
    a = host(mmq(kq, kind)(wd, xd, m, n, k))
    for _ in range(3):
        assert np.array_equal(a, host(mmq(kq, kind)(wd, xd, m, n, k)))


# ------------------------------------------------------------- K split -----

# Products too small to fill the device take the K split when given the
# workspace: the value projection 512 x 3584 at 2048 and 512 tokens, twice the
# rows, ragged tiles, the least k that splits (four superblocks), and the
# prefill down projection (448 tiles of 128 tokens, split in four).
KSPLIT = [(512, 2048, 3584), (512, 512, 3584), (1024, 2048, 3584), (300, 100, 2048), (129, 70, 1024),
          (33, 5, 1280), (3584, 2048, 18944)]


@pytest.mark.parametrize("m,n,k", KSPLIT, ids=[f"m{c[0]}-n{c[1]}-k{c[2]}" for c in KSPLIT])
def test_mmq_q6k_ksplit(kq, m, n, k):
    say(f"mmq q6k K split m={m} n={n} k={k}")
    nb = kq.kq_mmq_q6k_workspace_bytes(m, n, k)
    assert nb > 0 and nb % (m * n * 4) == 0 and nb // (m * n * 4) <= 3
    w, x, _ = random_case(m * 7 + n + k, "q6k", m, k, n)
    xq = oracle.quantize_q8_1(x)
    wd, xd = dev(w), dev(xq)
    ws = torch.full((nb,), 0x7F, dtype=torch.uint8, device="cuda")      # stale contents
    y = host(kq.mmq_q6k_ws(wd, xd, m, n, k, ws=ws))
    assert np.array_equal(y, host(kq.mmq_q6k_ws(wd, xd, m, n, k, ws=ws))), "not reproducible"
    if m * n * k <= 1 << 34:
        y_ref, den = oracle.matmul("q6k", w, xq, m, n, k)
        check_close(y, y_ref, den, f"mmq q6k split m{m} n{n} k{k}")
    else:
        tok, row = _sample_pairs(m, n, np.random.default_rng(m))
        y_ref, den = oracle.matmul_pairs("q6k", w, xq, m, n, k, tok, row)
        check_close(y[tok, row], y_ref, den, f"mmq q6k split m{m} n{n} k{k} ({tok.size} outputs)")
    # a workspace one byte short: the unsplit product, bit for bit
    short = kq.mmq_q6k_ws(wd, xd, m, n, k, ws=ws[: nb - 1])
    assert torch.equal(short, kq.mmq_q6k(wd, xd, m, n, k))


# Q4_K: the prefill down projection (304 tiles of 192 x 128, 1.2 rounds of
# one workgroup per CU: the 48 tiles past the first round in five K ranges),
# QKV (384 tiles: the last 128 in two), gate-sized grids whose last round is
# split, and small products split up to eight ways, one of them on the
# clamped tile form.
KSPLIT4 = [(3584, 2048, 18944), (4608, 2048, 3584), (400, 300, 4096), (129, 70, 1024),
           (1000, 1000, 2560), (7168, 2048, 1024)]


@pytest.mark.parametrize("m,n,k", KSPLIT4, ids=[f"m{c[0]}-n{c[1]}-k{c[2]}" for c in KSPLIT4])
def test_mmq_q4k_ksplit(kq, m, n, k):
    say(f"mmq q4k K split m={m} n={n} k={k}")
    nb = kq.kq_mmq_q4k_workspace_bytes(m, n, k)
    assert nb > 0 and nb % (n * 4) == 0 and nb <= 7 * m * n * 4   # ranges of the split rows
    w, x, _ = random_case(m * 5 + n + k, "q4k", m, k, n)
    xq = oracle.quantize_q8_1(x)
    wd, xd = dev(w), dev(xq)
    ws = torch.full((nb,), 0x7F, dtype=torch.uint8, device="cuda")      # stale contents
    y = host(kq.mmq_q4k_ws(wd, xd, m, n, k, ws=ws))
    assert np.array_equal(y, host(kq.mmq_q4k_ws(wd, xd, m, n, k, ws=ws))), "not reproducible"
    if m * n * k <= 1 << 36:
        y_ref, den = oracle.matmul("q4k", w, xq, m, n, k)
        check_close(y, y_ref, den, f"mmq q4k split m{m} n{n} k{k}")
    else:
        tok, row = _sample_pairs(m, n, np.random.default_rng(m))
        y_ref, den = oracle.matmul_pairs("q4k", w, xq, m, n, k, tok, row)
        check_close(y[tok, row], y_ref, den, f"mmq q4k split m{m} n{n} k{k} ({tok.size} outputs)")
    # a workspace one byte short: the best split that fits (fewer ranges),
    # still within the bound; no workspace: the unsplit product, bit for bit
    short = host(kq.mmq_q4k_ws(wd, xd, m, n, k, ws=ws[: nb - 1]))
    if m * n * k <= 1 << 36:
        check_close(short, y_ref, den, f"mmq q4k split, short workspace")
    else:
        check_close(short[tok, row], y_ref, den, f"mmq q4k split, short workspace")
    none = torch.empty((n, m), device="cuda")
    kq.kq_mmq_q4k_ws(wd, xd, none, m, n, k, None, 0)
    assert torch.equal(none, kq.mmq_q4k(wd, xd, m, n, k))


def test_mmq_q4k_ksplit_sizes(kq):
    """The split covers only the row blocks past the whole rounds of one
    workgroup per CU: gate 18944 x 3584 at 2048 tokens (1584 tiles: 6 rounds
    and 48 tiles) splits its last 512 rows into five ranges.  A single
    superblock and a grid of exactly one round are not split."""
    assert kq.kq_mmq_q4k_workspace_bytes(18944, 2048, 3584) == 4 * 2048 * 512 * 4
    assert kq.kq_mmq_q4k_workspace_bytes(7168, 2048, 256) == 0
    assert kq.kq_mmq_q4k_workspace_bytes(6144, 1024, 4096) == 0   # 32 x 8 = 256 tiles: one round


def test_mmq_q6k_ksplit_not_taken_when_tiles_fill(kq):
    """A product whose 128-token tiles already give every CU two workgroups
    needs no workspace and gives the kq_mmq_q6k bits."""
    m, n, k = 4096, 1024, 512
    say(f"mmq q6k no split m={m} n={n} k={k}")
    assert kq.kq_mmq_q6k_workspace_bytes(m, n, k) == 0
    w, x, _ = random_case(31, "q6k", m, k, n)
    wd, xd = dev(w), dev(oracle.quantize_q8_1(x))
    assert torch.equal(kq.mmq_q6k_ws(wd, xd, m, n, k), kq.mmq_q6k(wd, xd, m, n, k))


def test_mmq_q6k_ws_rejects_bad_workspace(kq):
    m, n, k = 512, 256, 3584
    say("mmq q6k workspace errors")
    nb = kq.kq_mmq_q6k_workspace_bytes(m, n, k)
    w, x, _ = random_case(32, "q6k", m, k, n)
    wd, xd = dev(w), dev(oracle.quantize_q8_1(x))
    y = torch.full((n, m), 7.0, device="cuda")
    ws = torch.empty(nb + 64, dtype=torch.uint8, device="cuda")
    with pytest.raises(kq.KQError, match="misaligned workspace"):
        kq.kq_mmq_q6k_ws(wd, xd, y, m, n, k, ws.data_ptr() + 4, nb, None)
    with pytest.raises(kq.KQError, match="overlaps"):
        kq.kq_mmq_q6k_ws(wd, xd, y, m, n, k, y, nb, None)
    assert torch.all(y == 7.0).item()


# ------------------------------------------------------ error handling ------

def test_bad_arguments_launch_nothing(kq):
    say("argument errors on real buffers")
    w, x, _ = random_case(1, "q4k", 64, 512, 2)
    xq = dev(oracle.quantize_q8_1(x))
    wd = dev(w)
    y = torch.full((2, 64), 7.0, device="cuda")
    for call in (
        lambda: kq.kq_gemv_q4k(wd, xq, y, None, 64, 500, 2),
        lambda: kq.kq_gemv_q4k(wd, xq, y, None, 64, 512, 9),
        lambda: kq.kq_gemv_q6k(wd, xq, y, y[:, 1:], 64, 512, 2),
        lambda: kq.kq_mmq_q4k(wd, xq, wd, 64, 2, 512),
        lambda: kq.kq_mmq_q6k(wd, xq, wd, 64, 2, 512),
        lambda: kq.kq_mmq_q6k(wd, xq, y, 64, 2, 500),
    ):
        with pytest.raises(kq.KQError):
            call()
    assert torch.all(y == 7.0).item()


# ----------------------------------------------------- segmented GEMV ----

SEG_CASES = [
    # (rows per segment, k, batch, residual on segments)
    ((4096, 1024, 1024), 4096, 1, (False, False, False)),
    ((4096, 1024, 1024), 4096, 4, (True, False, True)),
    ((2048, 512, 512), 4096, 8, (False, True, False)),
    ((0, 1, 7, 33, 300), 768, 3, (False, True, True, False, True)),
    ((700, 300), 14336, 4, (True, False)),          # activation exceeds 64 KB: one launch per segment
    ((14336, 14336), 4096, 1, (False, False)),      # gate and up as separate tensors
]


@pytest.mark.parametrize("ms,k,batch,res_on", SEG_CASES,
                         ids=[f"{'-'.join(map(str, c[0]))}-k{c[1]}-b{c[2]}" for c in SEG_CASES])
def test_gemv_seg_matches_single(kq, ms, k, batch, res_on):
    say(f"segmented gemv m={ms} k={k} batch={batch}")
    from kq_inputs import q4k_weights

    x = activations(61, 0, batch, k)
    xq_h = oracle.quantize_q8_1(x)
    xq = dev(xq_h)
    ws, res, ys_ref = [], [], []
    for s, m in enumerate(ms):
        wh = q4k_weights(61, 10 + s, m, k)
        rh = residual(61, 30 + s, batch, m) if res_on[s] else None
        ws.append(dev(wh))
        res.append(dev(rh) if rh is not None else None)
        if m:
            y_ref, den = oracle.matmul("q4k", wh, xq_h, m, batch, k, residual=rh)
            ys_ref.append((y_ref, den))
        else:
            ys_ref.append(None)
    ys = kq.gemv_q4k_seg(ws, ms, xq, k, batch, residuals=res)
    for s, m in enumerate(ms):
        if not m:
            continue
        single = kq.gemv_q4k(ws[s], xq, m, k, batch, residual=res[s])
        assert torch.equal(ys[s], single), f"segment {s} differs from the single-tensor call"
        check_close(host(ys[s]), ys_ref[s][0], ys_ref[s][1], f"segment {s} m={m}")


def test_gemv_seg_in_place_residual(kq):
    say("segmented gemv, residual in place")
    from kq_inputs import q4k_weights

    k, batch, ms = 2048, 2, (1000, 24)
    x = activations(62, 0, batch, k)
    xq_h = oracle.quantize_q8_1(x)
    ws = [dev(q4k_weights(62, 10 + s, m, k)) for s, m in enumerate(ms)]
    rs = [residual(62, 30 + s, batch, m) for s, m in enumerate(ms)]
    ys = [dev(r) for r in rs]
    kq.gemv_q4k_seg(ws, ms, dev(xq_h), k, batch, residuals=ys, outs=ys)
    for s, m in enumerate(ms):
        y_ref, den = oracle.matmul("q4k", ws[s].cpu().numpy(), xq_h, m, batch, k, residual=rs[s])
        check_close(host(ys[s]), y_ref, den, f"in place segment {s}")
