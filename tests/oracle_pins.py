"""Pins of the CPU oracle to facts outside itself.

Each ``pin_*`` function takes the ``oracle`` module and raises
``AssertionError`` when the oracle disagrees with something the pages or the
mathematics fix: hand-worked values (tests/golden), numpy's binary16
conversion, the exact-rational checker ``oracle/exact.py``, closed forms,
invariants and structural identities.  ``test_oracle_pins.py`` runs them on
the real oracle; ``test_oracle_mutants.py`` runs them on deliberately broken
builds of the oracle source and requires every mutant to fail at least one.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np

from conftest import load_golden, q4k_block_from_fields, q6k_block_from_fields
from kq_inputs import activations, q4k_weights, q6k_weights, random_case, residual
from oracle import exact

XHAT_ONE = 131064 / 131072  # f16(1/127) * 127: the dequantised code for x = 1.0


def _q8_fields(xq_row: np.ndarray, nblocks: int):
    blk = xq_row.reshape(nblocks, 36)
    d = blk[:, 0:2].copy().view(np.uint16).ravel()
    s = blk[:, 2:4].copy().view(np.uint16).ravel()
    q = blk[:, 4:36].view(np.int8)
    return d, s, q


def _xhat_numpy(xq: np.ndarray, rows: int, k: int) -> np.ndarray:
    """Dequantised activations via numpy's own binary16 decode (f64)."""
    blk = xq.reshape(rows, k // 32, 36)
    d = blk[:, :, 0:2].copy().view(np.float16)[..., 0].astype(np.float64)
    q = blk[:, :, 4:36].view(np.int8).astype(np.float64)
    return (d[:, :, None] * q).reshape(rows, k)


# ------------------------------------------------------------------ f16 ----

def pin_f16_encode_vs_numpy(O):
    rng = np.random.default_rng(11)
    parts = [
        rng.standard_normal(20000).astype(np.float32),
        (rng.standard_normal(20000) * 1e-5).astype(np.float32),   # f16 subnormal range
        (rng.standard_normal(5000) * 3e4).astype(np.float32),     # near overflow
        (rng.standard_normal(5000) * 1e-8).astype(np.float32),    # below f16 subnormals
        np.array([0.0, -0.0, 65504.0, 65519.996, 65520.0, 1e6, -1e6, 2.0 ** -24,
                  2.0 ** -25, 3 * 2.0 ** -26, 2.0 ** -14, 2.0 ** -14 * (1 - 2.0 ** -11)],
                 dtype=np.float32),
    ]
    # exact ties between f16 neighbours
    h = np.arange(0x0001, 0x7bff, 7, dtype=np.uint16)
    lo = h.view(np.float16).astype(np.float64)
    hi = (h + 1).view(np.float16).astype(np.float64)
    parts.append(((lo + hi) / 2).astype(np.float32))
    x = np.concatenate(parts)
    x = np.concatenate([x, -x])
    got = O.f32_to_f16_bits(x)
    with np.errstate(over="ignore"):   # values past the f16 range encode as inf on purpose
        want = x.astype(np.float16).view(np.uint16)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, f"f16 encode differs at {x[bad[:5]]}: {got[bad[:5]]} vs {want[bad[:5]]}"


def pin_f16_decode_vs_numpy(O):
    h = np.arange(0, 65536, dtype=np.uint32).astype(np.uint16)
    f = h.view(np.float16)
    keep = ~np.isnan(f)
    got = O.f16_bits_to_f32(h[keep])
    want = f[keep].astype(np.float32)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), "f16 decode differs from numpy"


# ----------------------------------------------------------------- q8_1 ----

def _check_q8_golden(O, name):
    g = load_golden(name)
    x = np.array(g["x"], dtype=np.float32)
    xq = O.quantize_q8_1(x[None, :])
    d, s, q = _q8_fields(xq[0], 1)
    assert int(d[0]) == g["d_bits"], f"{name}: d bits {d[0]:#x} != {g['d_bits']:#x}"
    assert int(s[0]) == g["s_bits"], f"{name}: s bits {s[0]:#x} != {g['s_bits']:#x}"
    assert list(q[0].astype(int)) == list(g["codes"]), f"{name}: codes {list(q[0])}"


def pin_q8_golden_e1(O):
    _check_q8_golden(O, "e1_q8_1_ties.txt")


def pin_q8_golden_e2(O):
    _check_q8_golden(O, "e2_q8_1_ramp.txt")


def _adversarial_blocks(seed=5, nrand=200):
    rng = np.random.default_rng(seed)
    blocks = []
    for scale in (1.0, 1e-3, 1e3, 1e-6, 3e-8, 7.0):
        blocks.append((rng.standard_normal((nrand // 6, 32)) * scale).astype(np.float32))
    # exact ties: amax = 127 * 2^e makes d = 2^e and every half-integer a tie
    for e in (-3, 0, 2):
        t = rng.integers(-120, 120, size=(20, 32)).astype(np.float64) + 0.5
        t[:, 0] = 127.0
        blocks.append((t * 2.0 ** e).astype(np.float32))
    # all-zero block, single nonzero, negative amax, constant blocks
    z = np.zeros((4, 32), dtype=np.float32)
    z[1, 7] = -3.25
    z[2, :] = 1.0
    z[3, :] = -0.001
    blocks.append(z)
    return np.concatenate(blocks)


def _tree_sum_f32(x: np.ndarray) -> np.ndarray:
    a = x.astype(np.float32).copy()
    h = 16
    while h >= 1:
        a[:, :h] = a[:, :h] + a[:, h:2 * h]
        h //= 2
    return a[:, 0]


def _distinguishing_blocks(seed=13, n=200000, keep=40):
    """Blocks on which plausible alternative readings give other bits:
    x/d instead of x*(1/d) for the codes, and a sequential (or wider) sum
    instead of the f32 tree for the source sum.  Found by a seeded search."""
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((n, 32)) * np.exp(rng.uniform(-3, 3, (n, 1)))).astype(np.float32)
    amax = np.abs(x).max(axis=1)
    d = amax / np.float32(127.0)
    idv = np.float32(1.0) / d
    q_mul = np.sign(x) * np.floor(np.abs(x * idv[:, None]).astype(np.float64) + 0.5)
    q_div = np.sign(x) * np.floor(np.abs(x / d[:, None]).astype(np.float64) + 0.5)
    div_rows = np.nonzero(np.any(q_mul != q_div, axis=1))[0][:keep]
    tree = _tree_sum_f32(x).astype(np.float16)
    seq = np.cumsum(x, axis=1, dtype=np.float32)[:, -1].astype(np.float16)
    wide = x.astype(np.float64).sum(axis=1).astype(np.float32).astype(np.float16)
    sum_rows = np.nonzero((tree != seq) | (tree != wide))[0][:keep]
    assert div_rows.size >= 5 and sum_rows.size >= 5
    # hand-built: the f32 tree rounds up to the f16 midpoint 1 + 3*2^-11 (which
    # then rounds to even, upwards) while the exact sum lies just below it
    hb = np.zeros((1, 32), dtype=np.float32)
    hb[0, 0] = np.float32(1 + 3 * 2.0 ** -11 - 2.0 ** -23)
    hb[0, 16] = np.float32(2.0 ** -24 + 2.0 ** -30)
    hb[0, 8] = np.float32(-2.0 ** -25)
    return np.concatenate([x[div_rows], x[sum_rows], hb])


def pin_q8_vs_exact(O):
    blocks = np.concatenate([_adversarial_blocks(), _distinguishing_blocks()])
    xq = O.quantize_q8_1(blocks.reshape(-1, 32))
    for i, xb in enumerate(blocks):
        d, s, q = _q8_fields(xq[i], 1)
        ed, es, eq = exact.quantize_block(xb)
        assert int(d[0]) == ed, f"block {i}: d {d[0]:#x} != {ed:#x}"
        assert int(s[0]) == es, f"block {i}: s {s[0]:#x} != {es:#x}"
        assert list(q[0].astype(int)) == eq, f"block {i}: codes differ"


def pin_q8_invariants(O):
    rng = np.random.default_rng(7)
    x = rng.standard_normal((64, 32 * 8)).astype(np.float32)
    x[3, :32] = 0.0
    xq = O.quantize_q8_1(x)
    nb = x.shape[1] // 32
    for r in range(x.shape[0]):
        d16, s16, q = _q8_fields(xq[r], nb)
        xb = x[r].reshape(nb, 32).astype(np.float64)
        amax = np.abs(xb).max(axis=1)
        d32 = (amax.astype(np.float32) / np.float32(127.0)).astype(np.float64)
        qi = q.astype(np.int64)
        assert np.all(np.abs(qi) <= 127)
        for b in range(nb):
            if amax[b] == 0:
                assert np.all(qi[b] == 0) and d16[b] == 0
                continue
            i = int(np.argmax(np.abs(xb[b])))
            assert abs(qi[b, i]) == 127 and np.sign(qi[b, i]) == np.sign(xb[b, i])
            err = np.abs(xb[b] - d32[b] * qi[b])
            assert np.all(err <= d32[b] * (0.5 + 2.0 ** -14)), "reconstruction error too large"
        # f16 of the scale and of the source sum
        assert np.array_equal(d16, d32.astype(np.float32).astype(np.float16).view(np.uint16))
        ssum = xb.sum(axis=1)
        s_val = s16.view(np.float16).astype(np.float64)
        assert np.all(np.abs(s_val - ssum) <= np.abs(ssum) * 2.0 ** -10 + 32 * 2.0 ** -24 * np.abs(xb).sum(axis=1) + 2.0 ** -24)
    # power-of-two scaling: same codes, scaled f16 scale and sum
    for e in (-4, 3):
        xq2 = O.quantize_q8_1(x * np.float32(2.0 ** e))
        for r in range(x.shape[0]):
            d1, s1, q1 = _q8_fields(xq[r], nb)
            d2, s2, q2 = _q8_fields(xq2[r], nb)
            assert np.array_equal(q1, q2), "codes changed under power-of-two scaling"
            assert np.array_equal(d1.view(np.float16).astype(np.float64) * 2.0 ** e,
                                  d2.view(np.float16).astype(np.float64))
            sv1 = s1.view(np.float16).astype(np.float64)
            sv2 = s2.view(np.float16).astype(np.float64)
            normal = (np.abs(sv1) >= 2.0 ** -14) & (np.abs(sv1 * 2.0 ** e) >= 2.0 ** -14)
            assert np.array_equal(sv1[normal] * 2.0 ** e, sv2[normal])


def pin_q8_sum_is_tree(O):
    """The source sum is the pairwise tree (a[i] += a[i+h], h = 16..1)
    rounded to f16, checked against an explicit f32 tree in numpy."""
    rng = np.random.default_rng(9)
    x = (rng.standard_normal((500, 32)) * np.exp(rng.standard_normal((500, 1)) * 3)).astype(np.float32)
    x = np.concatenate([x, _distinguishing_blocks()])
    xq = O.quantize_q8_1(x)
    want = _tree_sum_f32(x).astype(np.float16).view(np.uint16)
    got = xq[:, 2:4].copy().view(np.uint16).ravel()
    assert np.array_equal(got, want), "source sum is not the f32 tree sum"


# ------------------------------------------------------------ matmuls ------

def _one_superblock_y(O, kind, block, x_fill):
    x = np.full((1, 256), x_fill, dtype=np.float32)
    xq = O.quantize_q8_1(x)
    y, den = O.matmul(kind, block[None, :], xq, 1, 1, 256)
    return y[0, 0], den[0, 0]


def pin_e3_q4k_uniform(O):
    g = load_golden("e3_q4k_uniform.txt")
    b = q4k_block_from_fields(g["d_bits"], g["dmin_bits"], g["scales"], [g["qs_fill"]] * 128)
    w = O.dequant("q4k", b[None, :], 1, 256)[0]
    assert np.array_equal(w, np.repeat(np.array(g["w_subblock"], dtype=np.float32), 32))
    y, den = _one_superblock_y(O, "q4k", b, g["x_fill"])
    assert y == g["y"], f"E3 y = {y!r}"
    assert den == abs(g["y"])


def pin_e4_q4k_zero_codes(O):
    g = load_golden("e4_q4k_zero_codes.txt")
    b = q4k_block_from_fields(g["d_bits"], g["dmin_bits"], g["scales"], [g["qs_fill"]] * 128)
    w = O.dequant("q4k", b[None, :], 1, 256)[0]
    assert np.array_equal(w, np.repeat(np.array(g["w_subblock"], dtype=np.float32), 32))
    y, _ = _one_superblock_y(O, "q4k", b, g["x_fill"])
    assert y == g["y"], f"E4 y = {y!r}"


def pin_e5_q6k_uniform(O):
    g = load_golden("e5_q6k_uniform.txt")
    b = q6k_block_from_fields(g["d_bits"], g["scales"], [g["ql_fill"]] * 128, [g["qh_fill"]] * 64)
    y, _ = _one_superblock_y(O, "q6k", b, g["x_fill"])
    assert y == g["y"], f"E5 y = {y!r}"


def pin_e6_q6k_groups(O):
    g = load_golden("e6_q6k_groups.txt")
    ql = np.repeat(np.array(g["ql_quarters"], dtype=np.uint8), 32)
    qh = np.repeat(np.array(g["qh_halves"], dtype=np.uint8), 32)
    b = q6k_block_from_fields(g["d_bits"], g["scales"], ql, qh)
    w = O.dequant("q6k", b[None, :], 1, 256)[0]
    v = np.arange(256)
    want = np.array(g["scales"])[v // 16] * np.array(g["group_q"])[v // 32]
    assert np.array_equal(w, want.astype(np.float32)), f"E6 weights {w[::32]}"


def pin_e7_q4k_high_scales(O):
    g = load_golden("e7_q4k_high_scales.txt")
    qs = np.repeat(np.array(g["qs_chunks"], dtype=np.uint8), 32)
    b = q4k_block_from_fields(g["d_bits"], g["dmin_bits"], g["scales"], qs)
    w = O.dequant("q4k", b[None, :], 1, 256)[0]
    assert np.array_equal(w, np.repeat(np.array(g["w_subblock"], dtype=np.float32), 32)), \
        f"E7 weights {w[::32]}"
    y, _ = _one_superblock_y(O, "q4k", b, g["x_fill"])
    assert y == g["y"], f"E7 y = {y!r}"


def _mag(O, kind, w, xq, m, n, k):
    W = O.dequant(kind, w, m, k).astype(np.float64)
    X = _xhat_numpy(xq, n, k)
    return np.abs(X) @ np.abs(W).T  # [n, m]


def pin_identity_q4k(O):
    """Dequantise-then-dot equals the integer-factored form within the one
    f32 rounding of the Q4_K subtraction: 2^-24 * sum|w*xh|."""
    for seed, (m, n, k) in enumerate([(8, 3, 512), (5, 2, 1024), (3, 4, 256)]):
        w, x, _ = random_case(seed, "q4k", m, k, n)
        xq = O.quantize_q8_1(x)
        y, _ = O.matmul("q4k", w, xq, m, n, k)
        y2 = O.matmul_factored("q4k", w, xq, m, n, k)
        mag = _mag(O, "q4k", w, xq, m, n, k)
        assert np.all(np.abs(y - y2) <= 2.0 ** -24 * mag * 1.0001 + 1e-300), \
            f"identity broken (seed {seed}): {np.max(np.abs(y - y2) / mag)}"


def pin_identity_q6k(O):
    """Q6_K dequantisation is exact in f32, so both forms agree to f64
    summation-order rounding."""
    for seed, (m, n, k) in enumerate([(8, 3, 512), (4, 2, 768)]):
        w, x, _ = random_case(seed, "q6k", m, k, n)
        xq = O.quantize_q8_1(x)
        y, _ = O.matmul("q6k", w, xq, m, n, k)
        y2 = O.matmul_factored("q6k", w, xq, m, n, k)
        mag = _mag(O, "q6k", w, xq, m, n, k)
        assert np.all(np.abs(y - y2) <= 1e-13 * mag), "Q6_K identity broken"


def _exact_check(O, kind, w, x, m, n, k, res=None, rows=None):
    xq = O.quantize_q8_1(x)
    y, den = O.matmul(kind, w, xq, m, n, k, residual=res)
    rows = range(m) if rows is None else rows
    for t in range(n):
        for r in rows:
            ex, mag = exact.dot(kind, w[r], xq[t], k, None if res is None else res[t, r])
            assert abs(Fraction(float(y[t, r])) - ex) <= Fraction(1e-12) * mag, \
                f"{kind} output ({t},{r}) off: {float(y[t, r])} vs {float(ex)}"
            # den = sum_j |T_j| + |residual|, exactly up to f64 rounding
            xhat = exact.activation(xq[t], k)
            wv = exact.weights(kind, w[r], k)
            dsum = sum(abs(sum(wv[32 * j + i] * xhat[32 * j + i] for i in range(32)))
                       for j in range(k // 32))
            if res is not None:
                dsum += abs(Fraction(float(res[t, r])))
            assert abs(Fraction(float(den[t, r])) - dsum) <= Fraction(1e-12) * mag


def pin_exact_rational_cfg0(O):
    """Workload 0 (256x1024 Q4_K, seed 0): a sample of 12 rows checked exactly."""
    from kq_inputs import tensor
    w = tensor(0, "w")
    x = tensor(0, "x")
    _exact_check(O, "q4k", w, x, 256, 1, 1024, rows=[0, 1, 17, 64, 100, 127, 128, 129, 200, 201, 254, 255])


def pin_exact_rational_random(O):
    w, x, r = random_case(21, "q4k", 3, 512, 2, with_residual=True)
    _exact_check(O, "q4k", w, x, 3, 2, 512, res=r)
    w, x, r = random_case(22, "q6k", 3, 512, 2, with_residual=True)
    _exact_check(O, "q6k", w, x, 3, 2, 512, res=r)


def pin_closed_form_q6k_zero(O):
    """All Q6_K codes 32 (q - 32 = 0): y = 0 exactly, or exactly the residual."""
    rng = np.random.default_rng(3)
    m, n, k = 5, 2, 512
    w = q6k_weights(31, 0, m, k).reshape(m, k // 256, 210)
    w[:, :, 0:128] = 0x00
    w[:, :, 128:192] = 0xAA
    w = w.reshape(m, -1)
    x = rng.standard_normal((n, k)).astype(np.float32)
    xq = O.quantize_q8_1(x)
    y, den = O.matmul("q6k", w, xq, m, n, k)
    assert np.all(y == 0.0) and np.all(den == 0.0)
    res = rng.standard_normal((n, m)).astype(np.float32)
    y, den = O.matmul("q6k", w, xq, m, n, k, residual=res)
    assert np.array_equal(y, res.astype(np.float64))
    assert np.array_equal(den, np.abs(res).astype(np.float64))


def pin_closed_form_q4k_min_only(O):
    """Q4_K with every sub-block scale 0 and every min m = 37: w = -dmin*37
    whatever the codes, so y = -dmin*37 * sum_i xh_i (one superblock per row)."""
    m, n, k = 4, 3, 256
    w = q4k_weights(41, 0, m, k).reshape(m, 1, 144)
    w[:, :, 4:8] = 0x00
    w[:, :, 8:12] = 0xA5
    w[:, :, 12:16] = 0x50
    w = w.reshape(m, -1)
    x = activations(41, 1, n, k)
    xq = O.quantize_q8_1(x)
    y, _ = O.matmul("q4k", w, xq, m, n, k)
    dmin = w[:, 2:4].copy().view(np.float16)[:, 0].astype(np.float64)
    xs = _xhat_numpy(xq, n, k).sum(axis=1)
    want = -(dmin[None, :] * 37.0) * xs[:, None]
    assert np.all(np.abs(y - want) <= 1e-12 * np.abs(want) + 1e-300), "min-only closed form broken"


def pin_q6k_scale_negation(O):
    m, n, k = 6, 2, 512
    w, x, _ = random_case(51, "q6k", m, k, n)
    xq = O.quantize_q8_1(x)
    y, _ = O.matmul("q6k", w, xq, m, n, k)
    w2 = w.reshape(m, k // 256, 210).copy()
    sc = w2[:, :, 192:208].view(np.int8)
    sc[...] = -sc
    y2, _ = O.matmul("q6k", w2.reshape(m, -1), xq, m, n, k)
    assert np.array_equal(y2, -y), "negating the Q6_K scales does not negate y"


def pin_structure(O):
    rng = np.random.default_rng(61)
    for kind in ("q4k", "q6k"):
        m, n, k = 7, 3, 768
        w, x, res = random_case(62, kind, m, k, n, with_residual=True)
        xq = O.quantize_q8_1(x)
        y, den = O.matmul(kind, w, xq, m, n, k)
        # row permutation permutes the outputs exactly
        perm = rng.permutation(m)
        yp, _ = O.matmul(kind, w[perm], xq, m, n, k)
        assert np.array_equal(yp, y[:, perm])
        # batch column b equals the single-column result on x_b
        for b in range(n):
            yb, _ = O.matmul(kind, w, xq[b:b + 1], m, 1, k)
            assert np.array_equal(yb[0], y[b])
        # splitting K at a superblock boundary: partial sums add up
        bs = 144 if kind == "q4k" else 210
        w3 = w.reshape(m, k // 256, bs)
        k1 = 512
        wa = w3[:, : k1 // 256].reshape(m, -1)
        wb = w3[:, k1 // 256:].reshape(m, -1)
        ya, _ = O.matmul(kind, wa, O.quantize_q8_1(x[:, :k1]), m, n, k1)
        yb2, _ = O.matmul(kind, wb, O.quantize_q8_1(x[:, k1:]), m, n, k - k1)
        mag = _mag(O, kind, w, xq, m, n, k)
        assert np.all(np.abs(ya + yb2 - y) <= 1e-13 * mag)
        # the residual adds once to y and to the tolerance denominator
        yr, denr = O.matmul(kind, w, xq, m, n, k, residual=res)
        assert np.all(np.abs(yr - y - res) <= 1e-13 * (mag + np.abs(res)))
        assert np.all(np.abs(denr - den - np.abs(res)) <= 1e-13 * (den + np.abs(res)))
        # sampled outputs are the same numbers
        tok = rng.integers(0, n, 10)
        row = rng.integers(0, m, 10)
        ys, dens = O.matmul_pairs(kind, w, xq, m, n, k, tok, row, residual=res)
        assert np.array_equal(ys, yr[tok, row]) and np.array_equal(dens, denr[tok, row])


def pin_q8_roundtrip_dequant(O):
    """Dequantised q8_1 activations are f16(d) * code, exactly."""
    x = activations(71, 0, 3, 512)
    xq = O.quantize_q8_1(x)
    got = O.dequant_q8_1(xq, 3, 512).astype(np.float64)
    assert np.array_equal(got, _xhat_numpy(xq, 3, 512))


PINS = [
    pin_f16_encode_vs_numpy,
    pin_f16_decode_vs_numpy,
    pin_q8_golden_e1,
    pin_q8_golden_e2,
    pin_q8_vs_exact,
    pin_q8_invariants,
    pin_q8_sum_is_tree,
    pin_q8_roundtrip_dequant,
    pin_e3_q4k_uniform,
    pin_e4_q4k_zero_codes,
    pin_e5_q6k_uniform,
    pin_e6_q6k_groups,
    pin_e7_q4k_high_scales,
    pin_identity_q4k,
    pin_identity_q6k,
    pin_exact_rational_cfg0,
    pin_exact_rational_random,
    pin_closed_form_q6k_zero,
    pin_closed_form_q4k_min_only,
    pin_q6k_scale_negation,
    pin_structure,
]


# ------------------------------------------------------------- producers ----
# leone-cuda "CUDA kernel design": RMSNorm and SwiGLU write their q8_1 blocks
# themselves.  The reduction order and the exponential are this oracle's
# readings (see the oracle's header); the pins below fix them to hand-worked
# values, closed forms and the f64 definitions.

def _q8_block_fields(xq_row, b):
    blk = xq_row[36 * b: 36 * (b + 1)]
    d_bits = int(blk[0]) | (int(blk[1]) << 8)
    s_bits = int(blk[2]) | (int(blk[3]) << 8)
    return d_bits, s_bits, blk[4:].view(np.int8)


def pin_e8_rms_reduction_order(O):
    g = load_golden("e8_rms_reduction_order.txt")
    h = np.zeros(g["n"], dtype=np.float32)
    for i, v in zip(g["nonzero_index"], g["nonzero_value"]):
        h[i] = v
    assert O.rms_sumsq(h) == g["sumsq"]


def pin_e9_rmsnorm_constant_row(O):
    g = load_golden("e9_rmsnorm_constant_row.txt")
    n = g["n"]
    x = np.full((1, n), g["x_fill"], dtype=np.float32)
    y, xq = O.rmsnorm_q8_1(x, np.full(n, g["g_fill"], dtype=np.float32), g["eps"])
    assert np.all(y == g["y"])
    for b in range(n // 32):
        d_bits, s_bits, codes = _q8_block_fields(xq[0], b)
        assert d_bits == g["d_bits"] and s_bits == g["s_bits"]
        assert np.all(codes == g["code"])


def pin_e10_swiglu_saturated(O):
    g = load_golden("e10_swiglu_saturated.txt")
    gate = np.full((1, 64), g["gate"], dtype=np.float32)
    gate[0, 32:] = 0.0
    up = np.full((1, 64), g["up"], dtype=np.float32)
    y, xq = O.swiglu_q8_1(gate, up)
    assert np.all(y[0, :32] == g["y"]) and np.all(y[0, 32:] == 0.0)
    d_bits, s_bits, codes = _q8_block_fields(xq[0], 0)
    assert d_bits == g["d_bits"] and s_bits == g["s_bits"] and np.all(codes == g["code"])
    d_bits, s_bits, codes = _q8_block_fields(xq[0], 1)
    assert d_bits == 0 and s_bits == 0 and np.all(codes == 0)


def pin_exp_vs_f64(O):
    """e(a) within one ulp of exp over the whole normal range; exact at 0;
    +inf above the range, +0 below, NaN through."""
    a = np.concatenate([np.linspace(-87.0, 88.5, 400001), np.linspace(-1.0, 1.0, 20001)]).astype(np.float32)
    got = O.exp_f32(a).astype(np.float64)
    ref = np.exp(a.astype(np.float64))
    ulp = np.spacing(ref.astype(np.float32)).astype(np.float64)
    assert np.max(np.abs(got - ref) / ulp) <= 1.0
    assert O.exp_f32([0.0])[0] == 1.0
    sp = O.exp_f32([150.0, 100.5, -200.0, -110.5, np.nan])
    assert sp[0] == np.inf and sp[1] == np.inf and sp[2] == 0.0 and sp[3] == 0.0 and np.isnan(sp[4])


def pin_silu_vs_f64(O):
    """silu(t) = t / (1 + exp(-t)) within a few ulp; silu(0) = 0; silu(t) = t
    once exp(-t) is below half an ulp of 1; odd-part identity."""
    t = np.linspace(-80.0, 80.0, 160001).astype(np.float32)
    got = O.silu_f32(t).astype(np.float64)
    td = t.astype(np.float64)
    ref = td / (1.0 + np.exp(-td))
    nz = np.abs(ref) > 1e-30
    assert np.max(np.abs(got - ref)[nz] / np.abs(ref[nz])) < 4.0 * 2.0 ** -24
    assert O.silu_f32([0.0])[0] == 0.0
    big = np.array([17.0, 20.0, 33.5, 1e6], dtype=np.float32)
    assert np.array_equal(O.silu_f32(big), big)
    u = np.linspace(0.01, 30.0, 3001).astype(np.float32)
    diff = O.silu_f32(u).astype(np.float64) - O.silu_f32(-u).astype(np.float64)
    assert np.max(np.abs(diff - u) / u) < 4.0 * 2.0 ** -24


def _rmsnorm_f64(x, g, eps, res=None):
    h = x.astype(np.float64) + (0.0 if res is None else res.astype(np.float64))
    r = 1.0 / np.sqrt(np.mean(h * h, axis=1, keepdims=True) + eps)
    return h * r * g.astype(np.float64)


def pin_rmsnorm_vs_f64(O):
    """RMSNorm against its f64 definition (also with eps dominating and with a
    residual), within the rounding of an n-term sum of squares and four f32
    operations."""
    for n, scale, eps in [(256, 1.0, 1e-5), (256, 1e-3, 1e-5), (4096, 1.0, 1e-6), (512, 30.0, 0.0)]:
        x = activations(81, n, 3, n) * np.float32(scale)
        res = activations(82, n, 3, n) * np.float32(scale)
        g = (1.0 + 0.1 * activations(83, n, 1, n)[0]).astype(np.float32)
        for r in (None, res):
            y, _ = O.rmsnorm_q8_1(x, g, eps, residual=r)
            ref = _rmsnorm_f64(x, g, eps, r)
            bound = (n / 2 + 6) * 2.0 ** -24 * np.abs(ref) + 1e-37
            assert np.all(np.abs(y - ref) <= bound), (n, scale, eps)


def pin_rmsnorm_structure(O):
    """The residual form equals RMSNorm of the f32 sum; eps = 0 RMSNorm is
    invariant under power-of-two scaling; the q8_1 output is the quantiser
    applied to y."""
    n = 1024
    x = activations(84, 0, 2, n)
    res = activations(84, 1, 2, n)
    g = (1.0 + 0.1 * activations(84, 2, 1, n)[0]).astype(np.float32)
    y1, q1 = O.rmsnorm_q8_1(x, g, 1e-6, residual=res)
    y2, q2 = O.rmsnorm_q8_1((x + res).astype(np.float32), g, 1e-6)
    assert np.array_equal(y1, y2) and np.array_equal(q1, q2)
    y3, _ = O.rmsnorm_q8_1(x, g, 0.0)
    y4, _ = O.rmsnorm_q8_1(x * np.float32(2.0 ** -7), g, 0.0)
    assert np.array_equal(y3, y4)
    assert np.array_equal(q1, O.quantize_q8_1(y1))


def pin_swiglu_structure(O):
    """SwiGLU is silu(gate) * up elementwise, its q8_1 the quantiser of y, and
    it agrees with the f64 definition."""
    gate = activations(85, 0, 2, 512) * np.float32(4.0)
    up = activations(85, 1, 2, 512)
    y, xq = O.swiglu_q8_1(gate, up)
    assert np.array_equal(y, (O.silu_f32(gate).reshape(gate.shape) * up).astype(np.float32))
    assert np.array_equal(xq, O.quantize_q8_1(y))
    gd = gate.astype(np.float64)
    ref = gd / (1.0 + np.exp(-gd)) * up.astype(np.float64)
    assert np.all(np.abs(y - ref) <= 6.0 * 2.0 ** -24 * np.abs(ref) + 1e-37)


def pin_e11_q8_tiny_block(O):
    g = load_golden("e11_q8_1_tiny_block.txt")
    x = np.zeros((1, 32), dtype=np.float32)
    x[0, 0], x[0, 1] = g["x0"], g["x1"]
    assert x[0, 0] == -(2.0 ** -122) and x[0, 1] == 2.0 ** -130
    d_bits, s_bits, codes = _q8_block_fields(O.quantize_q8_1(x)[0], 0)
    assert d_bits == g["d_bits"] and s_bits == g["s_bits"]
    assert list(codes[:2]) == g["codes"] and np.all(codes[2:] == 0)


PINS += [
    pin_e11_q8_tiny_block,
    pin_e8_rms_reduction_order,
    pin_e9_rmsnorm_constant_row,
    pin_e10_swiglu_saturated,
    pin_exp_vs_f64,
    pin_silu_vs_f64,
    pin_rmsnorm_vs_f64,
    pin_rmsnorm_structure,
    pin_swiglu_structure,
]
