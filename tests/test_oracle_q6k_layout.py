"""Pins of the oracle's split Q6_K layout (a scale prefix of f16 super-scales
and 208-byte bodies, cajeta "One model, start to last token" 2, residency),
checked against tensors built so that every byte says where it came from."""
import numpy as np
import pytest

import oracle
from kq_inputs import q6k_weights


def _labelled(m, s):
    """Raw Q6_K bytes whose body byte b of superblock g is (g*7 + b) % 251 and
    whose d field is the f16 value g + 1."""
    g = np.arange(m * s).reshape(m * s, 1)
    raw = ((g * 7 + np.arange(210)) % 251).astype(np.uint8)
    raw[:, 208:210] = (np.arange(m * s) + 1).astype(np.float16).view(np.uint8).reshape(-1, 2)
    return raw.reshape(m, s * 210)


@pytest.mark.parametrize("m,s", [(1, 1), (3, 5), (7, 16), (2, 56)])
def test_split_places_every_byte(m, s):
    k = 256 * s
    raw = _labelled(m, s)
    wr = oracle.q6k_split(raw, m, k)
    prefix = (2 * m * s + 15) // 16 * 16
    assert wr.size == oracle.q6k_split_bytes(m, k) == prefix + 208 * m * s
    assert prefix % 16 == 0 and prefix - 2 * m * s < 16
    d = wr[: 2 * m * s].view(np.float16)
    assert np.array_equal(d, (np.arange(m * s) + 1).astype(np.float16))   # d of g at 2g
    assert not wr[2 * m * s: prefix].any()                                 # zero padding
    bodies = wr[prefix:].reshape(m * s, 208)
    g = np.arange(m * s).reshape(-1, 1)
    assert np.array_equal(bodies, ((g * 7 + np.arange(208)) % 251).astype(np.uint8))
    # every body starts 16-byte aligned (the point of the layout)
    assert all((prefix + 208 * i) % 16 == 0 for i in range(m * s))


@pytest.mark.parametrize("m,k", [(1, 256), (5, 768), (33, 4096)])
def test_split_round_trip_and_matmul(m, k):
    w = q6k_weights(3, 1, m, k)
    wr = oracle.q6k_split(w, m, k)
    assert np.array_equal(oracle.q6k_unsplit(wr, m, k), w)
    # same dequantised values: the layout is a pure byte permutation
    assert np.array_equal(oracle.dequant("q6k", oracle.q6k_unsplit(wr, m, k), m, k),
                          oracle.dequant("q6k", w, m, k))
