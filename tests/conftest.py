import os
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(ROOT, "tests", "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def load_golden(name: str) -> dict:
    """Parse a ``key: values`` fixture under tests/golden (comments start with #)."""
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, _, val = line.partition(":")
            toks = val.split()
            vals = [int(t, 0) if (t.startswith("0x") or t.lstrip("-").isdigit()) else float(t)
                    for t in toks]
            out[key.strip()] = vals if len(vals) != 1 else vals[0]
    return out


def q4k_block_from_fields(d_bits, dmin_bits, scales, qs) -> np.ndarray:
    """Place raw fields at the Q4_K byte offsets (no arithmetic)."""
    b = np.zeros(144, dtype=np.uint8)
    b[0:2] = np.array([d_bits], dtype=np.uint16).view(np.uint8)
    b[2:4] = np.array([dmin_bits], dtype=np.uint16).view(np.uint8)
    b[4:16] = np.asarray(scales, dtype=np.uint8)
    b[16:144] = np.asarray(qs, dtype=np.uint8)
    return b


def q6k_block_from_fields(d_bits, scales, ql, qh) -> np.ndarray:
    """Place raw fields at the Q6_K byte offsets (no arithmetic)."""
    b = np.zeros(210, dtype=np.uint8)
    b[0:128] = np.asarray(ql, dtype=np.uint8)
    b[128:192] = np.asarray(qh, dtype=np.uint8)
    b[192:208] = np.asarray(scales, dtype=np.int8).view(np.uint8)
    b[208:210] = np.array([d_bits], dtype=np.uint16).view(np.uint8)
    return b


@pytest.fixture(scope="session")
def oracle_lib():
    import oracle

    oracle.build(force=False)
    return oracle
