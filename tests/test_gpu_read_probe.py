"""kq_read_probe (the benchmark's streaming-read measurement) through the C
ABI: its per-wavefront xor checksums equal a numpy fold of the same bytes,
for whole and ragged sizes, so every byte is read exactly where the header
says."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def kq():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    import q6_q8_matmul_amd as kq

    kq.lib()
    return kq


def reference(data: np.ndarray) -> np.ndarray:
    """out[4c + w] = xor of the 32-bit words of 16-byte words
    2048c + 256u + 64w + l (u < 8, l < 64), zero past the end."""
    n16 = data.size // 16
    chunks = -(-n16 // 2048)
    words = np.zeros(chunks * 2048 * 4, dtype=np.uint32)
    words[: n16 * 4] = data.view(np.uint32)
    w = words.reshape(chunks, 8, 4, 64, 4)          # chunk, u, wave, lane, dword
    return np.bitwise_xor.reduce(w.transpose(0, 2, 1, 3, 4).reshape(chunks, 4, -1), axis=2).reshape(-1)


@pytest.mark.parametrize("nbytes", [16, 4096, 32768, 32768 + 48, 5 * 32768 + 16 * 1000, 1 << 22])
def test_read_probe_checksums(kq, nbytes):
    print(f"\n[case] read probe nbytes={nbytes}", flush=True)
    rng = np.random.default_rng(nbytes)
    data = rng.integers(0, 256, size=nbytes, dtype=np.uint8)
    words = kq.kq_read_probe_words(nbytes)
    out = torch.full((words,), 0xDEAD, dtype=torch.int32, device="cuda")
    src = torch.from_numpy(data).cuda()
    kq.kq_read_probe(src, nbytes, out)
    torch.cuda.synchronize()
    got = out.cpu().numpy().view(np.uint32)
    assert np.array_equal(got, reference(data))
