"""kq_read_probe (the benchmark's streaming-read measurement) through the C
ABI: its per-wavefront xor checksums equal a numpy fold of the same bytes,
for whole and ragged sizes, one-shot and persistent grids and every load
count, so every byte is read exactly where the header says."""
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


def reference(data: np.ndarray, grid: int, loads: int) -> np.ndarray:
    """out[4b + w] = xor, over chunks c = b (mod G), u < loads and l < 64, of
    the 32-bit words of 16-byte word 256*loads*c + 256u + 64w + l, zero past
    the end; G = grid (or the chunk count when grid is 0 or larger)."""
    n16 = data.size // 16
    chunks = -(-n16 // (256 * loads))
    g = chunks if grid == 0 else min(grid, chunks)
    words = np.zeros(chunks * 256 * loads * 4, dtype=np.uint32)
    words[: n16 * 4] = data.view(np.uint32)
    w = words.reshape(chunks, loads, 4, 64, 4)          # chunk, u, wave, lane, dword
    per_chunk = np.bitwise_xor.reduce(w.transpose(0, 2, 1, 3, 4).reshape(chunks, 4, -1), axis=2)
    out = np.zeros((g, 4), dtype=np.uint32)
    for c in range(chunks):
        out[c % g] ^= per_chunk[c]
    return out.reshape(-1)


CASES = [(n, 0, 8) for n in (16, 4096, 32768, 32768 + 48, 5 * 32768 + 16 * 1000, 1 << 22)] + [
    (1 << 22, 256, 4), (1 << 22, 7, 16), ((1 << 22) + 16, 512, 32), (5 * 32768 + 16 * 1000, 3, 32),
    (16, 5, 16)]


@pytest.mark.parametrize("nbytes,grid,loads", CASES, ids=[f"{c[0]}-g{c[1]}-u{c[2]}" for c in CASES])
def test_read_probe_checksums(kq, nbytes, grid, loads):
    print(f"\n[case] read probe nbytes={nbytes} grid={grid} loads={loads}", flush=True)
    rng = np.random.default_rng(nbytes + grid)
    data = rng.integers(0, 256, size=nbytes, dtype=np.uint8)
    words = kq.kq_read_probe_words(nbytes, grid, loads)
    out = torch.full((words,), 0xDEAD, dtype=torch.int32, device="cuda")
    src = torch.from_numpy(data).cuda()
    kq.kq_read_probe(src, nbytes, out, grid, loads)
    torch.cuda.synchronize()
    got = out.cpu().numpy().view(np.uint32)
    assert np.array_equal(got, reference(data, grid, loads))
