"""The read-rate measurement entry point (dsa_read_ceiling) reads what it says:
every wave's XOR word equals the XOR of the 8 KB tiles that the indexer's tiling
assigns to it, through the scattered-block mapping when paged, with streaming
and with default-policy loads."""
import numpy as np
import pytest
import torch

from sparse_long_context_relu_amd import binding as B

pytestmark = pytest.mark.gpu

CHUNK, TILE, BLOCK = 512 * 1024, 8192, 16384


def expected_words(words: np.ndarray, nbytes: int, paged: bool) -> np.ndarray:
    tiles = words.reshape(-1, TILE // 4)
    tile_xor = np.bitwise_xor.reduce(tiles, axis=1)
    nblk = nbytes // BLOCK
    out, seen = [], []
    for c in range(nbytes // CHUNK):
        for w in range(4):
            acc = np.uint32(0)
            for t in range(CHUNK // TILE // 4):
                g = c * (CHUNK // TILE) + 4 * t + w
                phys = ((((g >> 1) * 0x9E3779B1) & (nblk - 1)) << 1) | (g & 1) if paged else g
                seen.append(phys)
                acc ^= tile_xor[phys]
            out.append(acc)
    assert sorted(seen) == list(range(nbytes // TILE))      # every tile read exactly once
    return np.array(out, dtype=np.uint32)


@pytest.mark.parametrize("cached", [False, True])
@pytest.mark.parametrize("paged", [False, True])
def test_read_ceiling_reads_every_word(paged, cached):
    nbytes = 4 << 20
    gen = torch.Generator().manual_seed(11)
    host = torch.randint(-(2 ** 31), 2 ** 31 - 1, (nbytes // 4,), dtype=torch.int32, generator=gen)
    sink = B.read_ceiling(host.cuda(), paged, cached=cached)
    torch.cuda.synchronize()
    got = sink.cpu().numpy().view(np.uint32)
    assert np.array_equal(got, expected_words(host.numpy().view(np.uint32), nbytes, paged))
