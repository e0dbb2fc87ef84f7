"""The CPU oracle against its pins (hand-derived examples, closed forms, brute force,
independent library routines, invariants).  CPU only."""
import numpy as np
import pytest

import oracle
from tests import pins
from tests.helpers import small_workload, to_oracle
from workloads import generate, WORKLOADS


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda p: p.__name__)
def test_pin(pin):
    pin(oracle.dsa_oracle)


def test_generator_recipe():
    """Shapes, element types, poison and the e4m3 scale recipe of the generated inputs."""
    wl = small_workload(mode="decode", num_seqs=2, length=70, H_I=4, d_I=16, index_dtype="fp8",
                        mla_dtype="bf16", paged=True, block_size=64)
    inp = generate(wl, "cpu", lengths=[70, 5])
    assert inp.block_table.shape == (2, 2) and inp.num_blocks == 3
    assert int(inp.block_table[1, 1]) == -1
    assert sorted(inp.block_table[inp.block_table >= 0].tolist()) == [0, 1, 2]
    oi = to_oracle(inp)
    # per-token scale: amax of the dequantised key equals 448 * scale (the max code is used)
    for b, n in ((0, 70), (1, 5)):
        for s in range(n):
            blk, off = inp.block_table[b, s // 64], s % 64
            codes = oi.k_cache[blk, off]
            vals = oracle.decode_e4m3fn(codes)
            assert np.all(np.isfinite(vals)) and np.max(np.abs(vals)) == 448.0
    # tails of the last blocks are poisoned
    blk = int(inp.block_table[1, 0])
    assert np.all(oi.k_cache[blk, 5:] == 0x7F)
    assert np.all(np.isnan(oracle.decode_bf16(oi.kv_cache[blk, 5:])))
    assert inp.q_pos.tolist() == [69, 4]


def test_planted_keys():
    wl = WORKLOADS["prefill_16k_bf16"].replace(length=400, index_heads=2, heads=2)
    inp = generate(wl, "cpu")
    assert inp.planted.shape[0] == 20
    assert len(set(inp.planted.tolist())) == 20


def test_forward_rows_subset():
    wl = small_workload(mode="prefill", length=20, k=4)
    oi = to_oracle(generate(wl, "cpu"))
    full = oracle.forward(oi)
    part = oracle.forward(oi, rows=[3, 19])
    assert np.array_equal(full["out"][[3, 19]], part["out"])
