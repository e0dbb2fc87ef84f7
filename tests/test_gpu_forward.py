"""The fused path (indexer -> top-k -> sparse MLA) against the oracle, plus the
invariants that need no oracle: paged == contiguous bit for bit, run-to-run
determinism, k >= n reducing to dense causal attention, empty contexts."""
import math

import numpy as np
import pytest
import torch

import oracle
from tests.helpers import (OUT_TOL, check_attention, check_topk_row_e2e, score_magnitude, small_workload,
                           to_oracle)
from tests.test_gpu_ops import B, DEV, _say, big_dims
from workloads import generate

pytestmark = pytest.mark.gpu


def run_forward(inp):
    out, lse, idx = B().forward_inputs(inp)
    torch.cuda.synchronize()
    return out, lse, idx


def check_all_rows(inp, out, lse, idx, name):
    oi = to_oracle(inp)
    og, lg, ig = out.float().cpu().numpy(), lse.cpu().numpy(), idx.cpu().numpy()
    swaps = 0
    for t in range(inp.num_q):
        scores = oracle.query_index_scores(oi, t)
        scale = score_magnitude(oi, t) if inp.wl.w_low < 0 else None
        swaps += check_topk_row_e2e(ig[t], scores, inp.topk, f"{name} row {t}", scale=scale)
        m = min(inp.topk, scores.shape[0])
        o_ref, l_ref = oracle.query_attention(oi, t, ig[t, :m])
        check_attention(og[t], lg[t], o_ref, l_ref, OUT_TOL[inp.wl.mla_dtype], f"{name} row {t}")
    return swaps


FORWARD_CASES = [
    ("decode_contig", dict(mode="decode", num_seqs=4, length=6000, k=2048), [6000, 2048, 2049, 1]),
    ("decode_paged", dict(mode="decode", num_seqs=3, length=9000, k=2048, paged=True), [9000, 4097, 2000]),
    ("decode_paged_fp8", dict(mode="decode", num_seqs=3, length=5000, k=2048, paged=True, index_dtype="fp8"),
     [5000, 2100, 64]),
    ("prefill", dict(mode="prefill", length=2600, k=2048, prefill_q_start=2000), None),
    ("prefill_fp8", dict(mode="prefill", length=2300, k=2048, prefill_q_start=2030, index_dtype="fp8"), None),
    ("prefill_short_k", dict(mode="prefill", length=700, k=100), None),
    # mixed-sign head weights: rows of negative and positive scores through the fused top-k
    ("decode_paged_mixed_w", dict(mode="decode", num_seqs=3, length=7000, k=2048, paged=True, w_low=-1 / 8),
     [7000, 2050, 4096]),
    ("decode_paged_fp8_mixed_w", dict(mode="decode", num_seqs=3, length=6000, k=2048, paged=True,
                                      index_dtype="fp8", w_low=-1 / 8), [6000, 3000, 2100]),
    ("prefill_mixed_w", dict(mode="prefill", length=2500, k=2048, prefill_q_start=2040, w_low=-1 / 8), None),
    ("prefill_fp8_mixed_w", dict(mode="prefill", length=2400, k=2048, prefill_q_start=2100, index_dtype="fp8",
                                 w_low=-1 / 8), None),
]


@pytest.mark.parametrize("name,kw,lengths", FORWARD_CASES, ids=[c[0] for c in FORWARD_CASES])
def test_forward_parity(name, kw, lengths):
    _say("forward", name)
    inp = generate(big_dims(**kw), DEV, lengths=lengths)
    out, lse, idx = run_forward(inp)
    check_all_rows(inp, out, lse, idx, name)


def test_forward_f32_tiny_config():
    """The tiny fp32 prefill workload, every row."""
    from workloads import WORKLOADS
    _say("forward tiny_prefill_f32")
    inp = generate(WORKLOADS["tiny_prefill_f32"], DEV)
    out, lse, idx = run_forward(inp)
    check_all_rows(inp, out, lse, idx, "tiny_prefill_f32")


def test_forward_matches_staged_ops():
    """dsa_forward equals index_scores -> topk -> sparse_mla on the same inputs, bit for bit."""
    _say("forward vs staged")
    inp = generate(big_dims(mode="decode", num_seqs=3, length=5000, k=2048, paged=True), DEV,
                   lengths=[5000, 3000, 4100])
    out, lse, idx = run_forward(inp)
    pb = B().problem_from_inputs(inp)
    sc = B().index_scores(pb, inp.q_idx, inp.q_scale, inp.w, inp.k_cache, inp.k_scale)
    idx2 = B().topk(pb, sc)
    out2, lse2 = B().sparse_mla(pb, inp.sm_scale, inp.q, inp.kv_cache, idx2)
    torch.cuda.synchronize()
    assert torch.equal(idx, idx2)
    assert torch.equal(out, out2) and torch.equal(lse, lse2)


BATCH_CASES = [
    ("decode_paged_bf16_33", dict(mode="decode", num_seqs=33, length=9000, k=2048, paged=True),
     [9000 - 271 * i for i in range(31)] + [2048, 1]),
    ("decode_paged_fp8_20", dict(mode="decode", num_seqs=20, length=7000, k=2048, paged=True, index_dtype="fp8"),
     [7000 - 301 * i for i in range(19)] + [2049]),
    ("decode_contig_bf16_16", dict(mode="decode", num_seqs=16, length=4500, k=2048),
     [4500 - 150 * i for i in range(16)]),
]


@pytest.mark.parametrize("name,kw,lengths", BATCH_CASES, ids=[c[0] for c in BATCH_CASES])
def test_forward_decode_batches(name, kw, lengths):
    """Decode batches of 16 to 33 queries with ragged contexts (one of a single
    token, one of exactly k): every row against the oracle, and the same bits
    from the stage-timed call (events between the stages) and from a repeat."""
    _say("forward batch", name)
    inp = generate(big_dims(**kw), DEV, lengths=lengths)
    out, lse, idx = run_forward(inp)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    for e in ev:             # torch creates the HIP event on first record
        e.record()
    out2, lse2, idx2 = B().forward_inputs(inp, stage_events=ev)
    out3, lse3, idx3 = run_forward(inp)
    for x, y in ((idx, idx2), (out, out2), (lse, lse2), (idx, idx3), (out, out3), (lse, lse3)):
        assert torch.equal(x, y)
    check_all_rows(inp, out, lse, idx, name)


def _paged_copy(inp, rng):
    """The same logical caches re-laid into permuted 64-token blocks."""
    B_, L = inp.k_cache.shape[:2]
    nb = (L + 63) // 64
    perm = torch.from_numpy(rng.permutation(B_ * nb)).to(DEV)
    table = perm.reshape(B_, nb).to(torch.int32)
    kc = torch.zeros((B_ * nb, 64) + tuple(inp.k_cache.shape[2:]), dtype=inp.k_cache.dtype, device=DEV)
    vc = torch.zeros((B_ * nb, 64) + tuple(inp.kv_cache.shape[2:]), dtype=inp.kv_cache.dtype, device=DEV)
    pos = torch.arange(L, device=DEV)
    for b in range(B_):
        phys = table[b, pos // 64].long() * 64 + pos % 64
        kc.view(-1, *kc.shape[2:])[phys] = inp.k_cache[b]
        vc.view(-1, *vc.shape[2:])[phys] = inp.kv_cache[b]
    import dataclasses
    return dataclasses.replace(inp, block_table=table.contiguous(), num_blocks=B_ * nb, max_seq_len=0,
                               k_cache=kc, kv_cache=vc)


def test_paged_equals_contiguous_bitwise():
    _say("paged == contiguous")
    inp = generate(big_dims(mode="decode", num_seqs=3, length=4500, k=2048), DEV, lengths=[4500, 4000, 2222])
    a = run_forward(inp)
    pg = _paged_copy(inp, np.random.default_rng(3))
    b = run_forward(pg)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_determinism():
    _say("determinism")
    inp = generate(big_dims(mode="prefill", length=2400, k=2048, prefill_q_start=2200), DEV)
    a = run_forward(inp)
    b = run_forward(inp)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_k_at_least_n_is_dense_causal():
    """With k >= n every candidate is selected and the output is dense causal attention
    (computed here in float64 by torch's SDPA on the CPU)."""
    _say("k >= n dense")
    inp = generate(big_dims(mode="prefill", length=150, k=256), DEV)
    out, lse, idx = run_forward(inp)
    ig = idx.cpu().numpy()
    for t in range(150):
        assert list(ig[t, : t + 1]) == list(range(t + 1)) and np.all(ig[t, t + 1:] == -1)
    q = oracle.decode_bf16(inp.q.view(torch.int16).cpu().numpy().view(np.uint16))
    kv = oracle.decode_bf16(inp.kv_cache[0].view(torch.int16).cpu().numpy().view(np.uint16))
    qt = torch.from_numpy(q).permute(1, 0, 2).unsqueeze(0)                   # [1, H, T, D]
    kt = torch.from_numpy(kv).expand(128, 150, 576).unsqueeze(0)
    vt = torch.from_numpy(np.ascontiguousarray(kv[:, :512])).expand(128, 150, 512).unsqueeze(0)
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True, scale=inp.sm_scale)
    ref = ref[0].permute(1, 0, 2).numpy()
    err = np.abs(out.float().cpu().numpy() - ref).max()
    assert err <= 2e-2, err


def test_empty_and_single_candidate():
    """q_pos = -1 (no candidates): idx all -1, out 0, lse -inf; q_pos = 0: the query's own row."""
    _say("empty / single")
    inp = generate(big_dims(mode="decode", num_seqs=3, length=300, k=2048), DEV, lengths=[300, 1, 300])
    inp.q_pos[2] = -1
    out, lse, idx = run_forward(inp)
    assert torch.all(idx[2] == -1) and torch.all(out[2] == 0) and torch.all(torch.isneginf(lse[2]))
    assert int(idx[1, 0]) == 0 and torch.all(idx[1, 1:] == -1)
    assert torch.equal(out[1], inp.kv_cache[1, 0, :512].expand(128, 512))


# 16 queries with up to 131072 candidates: the fixed decode grid would be 16 x 64
# chunks (two rounds or more of the chip's 512 workgroup slots), so the fused
# forward's indexer takes the length-balanced grid (a row's workgroups in
# proportion to its candidates, 64-aligned chunks); the standalone index_scores
# op, which also writes -inf past each row's candidates, keeps the fixed grid.
BALANCED_LENGTHS = [131072, 1, 63, 64, 65, 2047, 2048, 2049, 70001, 100000, 4096, 129, 50000, 131071, 8191, 30000]


@pytest.mark.parametrize("index_dtype", ["bf16", "fp8"])
def test_forward_balanced_decode_grid(index_dtype):
    """Ragged decode batch on the length-balanced indexer grid (a row with no
    candidates, rows of 1, 63-65, 2047-2049 and up to 131072 candidates): the same
    bits as the staged ops on the fixed grid (key tiles start on 32-key boundaries
    in both, so each score is the same arithmetic), and every row against the
    oracle."""
    _say("forward balanced grid", index_dtype)
    kw = dict(mode="decode", num_seqs=len(BALANCED_LENGTHS), length=max(BALANCED_LENGTHS), k=2048, paged=True,
              index_dtype=index_dtype)
    inp = generate(big_dims(**kw), DEV, lengths=BALANCED_LENGTHS)
    inp.q_pos[1] = -1                                 # no candidates
    out, lse, idx = run_forward(inp)
    pb = B().problem_from_inputs(inp)
    sc = B().index_scores(pb, inp.q_idx, inp.q_scale, inp.w, inp.k_cache, inp.k_scale)
    idx2 = B().topk(pb, sc)
    out2, lse2 = B().sparse_mla(pb, inp.sm_scale, inp.q, inp.kv_cache, idx2)
    torch.cuda.synchronize()
    assert torch.equal(idx, idx2)
    assert torch.equal(out, out2) and torch.equal(lse, lse2)
    assert torch.all(idx[1] == -1) and torch.all(torch.isneginf(lse[1]))
    oi = to_oracle(inp)
    ig, og, lg = idx.cpu().numpy(), out.float().cpu().numpy(), lse.cpu().numpy()
    for t in range(inp.num_q):
        if t == 1:
            continue
        scores = oracle.query_index_scores(oi, t)
        check_topk_row_e2e(ig[t], scores, inp.topk, f"balanced {index_dtype} row {t}")
        m = min(inp.topk, scores.shape[0])
        o_ref, l_ref = oracle.query_attention(oi, t, ig[t, :m])
        check_attention(og[t], lg[t], o_ref, l_ref, OUT_TOL[inp.wl.mla_dtype], f"balanced {index_dtype} row {t}")
