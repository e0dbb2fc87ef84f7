"""Dense MLA (attention over every causal candidate, the comparison DSA is
measured against) and the short-prompt mode of the forward, through the C ABI.

Parity: the HIP path against oracle.dense_forward, element by element, on
contexts that span several splits (up to the 128-split maximum) with ragged
tails, paged and contiguous, plus sampled rows at the benchmark's full sizes.
The short-prompt forward (no query with more than k candidates) must give the
same bytes as the staged indexer -> top-k -> sparse MLA calls."""
import math
import zlib

import numpy as np
import pytest
import torch

import oracle
from tests.helpers import OUT_TOL, check_attention, small_workload, to_oracle, to_oracle_rows
from tests.test_gpu_ops import B, DEV, _say, big_dims
from tests.test_gpu_configs import sample_rows
from workloads import WORKLOADS, generate

pytestmark = pytest.mark.gpu


def _f32(**kw):
    base = dict(H_I=4, d_I=32, H=8, D=80, Dv=64, index_dtype="f32", mla_dtype="f32",
                qkv_std=1 / math.sqrt(80), w_high=1.0)
    base.update(kw)
    return small_workload(**base)


DENSE_CASES = [
    # 79 splits of 64 rows (more than one wave of split statistics in the merge)
    ("decode_contig_many_splits", big_dims(mode="decode", num_seqs=3, length=5000, k=64), [5000, 1, 2049], 1.0),
    ("decode_paged_ragged", big_dims(mode="decode", num_seqs=4, length=3000, k=64, paged=True),
     [3000, 64, 65, 2500], 1.0),
    ("decode_paged_sharp", big_dims(mode="decode", num_seqs=2, length=4100, k=64, paged=True), [4100, 2222],
     1200.0),
    # 128 splits of 1120 rows at 140000 candidates
    ("decode_long_128_splits", big_dims(mode="decode", num_seqs=2, length=140000, k=64), [140000, 70001], 1.0),
    ("prefill_one_split", big_dims(mode="prefill", length=300, k=64), None, 1.0),
    ("prefill_two_splits", big_dims(mode="prefill", length=2600, k=64, prefill_q_start=2400), None, 1.0),
    ("prefill_f32", _f32(mode="prefill", length=200, k=16), None, 1.0),
    ("decode_f32_paged", _f32(mode="decode", num_seqs=3, length=700, k=16, paged=True), [700, 1, 129], 1.0),
]


def _dense(inp):
    pb = B().problem_from_inputs(inp)
    out, lse = B().dense_mla(pb, inp.sm_scale, inp.q, inp.kv_cache)
    torch.cuda.synchronize()
    return out, lse


@pytest.mark.parametrize("name,wl,lengths,qmul", DENSE_CASES, ids=[c[0] for c in DENSE_CASES])
def test_dense_mla(name, wl, lengths, qmul):
    _say("dense_mla", name)
    inp = generate(wl, DEV, lengths=lengths)
    if qmul != 1.0:           # "sharp" logits: the running maxima move between splits
        inp.q = (inp.q.float() * qmul).to(inp.q.dtype)
    out, lse = _dense(inp)
    og, lg = out.float().cpu().numpy(), lse.cpu().numpy()
    oi = to_oracle(inp)
    for t in range(inp.num_q):
        o_ref, l_ref = oracle.dense_attention(oi, t)
        check_attention(og[t], lg[t], o_ref, l_ref, OUT_TOL[wl.mla_dtype], f"{name} row {t}")


def test_dense_mla_chunked_prefill():
    """4096 queries x 2 splits exceed one chunk of partials: rows on both sides of the
    chunk boundary (4064) and the last row against the oracle."""
    _say("dense_mla chunked prefill")
    inp = generate(big_dims(mode="prefill", length=4096, k=64), DEV)
    out, lse = _dense(inp)
    rows = [0, 1, 2047, 2048, 4063, 4064, 4065, 4095]
    oi, local = to_oracle_rows(inp, rows)
    og, lg = out.float().cpu().numpy(), lse.cpu().numpy()
    for i, t in enumerate(rows):
        o_ref, l_ref = oracle.dense_attention(oi, local[i])
        check_attention(og[t], lg[t], o_ref, l_ref, OUT_TOL["bf16"], f"chunked row {t}")


def test_dense_mla_empty_and_single():
    """q_pos = -1: out 0 and lse -inf; q_pos = 0: the query's own latent row."""
    _say("dense_mla empty / single")
    inp = generate(big_dims(mode="decode", num_seqs=3, length=3000, k=64), DEV, lengths=[3000, 1, 3000])
    inp.q_pos[2] = -1
    out, lse = _dense(inp)
    assert torch.all(out[2] == 0) and torch.all(torch.isneginf(lse[2]))
    assert torch.equal(out[1], inp.kv_cache[1, 0, :512].expand(128, 512))
    oi = to_oracle(inp)
    o_ref, l_ref = oracle.dense_attention(oi, 0)
    check_attention(out[0].float().cpu().numpy(), lse[0].cpu().numpy(), o_ref, l_ref, 2e-2, "full row")


DENSE_FULL = [("decode_128k_paged_bf16", 4), ("decode_128k_exact_paged_bf16", 2), ("prefill_16k_bf16", 6)]


@pytest.mark.parametrize("name,extra", DENSE_FULL, ids=[c[0] for c in DENSE_FULL])
def test_dense_mla_full_size(name, extra):
    """The benchmark's dense comparison at full size: sampled rows against the oracle."""
    _say("dense_mla full-size", name)
    inp = generate(WORKLOADS[name], DEV)
    out, lse = _dense(inp)
    assert torch.isfinite(out.float()).all() and not torch.isnan(lse).any()
    rows = sample_rows(inp, extra, seed=zlib.crc32(("dense" + name).encode()))
    oi, local = to_oracle_rows(inp, rows)
    og, lg = out.float().cpu().numpy(), lse.cpu().numpy()
    for i, t in enumerate(rows):
        o_ref, l_ref = oracle.dense_attention(oi, local[i])
        check_attention(og[t], lg[t], o_ref, l_ref, OUT_TOL["bf16"], f"{name} row {t}")


SHORT_CASES = [
    ("decode_paged_k_equals_max_ctx", big_dims(mode="decode", num_seqs=4, length=2048, k=2048, paged=True),
     [2048, 1, 700, 1500]),
    ("prefill_short", big_dims(mode="prefill", length=1000, k=2048), None),
    ("prefill_f32_short", _f32(mode="prefill", length=24, k=32), None),
]


@pytest.mark.parametrize("name,wl,lengths", SHORT_CASES, ids=[c[0] for c in SHORT_CASES])
def test_forward_short_prompt_equals_staged(name, wl, lengths):
    """max_ctx <= k: dsa_forward skips the indexer and the top-k; its bytes equal the
    staged calls' (which do run them), and the selection is every candidate."""
    _say("short-prompt forward", name)
    inp = generate(wl, DEV, lengths=lengths)
    out, lse, idx = B().forward_inputs(inp)
    pb = B().problem_from_inputs(inp)
    sc = B().index_scores(pb, inp.q_idx, inp.q_scale, inp.w, inp.k_cache, inp.k_scale)
    idx2 = B().topk(pb, sc)
    out2, lse2 = B().sparse_mla(pb, inp.sm_scale, inp.q, inp.kv_cache, idx2)
    torch.cuda.synchronize()
    assert torch.equal(idx, idx2)
    assert torch.equal(out, out2) and torch.equal(lse, lse2)
    oi = to_oracle(inp)
    og, lg = out.float().cpu().numpy(), lse.cpu().numpy()
    for t in (0, inp.num_q // 2, inp.num_q - 1):
        o_ref, l_ref = oracle.dense_attention(oi, t)
        check_attention(og[t], lg[t], o_ref, l_ref, OUT_TOL[wl.mla_dtype], f"{name} row {t}")
