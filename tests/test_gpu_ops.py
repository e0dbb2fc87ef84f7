"""Per-step parity of the HIP path against the CPU oracle, through the C ABI.

Sizes span several tiles with ragged tails; every case prints its name first
so a failing run names it."""
import math
import zlib

import numpy as np
import pytest
import torch

import oracle
from tests.helpers import (OUT_TOL, SCORE_TOL, check_attention, check_scores, check_topk_row_e2e,
                           check_topk_row_exact, score_magnitude, small_workload, to_oracle, to_oracle_rows)
from workloads import Workload, generate

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _say(*a):
    print("[case]", *a, flush=True)


def B():
    from sparse_long_context_relu_amd import binding
    return binding


def big_dims(**kw):
    """Indexer H_I=64, d_I=128; MLA H=128, D=576, Dv=512 (the supported bf16/fp8 shapes)."""
    base = dict(H_I=64, d_I=128, H=128, D=576, Dv=512, index_dtype="bf16", mla_dtype="bf16",
                w_high=1.0 / 8.0, qkv_std=1.0 / 24.0)
    base.update(kw)
    return small_workload(**base).replace(sm_scale=1.0 / math.sqrt(576.0))


INDEXER_CASES = [
    ("decode_contig_bf16", dict(mode="decode", num_seqs=5, length=5000, k=64), [1, 63, 2049, 4096, 5000]),
    ("decode_paged_bf16", dict(mode="decode", num_seqs=4, length=3000, k=64, paged=True), [1, 64, 65, 3000]),
    ("prefill_bf16", dict(mode="prefill", length=333, k=64), None),
    ("prefill_fp8", dict(mode="prefill", length=301, k=64, index_dtype="fp8"), None),
    ("decode_paged_fp8", dict(mode="decode", num_seqs=3, length=2500, k=64, paged=True, index_dtype="fp8"),
     [2500, 7, 1300]),
    # mixed-sign head weights: scores of either sign, negative ReLU-weighted heads
    ("decode_paged_bf16_mixed_w", dict(mode="decode", num_seqs=3, length=4100, k=64, paged=True, w_low=-1 / 8),
     [4100, 300, 2049]),
    ("prefill_bf16_mixed_w", dict(mode="prefill", length=290, k=64, w_low=-1 / 8), None),
    ("decode_paged_fp8_mixed_w", dict(mode="decode", num_seqs=3, length=2600, k=64, paged=True, index_dtype="fp8",
                                      w_low=-1 / 8), [2600, 33, 1999]),
    ("prefill_fp8_mixed_w", dict(mode="prefill", length=310, k=64, index_dtype="fp8", w_low=-1 / 8), None),
    # decode grids with fewer than 1024 workgroups of 2048 keys take smaller ones:
    # 32 rows of up to 16K keys -> 512-key workgroups, 16 rows of 64K -> 1024
    ("decode_paged_bf16_chunk512", dict(mode="decode", num_seqs=32, length=16384, k=64, paged=True),
     [16384 - 509 * i for i in range(32)]),
    ("decode_paged_fp8_chunk1024", dict(mode="decode", num_seqs=16, length=65536, k=64, paged=True,
                                        index_dtype="fp8"), [65536 - 3001 * i for i in range(16)]),
    ("prefill_f32", dict(mode="prefill", length=200, k=16, H_I=4, d_I=32, H=8, D=80, Dv=64,
                         index_dtype="f32", mla_dtype="f32", qkv_std=1 / math.sqrt(80), w_high=1.0), None),
    ("decode_f32_paged", dict(mode="decode", num_seqs=3, length=700, k=16, H_I=4, d_I=32, H=8, D=80, Dv=64,
                              index_dtype="f32", mla_dtype="f32", paged=True, w_high=1.0), [700, 1, 129]),
]


@pytest.mark.parametrize("name,kw,lengths", INDEXER_CASES, ids=[c[0] for c in INDEXER_CASES])
def test_index_scores(name, kw, lengths):
    _say("index_scores", name)
    wl = big_dims(**kw) if kw.get("index_dtype") != "f32" else small_workload(**kw)
    inp = generate(wl, DEV, lengths=lengths)
    pb = B().problem_from_inputs(inp)
    ld = inp.max_ctx + 5
    scores = B().index_scores(pb, inp.q_idx, inp.q_scale, inp.w, inp.k_cache, inp.k_scale, ld=ld)
    torch.cuda.synchronize()
    sc = scores.cpu().numpy()
    oi = to_oracle(inp)
    tol = SCORE_TOL[wl.index_dtype]
    for t in range(inp.num_q):
        n = int(inp.q_pos[t]) + 1
        ref = oracle.query_index_scores(oi, t)
        mixed = wl.w_low < 0          # mixed-sign weights: tolerance against the terms' magnitude
        check_scores(sc[t, :n], ref, tol, f"{name} row {t}", scale=score_magnitude(oi, t) if mixed else None)
        assert np.all(np.isneginf(sc[t, n:])), f"{name} row {t}: masked tail not -inf"


def _topk_rows(rows, n_max, kind, rng):
    """Score rows with the structures that stress the exact select."""
    x = rng.standard_normal((rows, n_max)).astype(np.float32)
    if kind == "ties":
        x = np.round(x * 4) / 4
    elif kind == "all_equal":
        x[:] = 1.5
    elif kind == "signed_zero":
        x = np.where(rng.random((rows, n_max)) < 0.5, np.float32(0.0), np.float32(-0.0)).astype(np.float32)
        x[:, ::97] = 1.0
    elif kind == "negative":
        x = -np.abs(x) - 1.0
    elif kind == "plateau":
        x = np.round(x, 1)
        x[:, 5000:9000] = 3.25                       # > 4096 equal scores at the threshold
    elif kind == "narrow":
        x = (18.0 + 1e-3 * x).astype(np.float32)     # one exponent, few mantissa bits differ
    return x


TOPK_CASES = [
    ("random_decode", 4, 10000, 2048, "normal", "decode"),
    ("ties", 3, 7000, 2048, "ties", "decode"),
    ("all_equal_overflow", 2, 9000, 2048, "all_equal", "decode"),
    ("signed_zero", 2, 6000, 300, "signed_zero", "decode"),
    ("negative", 3, 5000, 2048, "negative", "decode"),
    ("plateau_overflow", 2, 12000, 2048, "plateau", "decode"),
    ("narrow", 2, 20000, 2048, "narrow", "decode"),
    ("small_k", 5, 3000, 1, "normal", "decode"),
    ("k7", 5, 3000, 7, "ties", "decode"),
    ("prefill_rows", 300, 4200, 2048, "normal", "prefill"),
    # one workgroup per row (256 rows or more): candidate lists past the LDS
    # capacity (long rows), and rows whose threshold digit holds every key
    ("prefill_rows_overflow", 260, 40000, 2048, "normal", "prefill"),
    ("prefill_rows_all_equal", 256, 9000, 2048, "all_equal", "prefill"),
    ("prefill_rows_plateau", 256, 12000, 2048, "plateau", "prefill"),
    ("prefill_rows_narrow", 256, 20000, 2048, "narrow", "prefill"),
    ("prefill_rows_ties", 256, 7000, 2048, "ties", "prefill"),
    ("prefill_rows_signed_zero", 256, 5000, 300, "signed_zero", "prefill"),
    ("long_row", 2, 131072, 2048, "normal", "decode"),
]


@pytest.mark.parametrize("name,rows,n_max,k,kind,mode", TOPK_CASES, ids=[c[0] for c in TOPK_CASES])
def test_topk_isolated_bit_exact(name, rows, n_max, k, kind, mode):
    _say("topk", name)
    rng = np.random.default_rng(zlib.crc32(name.encode()))      # the same rows in every process
    x = _topk_rows(rows, n_max, kind, rng)
    if mode == "decode":
        pos = rng.integers(0, n_max, size=rows)
        pos[0] = n_max - 1
        if rows > 2:
            pos[1] = min(k - 1, n_max - 1)           # n == k exactly
            pos[2] = min(k, n_max - 1)               # n == k + 1
        bt = None
        num_seqs = rows
    else:
        pos = np.sort(rng.integers(0, n_max, size=rows))
        pos[-1] = n_max - 1
        num_seqs = 1
    q_pos = torch.tensor(pos, dtype=torch.int32, device=DEV)
    pb = B().make_problem(mode=mode, q_pos=q_pos, max_ctx=n_max, num_seqs=num_seqs, max_seq_len=n_max, topk=k)
    scores = torch.from_numpy(x).to(DEV)
    idx = B().topk(pb, scores, k)
    torch.cuda.synchronize()
    got = idx.cpu().numpy()
    for r in range(rows):
        n = int(pos[r]) + 1
        check_topk_row_exact(got[r], x[r, :n], k, f"{name} row {r} n={n}")


MLA_CASES = [
    ("bf16_decode_splits", dict(mode="decode", num_seqs=3, length=3000, k=2048), [3000, 1500, 40], 1.0),
    ("bf16_decode_sharp", dict(mode="decode", num_seqs=2, length=2600, k=2048, paged=True), [2600, 2100], 1200.0),
    ("bf16_prefill", dict(mode="prefill", length=300, k=64), None, 1.0),
    ("bf16_prefill_sharp", dict(mode="prefill", length=200, k=48), None, 1000.0),
    ("f32_prefill", dict(mode="prefill", length=120, k=32, H_I=4, d_I=32, H=8, D=80, Dv=64, index_dtype="f32",
                         mla_dtype="f32", qkv_std=1 / math.sqrt(80), w_high=1.0), None, 1.0),
]


@pytest.mark.parametrize("name,kw,lengths,qmul", MLA_CASES, ids=[c[0] for c in MLA_CASES])
def test_sparse_mla(name, kw, lengths, qmul):
    """Attention over a given index set (random valid positions, some -1 holes)."""
    _say("sparse_mla", name)
    wl = big_dims(**kw) if kw.get("mla_dtype") != "f32" else small_workload(**kw)
    inp = generate(wl, DEV, lengths=lengths)
    if qmul != 1.0:           # "sharp" logits: std of q.c*scale around 2
        inp.q = (inp.q.float() * qmul).to(inp.q.dtype)
    rng = np.random.default_rng(5)
    T, k = inp.num_q, wl.topk
    idx = np.full((T, k), -1, dtype=np.int32)
    for t in range(T):
        n = int(inp.q_pos[t]) + 1
        m = int(rng.integers(1, min(k, n) + 1)) if t % 3 else min(k, n)
        sel = np.sort(rng.choice(n, size=m, replace=False))
        idx[t, :m] = sel
        if m > 4 and t % 2:
            idx[t, 1] = -1                          # a hole inside the list
    idx_t = torch.from_numpy(idx).to(DEV)
    pb = B().problem_from_inputs(inp)
    out, lse = B().sparse_mla(pb, inp.sm_scale, inp.q, inp.kv_cache, idx_t)
    torch.cuda.synchronize()
    og, lg = out.float().cpu().numpy(), lse.cpu().numpy()
    oi = to_oracle(inp)
    for t in range(T):
        o_ref, l_ref = oracle.query_attention(oi, t, idx[t])
        check_attention(og[t], lg[t], o_ref, l_ref, OUT_TOL[wl.mla_dtype], f"{name} row {t}")


def test_sparse_mla_empty_and_invalid_entries():
    """A query with no valid entries gives out = 0 and lse = -inf; out-of-range entries are skipped."""
    _say("sparse_mla empty")
    wl = big_dims(mode="decode", num_seqs=2, length=500, k=64)
    inp = generate(wl, DEV, lengths=[500, 300])
    idx = torch.full((2, 64), -1, dtype=torch.int32, device=DEV)
    idx[1, :3] = torch.tensor([5, 400, 299], dtype=torch.int32)    # 400 is beyond q_pos = 299
    pb = B().problem_from_inputs(inp)
    out, lse = B().sparse_mla(pb, inp.sm_scale, inp.q, inp.kv_cache, idx)
    torch.cuda.synchronize()
    assert torch.all(out[0] == 0) and torch.all(torch.isneginf(lse[0]))
    oi = to_oracle(inp)
    o_ref, l_ref = oracle.query_attention(oi, 1, [5, 299])
    check_attention(out[1].float().cpu().numpy(), lse[1].cpu().numpy(), o_ref, l_ref, 2e-2, "invalid entries")


def test_zero_queries_is_a_no_op():
    _say("zero queries")
    wl = big_dims(mode="decode", num_seqs=2, length=100, k=64)
    inp = generate(wl, DEV)
    pb = B().make_problem(mode="decode", q_pos=inp.q_pos[:0], max_ctx=100, num_seqs=2, max_seq_len=100, topk=64)
    out, lse, idx = B().forward(pb, inp.q_idx, None, inp.w, inp.k_cache, None, inp.q, inp.kv_cache, inp.sm_scale)
    torch.cuda.synchronize()
    assert out.shape[0] == 0 and idx.shape[0] == 0
