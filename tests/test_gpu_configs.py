"""Every workload at its full size, in the launch configuration the benchmark times.

The oracle checks sampled query rows (scores, top-k within the near-tie band,
attention).  Every row of every workload is also checked without the oracle:
the fused path's selection equals dsa_topk on dsa_index_scores' own fp32 rows
bit for bit, and passes the top-k certificate on those rows (size, range,
separation, ties to the lower position)."""
import zlib

import numpy as np
import pytest
import torch

import oracle
from tests.helpers import (OUT_TOL, SCORE_TOL, check_attention, check_scores, check_topk_row_e2e,
                           to_oracle_rows)
from tests.test_gpu_ops import B, DEV, _say
from workloads import WORKLOADS, generate

pytestmark = pytest.mark.gpu


def certificate_all_rows(scores, idx, q_pos, k, chunk=1024):
    """Vectorised top-k certificate on the GPU for every row."""
    T = idx.shape[0]
    for r0 in range(0, T, chunk):
        sc = scores[r0:r0 + chunk]
        ix = idx[r0:r0 + chunk].long()
        n = q_pos[r0:r0 + chunk].long() + 1
        R, L = sc.shape
        m = torch.clamp(n, max=k)
        cnt = (ix >= 0).sum(1)
        assert torch.equal(cnt, m), "selection size"
        valid_slot = torch.arange(k, device=ix.device)[None, :] < m[:, None]
        assert torch.all((ix >= 0) == valid_slot), "padding"
        assert torch.all(ix[valid_slot] < n.repeat_interleave(m)), "range"
        srt = torch.where(valid_slot, ix, torch.full_like(ix, 1 << 40))
        s2 = srt.sort(1).values
        assert torch.all((s2[:, 1:] > s2[:, :-1]) | (s2[:, 1:] == (1 << 40))), "duplicates / order"
        sel = torch.zeros((R, L + 1), dtype=torch.bool, device=sc.device)   # column L: padding sink
        sel.scatter_(1, torch.where(valid_slot, ix, torch.full_like(ix, L)), valid_slot)
        sel = sel[:, :L]
        cand = torch.arange(L, device=sc.device)[None, :] < n[:, None]
        x = sc + 0.0
        lo = torch.where(sel, x, torch.full_like(x, float("inf"))).min(1).values
        hi = torch.where(cand & ~sel, x, torch.full_like(x, float("-inf"))).max(1).values
        assert torch.all(lo >= hi), "separation"
        tie = (lo == hi)
        if tie.any():
            pos = torch.arange(L, device=sc.device)[None, :].expand(R, L)
            eq = x == lo[:, None]
            last_sel = torch.where(sel & eq, pos, torch.full_like(pos, -1)).max(1).values
            first_un = torch.where(cand & ~sel & eq, pos, torch.full_like(pos, L)).min(1).values
            assert torch.all((last_sel < first_un) | ~tie), "ties must go to the lower position"


def sample_rows(inp, extra, seed):
    T = inp.num_q
    if inp.mode == "decode":
        rng = np.random.default_rng(seed)
        return sorted(rng.choice(T, size=min(extra, T), replace=False).tolist())
    base = [0, 1, 2046, 2047, 2048, 2049, T - 1]
    rng = np.random.default_rng(seed)
    rows = set(t for t in base if t < T) | set(rng.integers(0, T, size=extra).tolist())
    return sorted(rows)


CASES = [
    ("tiny_prefill_f32", 64),
    ("decode_8k_bf16", 16),
    ("prefill_16k_bf16", 24),
    ("decode_128k_paged_bf16", 6),
    ("decode_128k_exact_paged_bf16", 3),
    ("decode_128k_paged_fp8", 4),
    ("prefill_64k_fp8", 10),
]


@pytest.mark.parametrize("name,extra", CASES, ids=[c[0] for c in CASES])
def test_workload_full_size(name, extra):
    _say("full-size", name)
    inp = generate(WORKLOADS[name], DEV)
    torch.cuda.synchronize()
    out, lse, idx = B().forward_inputs(inp)
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all() and not torch.isnan(lse).any()

    # every row: fused selection == dsa_topk on dsa_index_scores, and the certificate
    pb = B().problem_from_inputs(inp)
    scores = B().index_scores(pb, inp.q_idx, inp.q_scale, inp.w, inp.k_cache, inp.k_scale)
    idx2 = B().topk(pb, scores)
    torch.cuda.synchronize()
    assert torch.equal(idx, idx2), "fused path differs from the staged ops"
    certificate_all_rows(scores, idx, inp.q_pos, inp.topk)

    # sampled rows against the oracle
    rows = sample_rows(inp, extra, seed=zlib.crc32(name.encode()))
    oi, local = to_oracle_rows(inp, rows)
    sc_h = scores[rows].cpu().numpy() if inp.mode == "prefill" else scores.cpu().numpy()
    ig, og, lg = idx.cpu().numpy(), out.float().cpu().numpy(), lse.cpu().numpy()
    tol_s = SCORE_TOL[inp.wl.index_dtype]
    for i, t in enumerate(rows):
        li = local[i]
        ref = oracle.query_index_scores(oi, li)
        n = ref.shape[0]
        check_scores((sc_h[i] if inp.mode == "prefill" else sc_h[t])[:n], ref, tol_s, f"{name} row {t}")
        check_topk_row_e2e(ig[t], ref, inp.topk, f"{name} row {t}")
        m = min(inp.topk, n)
        o_ref, l_ref = oracle.query_attention(oi, li, ig[t, :m])
        check_attention(og[t], lg[t], o_ref, l_ref, OUT_TOL[inp.wl.mla_dtype], f"{name} row {t}")


RAGGED_CASES = [
    # T = 8192 + 100: one full query chunk, then a 100-row chunk (sliced top-k, split attention rows)
    ("prefill_8292_bf16", dict(mode="prefill", length=8292, k=2048)),
    # T = 8192 + 255 with the e4m3fn indexer and a paged cache
    ("prefill_8447_fp8_paged", dict(mode="prefill", length=8447, k=2048, index_dtype="fp8", paged=True)),
]


@pytest.mark.parametrize("name,kw", RAGGED_CASES, ids=[c[0] for c in RAGGED_CASES])
def test_prefill_ragged_tail_chunk(name, kw):
    """A prefill whose last query chunk is short runs it with its own top-k and
    attention layouts inside the workspace sized by dsa_workspace_size: every row
    equals the staged ops bit for bit and passes the certificate, and sampled rows
    on both sides of the chunk boundary match the oracle."""
    from tests.test_gpu_ops import big_dims
    _say("ragged tail chunk", name)
    inp = generate(big_dims(**kw), DEV)
    pb = B().problem_from_inputs(inp)
    assert B().forward_chunk_rows(pb) == 8192 and 0 < inp.num_q % 8192 < 256
    out, lse, idx = B().forward_inputs(inp)
    scores = B().index_scores(pb, inp.q_idx, inp.q_scale, inp.w, inp.k_cache, inp.k_scale)
    idx2 = B().topk(pb, scores)
    out2, lse2 = B().sparse_mla(pb, inp.sm_scale, inp.q, inp.kv_cache, idx2)
    torch.cuda.synchronize()
    assert torch.equal(idx, idx2), "fused selection differs from the staged ops"
    certificate_all_rows(scores, idx, inp.q_pos, inp.topk)
    # the staged attention runs every row in one launch (other splits): within tolerance
    assert torch.max(torch.abs(out.float() - out2.float())).item() <= 2e-2
    T = inp.num_q
    rows = [0, 2048, 8191, 8192, 8193, T - 2, T - 1]
    oi, local = to_oracle_rows(inp, rows)
    sc_h = scores[rows].cpu().numpy()
    ig, og, lg = idx.cpu().numpy(), out.float().cpu().numpy(), lse.cpu().numpy()
    for i, t in enumerate(rows):
        ref = oracle.query_index_scores(oi, local[i])
        n = ref.shape[0]
        check_scores(sc_h[i][:n], ref, SCORE_TOL[inp.wl.index_dtype], f"{name} row {t}")
        check_topk_row_e2e(ig[t], ref, inp.topk, f"{name} row {t}")
        o_ref, l_ref = oracle.query_attention(oi, local[i], ig[t, :min(inp.topk, n)])
        check_attention(og[t], lg[t], o_ref, l_ref, OUT_TOL["bf16"], f"{name} row {t}")
