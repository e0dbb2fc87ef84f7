"""Stage 2 of training on the GPU, through the C ABI, against the oracle: the
sparse attention's gradient (dq, and the latent-row gradients summed into the
cache rows), the indexer's target over the selection, and the indexer's KL on
the selected subset with its gradient.

Tolerances (the pages state none for training; derived from the arithmetic).
The GPU forms P = exp(z - lse) and dS = P (dP - Delta) in fp32 and rounds P and
sm_scale dS to bf16 as MFMA operands (relative 2^-9); Delta uses the forward's
bf16 output (each term off by at most 2^-9 of |dout out|).  So every element
of dq and of a cache row's gradient lies within

    2^-7 * (sum of the magnitudes of its bf16-operand terms)
    + sm_scale * sum_j P_j |Delta error| |operand|

of the exact value (2^-7 covers the operand rounding, the fp32 sums and the
fp32 logits with a 2x margin), and the norms agree to 1e-2 relative.  The KL
rows are fp32 on the same inputs: 1e-4 relative."""
import math

import numpy as np
import pytest
import torch

import oracle
from tests.helpers import to_oracle, to_oracle_rows
from tests.test_gpu_loss import _bwd_with_bounds, _check_within, _rel_rms
from tests.test_gpu_ops import B, DEV, _say, big_dims
from workloads import generate, raw_numpy

pytestmark = pytest.mark.gpu


def _dout(inp, seed):
    g = torch.Generator(device=DEV).manual_seed(seed)
    return (torch.randn((inp.num_q, inp.wl.heads, inp.wl.v_dim), device=DEV, generator=g) * 0.05).to(torch.bfloat16)


def _exact_parts(oi, t, sel, dout_t, out_gpu_t):
    """Exact P, dS (float64) of query t over `sel`, the rows and q, and a bound on
    |Delta_gpu - Delta| per head from the bf16 rounding of the forward output."""
    b = oracle.sequence_of(oi, t)
    q = oracle.decode(oi.q[t], oi.mla_dtype)
    rows = oracle.decode(oracle.gather_rows(oi.kv_cache, oi, b, sel), oi.mla_dtype)
    Dv = oi.v_dim
    z = oi.sm_scale * (q @ rows.T)
    p = np.exp(z - z.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    dp = dout_t @ rows[:, :Dv].T
    ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
    ddelta = 2.0 ** -8 * np.abs(dout_t * out_gpu_t).sum(axis=1)
    return p, ds, q, rows, ddelta


def _dq_bound(oi, p, ds, rows, ddelta):
    s = oi.sm_scale
    return 2.0 ** -7 * s * (np.abs(ds) @ np.abs(rows)) + s * (ddelta[:, None] * (p @ np.abs(rows)))


def _row_terms(oi, p, ds, q, dout_t, ddelta):
    """Per selected row: the magnitude bound of its gradient from this query."""
    s, Dv = oi.sm_scale, oi.v_dim
    mag = 2.0 ** -7 * s * (np.abs(ds).T @ np.abs(q))
    mag[:, :Dv] += 2.0 ** -7 * (p.T @ np.abs(dout_t))
    mag += s * ((p * ddelta[:, None]).T @ np.abs(q))
    return mag


def _run(inp, dout):
    pb = B().problem_from_inputs(inp)
    out, lse, idx = B().forward_inputs(inp)
    dq, dkv, probs = B().sparse_mla_backward(pb, inp.sm_scale, inp.q, inp.kv_cache, idx, out, lse, dout)
    torch.cuda.synchronize()
    return out, lse, idx, dq, dkv, probs


BWD_CASES = [
    # two query chunks (256 + 44 rows), k = 64 of up to 300 candidates
    ("prefill_300_k64", dict(mode="prefill", length=300, k=64), 1.0),
    # every candidate selected (n <= k): the padded tail of each list is absent
    ("prefill_600_all", dict(mode="prefill", length=600, k=2048, prefill_q_start=400), 1.0),
    # paged cache, sharp logits (q scaled so the weights are far from uniform)
    ("prefill_520_paged_sharp", dict(mode="prefill", length=520, k=128, paged=True), 1000.0),
    # long lists: 2048 of up to 2600 candidates
    ("prefill_2600_k2048", dict(mode="prefill", length=2600, k=2048, prefill_q_start=2520), 1.0),
]


@pytest.mark.parametrize("name,kw,qmul", BWD_CASES, ids=[c[0] for c in BWD_CASES])
def test_sparse_mla_backward(name, kw, qmul):
    _say("sparse_mla_backward", name)
    inp = generate(big_dims(**kw), DEV)
    if qmul != 1.0:
        inp.q = (inp.q.float() * qmul).to(inp.q.dtype)
    dout = _dout(inp, 5)
    out, lse, idx, dq, dkv, probs = _run(inp, dout)
    oi = to_oracle(inp)
    ig = idx.cpu().numpy()
    D = inp.wl.qk_dim
    dout_h = dout.float().cpu().numpy().astype(np.float64)
    out_h = out.float().cpu().numpy().astype(np.float64)
    ref = oracle.sparse_attention_backward(oi, ig, dout_h)
    dqg, dkvg, pg = dq.cpu().numpy(), dkv.cpu().numpy(), probs.cpu().numpy()
    assert _rel_rms(dqg, ref["dq"]) <= 1e-2, f"{name}: dq rel RMS {_rel_rms(dqg, ref['dq']):.3e}"
    kvb = np.zeros(ref["dkv"].shape)
    for t in range(inp.num_q):
        sel = ig[t][ig[t] >= 0]
        p, ds, q, rows, dd = _exact_parts(oi, t, sel, dout_h[t], out_h[t])
        _check_within(dqg[t], ref["dq"][t], _dq_bound(oi, p, ds, rows, dd), f"{name}: dq of query {t}")
        oracle.dsa_oracle._add_rows(kvb, oi, 0, sel, _row_terms(oi, p, ds, q, dout_h[t], dd))
        # the Stage-2 target: head-mean weights over the selection, slot by slot
        want = oracle.sparse_attention_distribution(oi, t, sel)
        got = pg[t][ig[t] >= 0]
        assert np.max(np.abs(got - want)) <= 2e-3 * want.max() and np.abs(got - want).sum() <= 2e-3, f"probs {t}"
        assert np.all(pg[t][ig[t] < 0] == 0)
    rows_kv = ref["dkv"].reshape(-1, D)
    assert _rel_rms(dkvg.reshape(-1, D), rows_kv) <= 1e-2, f"{name}: dkv rel RMS"
    _check_within(dkvg.reshape(-1, D), rows_kv, kvb.reshape(-1, D), f"{name}: dkv")


def test_sparse_mla_backward_deterministic_and_paged():
    """Two runs give the same bytes; the same logical cache in permuted 64-token
    blocks gives the same dq bytes and the same row gradients at the mapped slots."""
    _say("sparse_mla_backward determinism / paged")
    from tests.test_gpu_forward import _paged_copy
    inp = generate(big_dims(mode="prefill", length=700, k=256), DEV)
    dout = _dout(inp, 6)
    a = _run(inp, dout)
    b = _run(inp, dout)
    for x, y in zip(a, b):
        assert torch.equal(x, y)
    pg = _paged_copy(inp, np.random.default_rng(8))
    c = _run(pg, dout)
    assert torch.equal(a[2], c[2]) and torch.equal(a[3], c[3])
    table = pg.block_table[0].long()
    pos = torch.arange(inp.max_ctx, device=DEV)
    phys = table[pos // 64] * 64 + pos % 64
    assert torch.equal(c[4].view(-1, 576)[phys], a[4][0, : inp.max_ctx])


def test_sparse_indexer_kl():
    """The KL rows on the selection against the oracle's kl_rows on the same fp32
    scores and target; then the Stage-2 indexer objective end to end (selection,
    target, loss, and dq, dw, dk through dsa_indexer_backward) against the oracle's,
    element by element for the score gradient the GPU used."""
    _say("sparse_indexer_kl")
    inp = generate(big_dims(mode="prefill", length=700, k=128, w_low=-1 / 8), DEV)
    pb = B().problem_from_inputs(inp)
    dout = _dout(inp, 9)
    out, lse, idx, dq, dkv, probs = _run(inp, dout)
    scores = B().index_scores(pb, inp.q_idx, inp.q_scale, inp.w, inp.k_cache, inp.k_scale)
    torch.cuda.synchronize()
    I = scores.cpu().numpy().astype(np.float64)
    P = probs.cpu().numpy().astype(np.float64)
    ig = idx.cpu().numpy()
    loss = B().sparse_indexer_kl(pb, scores, idx, probs)
    torch.cuda.synchronize()
    G, L = scores.cpu().numpy(), loss.cpu().numpy()
    for t in range(inp.num_q):
        n = int(inp.q_pos[t]) + 1
        sel = ig[t][ig[t] >= 0]
        l_ref, g_ref = oracle.kl_rows(I[t, sel], P[t][ig[t] >= 0])
        assert abs(L[t] - l_ref) <= 1e-4 * max(abs(l_ref), 1e-3), f"row {t}: loss {L[t]} vs {l_ref}"
        assert np.max(np.abs(G[t, sel] - g_ref)) <= 1e-5 * max(np.abs(g_ref).max(), 1e-6), f"row {t}: grad"
        off = np.ones(G.shape[1], bool)
        off[sel] = False
        assert np.all(G[t, off] == 0), f"row {t}: gradient outside the selection"
    # end to end against the oracle's Stage-2 objective on the GPU's selection
    dqi, dwi, dki = B().indexer_backward(pb, inp.q_idx, inp.w, inp.k_cache, scores)
    torch.cuda.synchronize()
    oi = to_oracle(inp)
    ref = oracle.sparse_indexer_kl_loss(oi, selections=[ig[t][ig[t] >= 0] for t in range(inp.num_q)])
    assert np.max(np.abs(L - ref["loss"]) / np.maximum(np.abs(ref["loss"]), 1e-3)) <= 1e-3
    # the same gradients summed over the selected keys only
    dqs, dws, dks = B().indexer_backward_selected(pb, inp.q_idx, inp.w, inp.k_cache, scores, idx)
    torch.cuda.synchronize()
    assert torch.equal(dks, dki)                  # dk: the same kernel on the same gradient
    dqg, dwg = dqi.cpu().numpy(), dwi.cpu().numpy()
    dqsg, dwsg = dqs.cpu().numpy(), dws.cpu().numpy()
    Gd = G.astype(np.float64)
    for t in range(inp.num_q):
        q_t, w_t, keys = oracle.query_index_operands(oi, t)
        n = keys.shape[0]
        dq_r, dw_r, _, dq_b, dw_b, _, _ = _bwd_with_bounds(q_t, w_t, keys, Gd[t, :n])
        _check_within(dqg[t], dq_r, dq_b, f"stage-2 indexer dq of query {t}")
        _check_within(dwg[t], dw_r, dw_b, f"stage-2 indexer dw of query {t}")
        _check_within(dqsg[t], dq_r, dq_b, f"stage-2 indexer dq over the selection, query {t}")
        _check_within(dwsg[t], dw_r, dw_b, f"stage-2 indexer dw over the selection, query {t}")
    assert _rel_rms(dqg, ref["dq"]) <= 2e-2 and _rel_rms(dwg, ref["dw"]) <= 1e-3
    assert _rel_rms(dqsg, ref["dq"]) <= 2e-2 and _rel_rms(dwsg, ref["dw"]) <= 1e-3
    assert _rel_rms(dki.cpu().numpy(), ref["dk"]) <= 2e-2


def test_indexer_backward_selected_decode_paged():
    """dq, dw over the selection on a paged decode batch (rows shorter than k, a
    one-token row, a row of exactly k) for a score gradient that is random on
    the selected positions and zero elsewhere: element by element against the
    oracle's gradient bound, dk equal to dsa_indexer_backward's."""
    _say("indexer_backward_selected decode paged")
    inp = generate(big_dims(mode="decode", num_seqs=5, length=3000, k=2048, paged=True, w_low=-1 / 8), DEV,
                   lengths=[3000, 2100, 2048, 700, 1])
    pb = B().problem_from_inputs(inp)
    _, _, idx = B().forward_inputs(inp)
    torch.cuda.synchronize()
    ig = idx.cpu().numpy()
    rng = np.random.default_rng(5)
    G = np.zeros((inp.num_q, pb.seqs.max_ctx), np.float32)
    for t in range(inp.num_q):
        sel = ig[t][ig[t] >= 0]
        G[t, sel] = rng.standard_normal(sel.shape[0]).astype(np.float32) * 1e-3
    grad = torch.from_numpy(G).to(DEV)
    dqi, dwi, dki = B().indexer_backward(pb, inp.q_idx, inp.w, inp.k_cache, grad)
    dqs, dws, dks = B().indexer_backward_selected(pb, inp.q_idx, inp.w, inp.k_cache, grad, idx)
    torch.cuda.synchronize()
    assert torch.equal(dks, dki)
    oi = to_oracle(inp)
    dqsg, dwsg = dqs.cpu().numpy(), dws.cpu().numpy()
    for t in range(inp.num_q):
        q_t, w_t, keys = oracle.query_index_operands(oi, t)
        n = keys.shape[0]
        dq_r, dw_r, _, dq_b, dw_b, _, _ = _bwd_with_bounds(q_t, w_t, keys, G[t, :n].astype(np.float64))
        _check_within(dqsg[t], dq_r, dq_b, f"dq over the selection, query {t}")
        _check_within(dwsg[t], dw_r, dw_b, f"dw over the selection, query {t}")


def test_stage2_full_size():
    """The 16K-token prefill of the benchmark through forward and Stage-2 backward:
    sampled query rows' dq and target, and the gradients of late tokens (each
    selected by few queries, all of which the oracle recomputes) against the oracle."""
    from workloads import WORKLOADS
    _say("stage 2 full size", "prefill_16k_bf16")
    inp = generate(WORKLOADS["prefill_16k_bf16"], DEV)
    dout = _dout(inp, 11)
    out, lse, idx, dq, dkv, probs = _run(inp, dout)
    assert torch.isfinite(dq).all() and torch.isfinite(dkv).all() and torch.isfinite(probs).all()
    T = inp.num_q
    ig = idx.cpu().numpy()
    rows = [0, 2047, 2048, 9000, T - 1]
    oi, local = to_oracle_rows(inp, rows)
    dout_h = dout.float()[rows].cpu().numpy().astype(np.float64)
    out_h = out.float()[rows].cpu().numpy().astype(np.float64)
    dqg, pg = dq[rows].cpu().numpy(), probs[rows].cpu().numpy()
    for i, t in enumerate(rows):
        sel = ig[t][ig[t] >= 0]
        p, ds, q, crow, dd = _exact_parts(oi, local[i], sel, dout_h[i], out_h[i])
        want_dq = oi.sm_scale * (ds @ crow)
        _check_within(dqg[i], want_dq, _dq_bound(oi, p, ds, crow, dd), f"dq of query {t}")
        assert _rel_rms(dqg[i], want_dq) <= 1e-2
        want_p = p.mean(axis=0)
        assert np.max(np.abs(pg[i][ig[t] >= 0] - want_p)) <= 2e-3 * want_p.max()
    # late tokens: every query that selected them
    keys = [s for s in range(T - 40, T) if 0 < np.sum(ig[s:] == s) <= 6][:3]
    assert keys, "no late token selected by a few queries"
    for s in keys:
        ts = [t for t in range(s, T) if s in set(ig[t].tolist())]
        oi_k, loc = to_oracle_rows(inp, ts)
        d_k = dout.float()[ts].cpu().numpy().astype(np.float64)
        o_k = out.float()[ts].cpu().numpy().astype(np.float64)
        want = np.zeros(576)
        bound = np.zeros(576)
        for i, t in enumerate(ts):
            sel = ig[t][ig[t] >= 0]
            p, ds, q, crow, dd = _exact_parts(oi_k, loc[i], sel, d_k[i], o_k[i])
            j = int(np.nonzero(sel == s)[0][0])
            g = oi.sm_scale * (ds[:, j] @ q)
            g[:512] += p[:, j] @ d_k[i]
            want += g
            bound += _row_terms(oi, p, ds, q, d_k[i], dd)[j]
        got = dkv[0, s].cpu().numpy()
        _check_within(got, want, bound, f"dkv of token {s} ({len(ts)} queries)")
