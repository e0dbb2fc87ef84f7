"""The indexer's warm-up objective on the GPU, through the C ABI, against the oracle:
the head-aggregated dense attention distribution, the per-query KL rows with
their score gradient, and the gradients into q_I, w and k_I.

Tolerances (the pages state none for this path; derived from the arithmetic):
the target distribution is exp(z - lse) with fp32 logits of exact bf16
products, so its entries agree to 2e-3 of the row's largest weight and in L1
distance; the KL rows are fp32 over at most 2^18 terms, checked to 1e-4
relative on the same fp32 inputs.  For a given score gradient, dw (fp32
throughout) agrees to 1e-4 relative RMS and dq, dk, which take the masked,
weighted score gradient as a bf16 MFMA operand (2^-9 relative rounding), to
1e-2; end to end, where the two sides' score gradients differ as well, 1e-3
and 2e-2.  Beside these norm gates every element of dq, dw and dk is checked
against a bound derived from the same arithmetic (``_bwd_with_bounds``), for
the score gradient the GPU used."""
import math

import numpy as np
import pytest
import torch

import oracle
from tests.helpers import to_oracle, to_oracle_rows
from tests.test_gpu_ops import B, DEV, _say, big_dims
from workloads import generate

pytestmark = pytest.mark.gpu


def _probs(inp, ld=None):
    pb = B().problem_from_inputs(inp)
    lse = torch.empty((inp.num_q, inp.wl.heads), dtype=torch.float32, device=DEV)
    probs, _ = B().attention_probs(pb, inp.sm_scale, inp.q, inp.kv_cache, ld=ld, lse=lse)
    torch.cuda.synchronize()
    return probs, lse


def check_distribution(got, want, what):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    assert got.shape == want.shape, what
    if want.size == 0:
        return
    err = np.abs(got - want)
    assert err.max() <= 2e-3 * want.max(), f"{what}: max err {err.max():.3e} vs max p {want.max():.3e}"
    assert err.sum() <= 2e-3, f"{what}: L1 distance {err.sum():.3e}"


PROB_CASES = [
    ("decode_paged_ragged", big_dims(mode="decode", num_seqs=4, length=5000, k=64, paged=True), [5000, 1, 64, 2049], 1.0),
    ("decode_sharp", big_dims(mode="decode", num_seqs=2, length=4100, k=64), [4100, 1300], 1200.0),
    ("decode_long_128_splits", big_dims(mode="decode", num_seqs=1, length=140000, k=64), [140000], 1.0),
    ("prefill_one_split", big_dims(mode="prefill", length=300, k=64), None, 1.0),
    ("prefill_odd_rows", big_dims(mode="prefill", length=301, k=64), None, 1.0),     # last query pair has one row
    ("prefill_odd_rows_sharp", big_dims(mode="prefill", length=2500, k=64, prefill_q_start=2187), None, 900.0),
    ("prefill_two_splits", big_dims(mode="prefill", length=2600, k=64, prefill_q_start=2450), None, 1.0),
]


@pytest.mark.parametrize("name,wl,lengths,qmul", PROB_CASES, ids=[c[0] for c in PROB_CASES])
def test_attention_probs(name, wl, lengths, qmul):
    _say("attention_probs", name)
    inp = generate(wl, DEV, lengths=lengths)
    if qmul != 1.0:
        inp.q = (inp.q.float() * qmul).to(inp.q.dtype)
    ld = inp.max_ctx + 37
    probs, lse = _probs(inp, ld=ld)
    pg, lg = probs.cpu().numpy(), lse.cpu().numpy()
    oi = to_oracle(inp)
    for t in range(inp.num_q):
        n = int(inp.q_pos[t]) + 1
        check_distribution(pg[t, :n], oracle.attention_distribution(oi, t), f"{name} row {t}")
        assert np.all(pg[t, n:] == 0), f"{name} row {t}: entries past the candidates"
        _, l_ref = oracle.dense_attention(oi, t)
        assert np.max(np.abs(lg[t] - l_ref)) <= 2e-3, f"{name} row {t}: lse"


def test_attention_probs_given_lse():
    """The target from the lse that dsa_dense_mla returns (one pass instead of two)."""
    _say("attention_probs given lse")
    inp = generate(big_dims(mode="prefill", length=2600, k=64, prefill_q_start=2450), DEV)
    pb = B().problem_from_inputs(inp)
    _, lse = B().dense_mla(pb, inp.sm_scale, inp.q, inp.kv_cache)
    probs, _ = B().attention_probs(pb, inp.sm_scale, inp.q, inp.kv_cache, lse=lse, lse_given=True)
    own, _ = _probs(inp)
    torch.cuda.synchronize()
    oi = to_oracle(inp)
    pg = probs.cpu().numpy()
    assert np.max(np.abs(pg - own.cpu().numpy())) <= 1e-6
    for t in (0, 75, inp.num_q - 1):
        n = int(inp.q_pos[t]) + 1
        oi_rows, local = to_oracle_rows(inp, [t])
        check_distribution(pg[t, :n], oracle.attention_distribution(oi_rows, local[0]), f"given lse row {t}")


def _kl_inputs(wl, lengths=None):
    inp = generate(wl, DEV, lengths=lengths)
    pb = B().problem_from_inputs(inp)
    scores = B().index_scores(pb, inp.q_idx, inp.q_scale, inp.w, inp.k_cache, inp.k_scale)
    probs, _ = _probs(inp, ld=scores.stride(0))
    return inp, pb, scores, probs


KL_CASES = [
    ("decode_paged_ragged", big_dims(mode="decode", num_seqs=3, length=5000, k=64, paged=True), [5000, 1, 3001]),
    ("prefill", big_dims(mode="prefill", length=700, k=64)),
]


@pytest.mark.parametrize("name,wl,lengths", [c + (None,) if len(c) == 2 else c for c in KL_CASES],
                         ids=[c[0] for c in KL_CASES])
def test_indexer_kl_rows(name, wl, lengths):
    """The KL kernel against the oracle's kl_rows on the same fp32 scores and target,
    then the loss end to end against the oracle's objective."""
    _say("indexer_kl", name)
    inp, pb, scores, probs = _kl_inputs(wl, lengths)
    I = scores.cpu().numpy().astype(np.float64)
    P = probs.cpu().numpy().astype(np.float64)
    loss = B().indexer_kl(pb, scores, probs)
    torch.cuda.synchronize()
    G, L = scores.cpu().numpy(), loss.cpu().numpy()
    oi = to_oracle(inp)
    for t in range(inp.num_q):
        n = int(inp.q_pos[t]) + 1
        l_ref, g_ref = oracle.kl_rows(I[t, :n], P[t, :n])
        assert abs(L[t] - l_ref) <= 1e-4 * max(abs(l_ref), 1e-3), f"{name} row {t}: loss {L[t]} vs {l_ref}"
        assert np.max(np.abs(G[t, :n] - g_ref)) <= 1e-5 * max(np.abs(g_ref).max(), 1e-6), f"{name} row {t}: grad"
        assert np.all(G[t, n:] == 0), f"{name} row {t}: gradient past the candidates"
    rows = list(range(inp.num_q)) if inp.mode == "decode" else [0, 1, 350, inp.num_q - 1]
    oi, local = to_oracle_rows(inp, rows)
    ref = oracle.indexer_kl_loss(oi, local)
    for i, t in enumerate(rows):
        assert abs(L[t] - ref["loss"][i]) <= 1e-3 * max(abs(ref["loss"][i]), 1e-3), f"{name} row {t}: end to end"


def _bwd_with_bounds(q_t, w_t, keys, g):
    """The oracle's dq, dw, dk of one query for the score gradient g, with a bound on
    each element's error that follows from the kernels' arithmetic:

    * x = q . k is an fp32 MFMA sum of exact bf16 products, off by at most
      eps = 2^-16 * sum_d |q_d k_d| (a 256x margin over fp32 rounding of 128 terms);
      where |x| <= eps the GPU's ReLU mask may differ from the oracle's, and such a
      term may be wholly present or absent (it is added to the bound in full).
    * G = g w [x > 0] enters the dq and dk products as a bf16 operand: relative
      rounding 2^-9, bounded here by 2^-8; the fp32 accumulation of N terms adds at
      most N 2^-23 of the sum of their magnitudes.
    * dw = sum_s g ReLU(x) is fp32 throughout, and ReLU is continuous, so a mask
      flip costs at most |g| eps.

    Returns (dq, dw, dk, dq_bound, dw_bound, dk_bound) for this query; the dk
    terms carry the N used (heads x keys for dq, heads for one query's dk)."""
    x = q_t @ keys.T                                             # [H_I, n]
    eps = 2.0 ** -16 * (np.abs(q_t) @ np.abs(keys).T)
    amb = np.abs(x) <= eps
    on = x > 0
    H_I, n = x.shape
    gm = np.abs(g)[None, :] * np.abs(w_t)[:, None]               # |g w| per (head, key)
    dq, dw, dk = oracle.index_scores_backward(q_t, w_t, keys, g)
    a_on = (gm * on) @ np.abs(keys)                              # sum of |G k| over the keys
    a_amb = (gm * amb) @ np.abs(keys)
    dq_b = (2.0 ** -8 + n * 2.0 ** -23) * a_on + a_amb
    dw_b = (np.abs(g)[None, :] * eps).sum(axis=1) + n * 2.0 ** -23 * (np.abs(g)[None, :] * np.maximum(x, 0)).sum(axis=1)
    k_on = (gm * on).T @ np.abs(q_t)                             # [n, d_I]
    k_amb = (gm * amb).T @ np.abs(q_t)
    dk_b = (2.0 ** -8) * k_on + k_amb
    return dq, dw, dk, dq_b, dw_b, dk_b, k_on


def _check_within(got, want, bound, what):
    """Element-wise |got - want| <= bound (+ a 1e-30 floor for exact zeros)."""
    got = np.asarray(got, dtype=np.float64)
    d = np.abs(got - want) - bound - 1e-30
    if np.any(d > 0):
        i = np.unravel_index(np.argmax(d), d.shape)
        raise AssertionError(f"{what}: {int((d > 0).sum())} elements outside the bound; worst at {i}: "
                             f"got {got[i]:.6e} want {want[i]:.6e} bound {bound[i]:.3e}")


def _rel_rms(got, want):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    nrm = np.linalg.norm(want)
    return np.linalg.norm(got - want) / nrm if nrm > 0 else np.linalg.norm(got)


BWD_CASES = [
    ("prefill_700", big_dims(mode="prefill", length=700, k=64), None),                    # 2 query splits for dk
    ("prefill_few_rows", big_dims(mode="prefill", length=2600, k=64, prefill_q_start=2450), None),   # dq key splits
    ("decode_paged_ragged", big_dims(mode="decode", num_seqs=3, length=5000, k=64, paged=True), [5000, 1, 3001]),
    ("decode_contig", big_dims(mode="decode", num_seqs=2, length=2100, k=64), [2100, 64]),
]


@pytest.mark.parametrize("name,wl,lengths", BWD_CASES, ids=[c[0] for c in BWD_CASES])
def test_indexer_backward(name, wl, lengths):
    """dq, dw, dk for a given score gradient (seeded random) against the oracle's
    index_scores_backward on the same values; dk rows no query sees stay 0."""
    _say("indexer_backward", name)
    inp = generate(wl, DEV, lengths=lengths)
    pb = B().problem_from_inputs(inp)
    gen = torch.Generator(device=DEV).manual_seed(7)
    ld = inp.max_ctx + 3
    grad = torch.randn((inp.num_q, ld), device=DEV, generator=gen, dtype=torch.float32) * 1e-3
    dq, dw, dk = B().indexer_backward(pb, inp.q_idx, inp.w, inp.k_cache, grad)
    torch.cuda.synchronize()
    G = grad.cpu().numpy().astype(np.float64)
    oi = to_oracle(inp)
    dk_ref = np.zeros(dk.shape, dtype=np.float64)
    dk_bnd = np.zeros(dk.shape, dtype=np.float64)
    dk_mag = np.zeros(dk.shape, dtype=np.float64)
    dk_cnt = np.zeros(dk.shape[:-1], dtype=np.float64)
    dqg, dwg, dkg = dq.cpu().numpy(), dw.cpu().numpy(), dk.cpu().numpy()
    dq_ref = np.zeros(dqg.shape)
    dw_ref = np.zeros(dwg.shape)
    for t in range(inp.num_q):
        q_t, w_t, keys = oracle.query_index_operands(oi, t)
        n = keys.shape[0]
        dq_ref[t], dw_ref[t], dk_t, dq_b, dw_b, dk_b, k_on = _bwd_with_bounds(q_t, w_t, keys, G[t, :n])
        _check_within(dqg[t], dq_ref[t], dq_b, f"{name}: dq of query {t}")
        _check_within(dwg[t], dw_ref[t], dw_b, f"{name}: dw of query {t}")
        b = oracle.sequence_of(oi, t)
        pos = np.arange(n)
        if oi.block_table is None:
            where = (np.full(n, b), pos)
        else:
            blocks = np.asarray(oi.block_table[b], dtype=np.int64)[pos // oi.block_size]
            where = (blocks, pos % oi.block_size)
        np.add.at(dk_ref, where, dk_t)
        np.add.at(dk_bnd, where, dk_b)
        np.add.at(dk_mag, where, k_on)
        np.add.at(dk_cnt, where, float(q_t.shape[0]))
    # fp32 accumulation over every (query, head) term of a key
    _check_within(dkg, dk_ref, dk_bnd + dk_cnt[..., None] * 2.0 ** -23 * dk_mag, f"{name}: dk")
    assert _rel_rms(dwg, dw_ref) <= 1e-4, f"{name}: dw rel RMS {_rel_rms(dwg, dw_ref):.3e}"
    assert _rel_rms(dqg, dq_ref) <= 1e-2, f"{name}: dq rel RMS {_rel_rms(dqg, dq_ref):.3e}"
    assert _rel_rms(dkg, dk_ref) <= 1e-2, f"{name}: dk rel RMS {_rel_rms(dkg, dk_ref):.3e}"
    for t in range(inp.num_q):
        assert _rel_rms(dqg[t], dq_ref[t]) <= 2e-2, f"{name}: dq row {t}"
    # rows of keys nobody sees are untouched (zeros from the default output)
    seen = np.abs(dk_ref).sum(axis=-1) > 0
    assert np.all(dkg[~seen] == 0) or np.all(np.abs(dkg[~seen]) <= 1e-12), f"{name}: dk written where unseen"


def test_indexer_objective_end_to_end():
    """probs -> index scores -> KL -> backward on the GPU, against the oracle's whole
    objective (loss per query, dq, dw, dk)."""
    _say("indexer objective end to end")
    inp = generate(big_dims(mode="prefill", length=600, k=64), DEV)
    pb = B().problem_from_inputs(inp)
    scores = B().index_scores(pb, inp.q_idx, inp.q_scale, inp.w, inp.k_cache, inp.k_scale)
    probs, _ = _probs(inp, ld=scores.stride(0))
    loss = B().indexer_kl(pb, scores, probs)
    dq, dw, dk = B().indexer_backward(pb, inp.q_idx, inp.w, inp.k_cache, scores)
    torch.cuda.synchronize()
    oi = to_oracle(inp)
    ref = oracle.indexer_kl_loss(oi)
    lg = loss.cpu().numpy()
    assert np.max(np.abs(lg - ref["loss"]) / np.maximum(np.abs(ref["loss"]), 1e-3)) <= 1e-3
    assert _rel_rms(dw.cpu().numpy(), ref["dw"]) <= 1e-3
    assert _rel_rms(dq.cpu().numpy(), ref["dq"]) <= 2e-2
    assert _rel_rms(dk.cpu().numpy(), ref["dk"]) <= 2e-2
    # element by element, for the score gradient the GPU computed (written over the scores)
    G = scores.cpu().numpy().astype(np.float64)
    dqg, dwg = dq.cpu().numpy(), dw.cpu().numpy()
    for t in range(inp.num_q):
        q_t, w_t, keys = oracle.query_index_operands(oi, t)
        n = keys.shape[0]
        dq_r, dw_r, _, dq_b, dw_b, _, _ = _bwd_with_bounds(q_t, w_t, keys, G[t, :n])
        _check_within(dqg[t], dq_r, dq_b, f"end to end: dq of query {t}")
        _check_within(dwg[t], dw_r, dw_b, f"end to end: dw of query {t}")


def test_indexer_objective_full_size():
    """The fused objective on the 16K-token prefill the benchmark times: sampled query
    rows (loss end to end; dq, dw for the GPU's own score gradient) and sampled keys
    (dk summed over every query that sees the key) against the oracle."""
    from workloads import WORKLOADS, raw_numpy
    _say("indexer objective full size", "prefill_16k_bf16")
    inp = generate(WORKLOADS["prefill_16k_bf16"], DEV)
    pb = B().problem_from_inputs(inp)
    ws = torch.empty(B().workspace_size(B().OP_INDEXER_KL_LOSS, pb), dtype=torch.uint8, device=DEV)
    loss, dq, dw, dk = B().indexer_kl_loss(pb, inp.q_idx, inp.w, inp.k_cache, inp.q, inp.kv_cache, inp.sm_scale,
                                           ws=ws)
    torch.cuda.synchronize()
    T = inp.num_q
    ld = (inp.max_ctx + 63) // 64 * 64
    grad = ws[: T * ld * 4].view(torch.float32).view(T, ld)
    assert torch.isfinite(loss).all() and torch.isfinite(dq).all() and torch.isfinite(dk).all()
    rows = [0, 1, 2047, 2048, 9000, T - 1]
    oi, local = to_oracle_rows(inp, rows)
    ref = oracle.indexer_kl_loss(oi, local)
    L, G = loss.cpu().numpy(), grad[rows].cpu().numpy().astype(np.float64)
    for i, t in enumerate(rows):
        assert abs(L[t] - ref["loss"][i]) <= 1e-3 * max(abs(ref["loss"][i]), 1e-3), f"row {t}: loss"
        q_t, w_t, keys = oracle.query_index_operands(oi, local[i])
        n = keys.shape[0]
        dq_ref, dw_ref, _, dq_b, dw_b, _, _ = _bwd_with_bounds(q_t, w_t, keys, G[i, :n])
        assert _rel_rms(dw[t].cpu().numpy(), dw_ref) <= 1e-4, f"row {t}: dw"
        assert _rel_rms(dq[t].cpu().numpy(), dq_ref) <= 1e-2, f"row {t}: dq"
        _check_within(dq[t].cpu().numpy(), dq_ref, dq_b, f"row {t}: dq")
        _check_within(dw[t].cpu().numpy(), dw_ref, dw_b, f"row {t}: dw")
    # dk of sampled keys from every query's gradient column, in chunks of queries
    keys_s = [0, 5, 8000, T - 1]
    kc = oracle.decode_bf16(raw_numpy(inp.k_cache[0, :T]))
    qpos = raw_numpy(inp.q_pos).astype(np.int64)
    wv = raw_numpy(inp.w).astype(np.float64)
    gcols = grad[:, keys_s].cpu().numpy().astype(np.float64)
    dk_ref = np.zeros((len(keys_s), 128))
    dk_bnd = np.zeros((len(keys_s), 128))
    dk_mag = np.zeros((len(keys_s), 128))
    dk_cnt = np.zeros(len(keys_s))
    for c0 in range(0, T, 1024):
        qc = oracle.decode_bf16(raw_numpy(inp.q_idx[c0:c0 + 1024]))              # [c, 64, 128]
        for j, s in enumerate(keys_s):
            x = qc @ kc[s]                                                        # [c, 64]
            eps = 2.0 ** -16 * (np.abs(qc) @ np.abs(kc[s]))
            seen = (qpos[c0:c0 + 1024] >= s)[:, None]
            gw = gcols[c0:c0 + 1024, j][:, None] * wv[c0:c0 + 1024] * seen
            gm = gw * (x > 0)
            dk_ref[j] += np.einsum("ch,chd->d", gm, qc)
            k_on = np.einsum("ch,chd->d", np.abs(gm), np.abs(qc))
            dk_mag[j] += k_on
            dk_bnd[j] += 2.0 ** -8 * k_on + np.einsum("ch,chd->d", np.abs(gw) * (np.abs(x) <= eps), np.abs(qc))
            dk_cnt[j] += 64 * int(seen.sum())
    dkg = dk[0, keys_s].cpu().numpy()
    for j, s in enumerate(keys_s):
        assert _rel_rms(dkg[j], dk_ref[j]) <= 2e-2, f"key {s}: dk rel RMS {_rel_rms(dkg[j], dk_ref[j]):.3e}"
        _check_within(dkg[j], dk_ref[j], dk_bnd[j] + dk_cnt[j] * 2.0 ** -23 * dk_mag[j], f"key {s}: dk")


def test_indexer_objective_edge_cases():
    """A query with no candidates and one with a single candidate: loss 0, zero gradients
    (one candidate: p = softmax(I) = [1]); a full row next to them matches the oracle."""
    _say("indexer objective edge cases")
    inp = generate(big_dims(mode="decode", num_seqs=3, length=3000, k=64, paged=True), DEV, lengths=[3000, 1, 2000])
    inp.q_pos[2] = -1
    pb = B().problem_from_inputs(inp)
    dk0 = torch.full(tuple(inp.k_cache.shape), 7.0, dtype=torch.float32, device=DEV)
    loss, dq, dw, dk = B().indexer_kl_loss(pb, inp.q_idx, inp.w, inp.k_cache, inp.q, inp.kv_cache, inp.sm_scale,
                                           dk=dk0)
    torch.cuda.synchronize()
    L = loss.cpu().numpy()
    assert L[1] == 0.0 and L[2] == 0.0
    assert torch.all(dq[1:] == 0) and torch.all(dw[1:] == 0)
    # the sequence without a query sees no key: its slots keep their contents
    bt = inp.block_table[2]
    for blk in bt[: (2000 + 63) // 64].tolist():
        assert torch.all(dk[blk] == 7.0)
    # the single candidate's slot is written with 0
    assert torch.all(dk[int(inp.block_table[1, 0]), 0] == 0)
    ref = oracle.indexer_kl_loss(to_oracle(inp), [0])
    assert abs(L[0] - ref["loss"][0]) <= 1e-3 * abs(ref["loss"][0])
    assert _rel_rms(dq[0].cpu().numpy(), ref["dq"][0]) <= 2e-2
