"""Pins of the CPU oracle to facts fixed outside it.

Each ``pin_*`` takes the oracle module and raises ``AssertionError`` when the
oracle disagrees with: hand-derived worked examples (tests/golden), closed
forms, brute force on tiny inputs, an independent library routine (torch's
dtype casts, torch's scaled_dot_product_attention in float64), or an
invariant of the definition.  ``test_oracle.py`` runs every pin on the real
oracle; ``test_oracle_mutations.py`` runs them on deliberately broken copies
and requires each break to be caught.
"""
from __future__ import annotations

import itertools
import json
import math
import os

import numpy as np
import torch

from workloads import generate
from tests.helpers import small_workload, to_oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _close(a, b, tol=1e-12, what=""):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} != {b.shape}"
    err = np.max(np.abs(a - b) / (1.0 + np.abs(b))) if a.size else 0.0
    assert err <= tol, f"{what}: max rel err {err:.3e} > {tol}"


# ---------------------------------------------------------------- decoding

def pin_bf16_decode(o):
    """All 65536 bf16 patterns against torch's bfloat16 -> float64 cast."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    got = o.decode_bf16(bits)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan), "bf16 NaN patterns"
    assert np.array_equal(got[~nan], ref[~nan]), "bf16 values"
    assert np.signbit(got[0x8000]) and got[0x8000] == 0.0


def pin_e4m3_table(o):
    """All 256 e4m3fn codes against torch.float8_e4m3fn -> float64 (an independent implementation)."""
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = o.decode_e4m3fn(codes)
    nan = np.isnan(ref)
    assert nan.sum() == 2 and nan[0x7F] and nan[0xFF]
    assert np.array_equal(np.isnan(got), nan), "e4m3fn NaN codes"
    assert np.array_equal(got[~nan], ref[~nan]), "e4m3fn values"
    assert got[0x7E] == 448.0 and got[0x01] == 2.0 ** -9 and got[0x38] == 1.0


# ---------------------------------------------------------------- indexer (eq. I)

def pin_indexer_golden(o):
    d = _golden("indexer_hand.json")
    for c in d["cases"]:
        got = o.index_scores(np.array(c["q"], float), np.array(c["w"], float),
                             np.array(c["keys"], float))
        assert np.array_equal(got, np.array(c["expected"], float)), c["name"]
    for c in d["fp8_cases"]:
        n = len(c["k_codes"])
        inp = o.OracleInputs(
            mode="decode", q_pos=np.array([n - 1]), block_table=None, block_size=64,
            index_dtype="fp8", q_idx=np.array([c["q_codes"]], np.uint8),
            q_scale=np.array([c["q_scale"]], np.float32), w=np.array([c["w"]], np.float32),
            k_cache=np.array([c["k_codes"]], np.uint8), k_scale=np.array([c["k_scale"]], np.float32),
            mla_dtype="f32", q=np.zeros((1, 1, 2), np.float32), kv_cache=np.zeros((1, n, 2), np.float32),
            topk=1, sm_scale=1.0, v_dim=1)
        got = o.query_index_scores(inp, 0)
        assert np.array_equal(got, np.array(c["expected"], float)), c["name"]


def pin_indexer_bruteforce(o):
    """Explicit loops over heads, dims and keys on tiny random inputs."""
    rng = np.random.default_rng(7)
    for _ in range(25):
        H_I, d_I, n = rng.integers(1, 5), rng.integers(1, 6), rng.integers(1, 8)
        q = rng.normal(size=(H_I, d_I))
        w = rng.normal(size=H_I)
        keys = rng.normal(size=(n, d_I))
        want = []
        for s in range(n):
            tot = 0.0
            for j in range(H_I):
                dot = 0.0
                for dd in range(d_I):
                    dot += q[j, dd] * keys[s, dd]
                tot += w[j] * (dot if dot > 0.0 else 0.0)
            want.append(tot)
        _close(o.index_scores(q, w, keys), want, 1e-12, "indexer brute force")


def pin_indexer_homogeneity(o):
    """ReLU is positively homogeneous: scaling a key by c > 0 scales its score by c;
    moving a positive factor from a head's query to its weight changes nothing;
    scaling all weights by c > 0 keeps the top-k; the folded fp8 form
    k_scale(s) * sum_j (w_j q_scale_j) ReLU(q8_j . k8_s) equals dequantise-first."""
    rng = np.random.default_rng(8)
    q = rng.normal(size=(4, 6))
    w = rng.uniform(-1, 1, size=4)
    keys = rng.normal(size=(9, 6))
    base = o.index_scores(q, w, keys)
    c = rng.uniform(0.1, 5.0, size=9)
    _close(o.index_scores(q, w, keys * c[:, None]), base * c, 1e-12, "key scaling")
    f = rng.uniform(0.1, 5.0, size=4)
    _close(o.index_scores(q * f[:, None], w / f, keys), base, 1e-12, "query/weight factor")
    wp = np.abs(w)
    sel = o.topk(o.index_scores(q, wp, keys), 4)
    sel2 = o.topk(o.index_scores(q, 3.7 * wp, keys), 4)
    assert np.array_equal(sel, sel2)

    wl = small_workload(mode="decode", num_seqs=2, length=33, H_I=4, d_I=16, index_dtype="fp8")
    oi = to_oracle(generate(wl, "cpu"))
    for t in range(2):
        got = o.query_index_scores(oi, t)
        n = int(oi.q_pos[t]) + 1
        q8 = o.decode_e4m3fn(oi.q_idx[t])
        k8 = o.decode_e4m3fn(oi.k_cache[t, :n])
        ws = oi.w[t].astype(float) * oi.q_scale[t].astype(float)
        folded = oi.k_scale[t, :n].astype(float) * (ws @ np.maximum(q8 @ k8.T, 0.0))
        _close(got, folded, 1e-12, "fp8 folded form")


def pin_indexer_single_head_textbook(o):
    """H_I = 1, w = 1: I = ReLU(q . k); its top-k is a plain stable sort by (-score, position)."""
    rng = np.random.default_rng(9)
    q = rng.normal(size=(1, 5))
    keys = rng.normal(size=(40, 5))
    keys[::7] = -keys[::7]
    I = o.index_scores(q, np.ones(1), keys)
    dots = [float(np.dot(q[0], keys[s])) for s in range(40)]
    _close(I, [max(d, 0.0) for d in dots], 1e-12, "single head")
    want = sorted(range(40), key=lambda s: (-max(dots[s], 0.0), s))[:12]
    assert list(o.topk(I, 12)) == want


# ---------------------------------------------------------------- top-k

def pin_topk_golden(o):
    for c in _golden("topk_hand.json")["cases"]:
        got = list(o.topk(np.array(c["scores"], float), c["k"]))
        assert got == c["expected"], (c, got)
        pad = o.topk_padded(np.array(c["scores"], float), c["k"])
        assert list(pad[: len(c["expected"])]) == c["expected"] and all(pad[len(c["expected"]):] == -1)


def pin_topk_bruteforce(o):
    """Every subset of size min(k, n) for n <= 9: the selection has the largest score
    multiset, and among those the lexicographically smallest position tuple."""
    rng = np.random.default_rng(10)
    for n in range(0, 10):
        for _ in range(4):
            s = rng.integers(-2, 3, size=n).astype(float)
            for k in range(1, n + 2):
                m = min(k, n)
                best = None
                for sub in itertools.combinations(range(n), m):
                    key = (sorted((s[i] for i in sub), reverse=True), [-i for i in sub])
                    if best is None or key > best[0]:
                        best = (key, sub)
                got = o.topk(s, k)
                assert sorted(got.tolist()) == list(best[1]), (s, k, got, best)
                order = [(-s[i], i) for i in got]
                assert order == sorted(order), "selection order"


def certificate(scores, sel, k):
    """The O(n) top-k certificate (no sort): size, uniqueness, range, separation, ties."""
    s = np.asarray(scores, float) + 0.0
    n = s.shape[0]
    sel = np.asarray(sel, dtype=np.int64)
    m = min(k, n)
    assert sel.shape[0] == m, f"selected {sel.shape[0]} != {m}"
    assert np.unique(sel).shape[0] == m, "duplicate selection"
    assert np.all((sel >= 0) & (sel < n)), "selection out of range"
    if m == n:
        return
    mask = np.zeros(n, bool)
    mask[sel] = True
    lo = s[mask].min()
    hi = s[~mask].max()
    assert lo >= hi, f"separation {lo} < {hi}"
    if lo == hi:
        assert np.max(np.nonzero(mask & (s == lo))[0]) < np.min(np.nonzero(~mask & (s == lo))[0]), "tie order"


def pin_topk_certificate(o):
    rng = np.random.default_rng(11)
    for _ in range(40):
        n = int(rng.integers(1, 300))
        s = rng.normal(size=n)
        if rng.random() < 0.5:
            s = np.round(s * 2) / 2                       # many ties
        k = int(rng.integers(1, 320))
        certificate(s, o.topk(s, k), k)


# ---------------------------------------------------------------- sparse MLA (eq. U)

def pin_mla_golden(o):
    for c in _golden("mla_hand.json")["cases"]:
        out, lse = o.sparse_mla(np.array(c["q"], float), np.array(c["rows"], float),
                                c["v_dim"], c["sm_scale"])
        _close(out, c["expected_out"], 1e-14, c["name"])
        _close(lse, c["expected_lse"], 1e-14, c["name"])


def pin_mla_closed_forms(o):
    rng = np.random.default_rng(12)
    H, D, Dv, m = 3, 10, 6, 7
    rows = rng.normal(size=(m, D))
    out, lse = o.sparse_mla(np.zeros((H, D)), rows, Dv, 0.3)            # q = 0: plain mean
    _close(out, np.tile(rows[:, :Dv].mean(axis=0), (H, 1)), 1e-13, "q=0 mean")
    _close(lse, np.full(H, math.log(m)), 1e-13, "q=0 lse")
    same = np.tile(rows[:1], (m, 1))                                    # identical rows
    out, _ = o.sparse_mla(rng.normal(size=(H, D)), same, Dv, 0.3)
    _close(out, np.tile(rows[0, :Dv], (H, 1)), 1e-13, "identical rows")
    qh = rng.normal(size=(H, D))                                        # one row
    out, lse = o.sparse_mla(qh, rows[2:3], Dv, 0.3)
    assert np.array_equal(out, np.tile(rows[2, :Dv], (H, 1)))
    _close(lse, 0.3 * qh @ rows[2], 1e-13, "one-row lse")
    out, lse = o.sparse_mla(qh, rows[:0], Dv, 0.3)                     # empty
    assert np.all(out == 0) and np.all(np.isneginf(lse))
    out, _ = o.sparse_mla(rng.normal(size=(H, D)) * 4, rows, Dv, 1.0)   # convex hull
    lo, hi = rows[:, :Dv].min(axis=0), rows[:, :Dv].max(axis=0)
    assert np.all(out >= lo - 1e-12) and np.all(out <= hi + 1e-12)


def _sdpa(q, rows, Dv, scale, mask):
    """torch float64 SDPA, MQA: every head reads the same rows; mask [n] True = attend."""
    H, D = q.shape
    n = rows.shape[0]
    qt = torch.from_numpy(q).reshape(1, H, 1, D)
    kt = torch.from_numpy(rows).reshape(1, 1, n, D).expand(1, H, n, D)
    vt = torch.from_numpy(np.ascontiguousarray(rows[:, :Dv])).reshape(1, 1, n, Dv).expand(1, H, n, Dv)
    mt = torch.from_numpy(np.asarray(mask, bool)).reshape(1, 1, 1, n)
    out = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mt, scale=scale)
    logits = (qt @ kt.transpose(-1, -2)) * scale
    lse = torch.logsumexp(logits.masked_fill(~mt, -math.inf), dim=-1)
    return out.reshape(H, Dv).numpy(), lse.reshape(H).numpy()


def pin_mla_dense_masked(o):
    """Sparse attention over the chosen rows == dense attention over every candidate
    with a mask equal to the chosen set (baseten (1): the selector acts as a mask)."""
    rng = np.random.default_rng(13)
    for _ in range(10):
        H, D, Dv, n = 4, 12, 8, int(rng.integers(2, 40))
        q = rng.normal(size=(H, D))
        rows = rng.normal(size=(n, D))
        sel = np.sort(rng.choice(n, size=int(rng.integers(1, n + 1)), replace=False))
        mask = np.zeros(n, bool)
        mask[sel] = True
        want_out, want_lse = _sdpa(q, rows, Dv, 0.37, mask)
        out, lse = o.sparse_mla(q, rows[sel], Dv, 0.37)
        _close(out, want_out, 1e-12, "masked dense out")
        _close(lse, want_lse, 1e-12, "masked dense lse")


# ---------------------------------------------------------------- whole path

def pin_forward_dense_causal(o):
    """k >= n: every causal candidate is selected and the path is dense causal MLA
    (short prompts behave like dense attention, zeroshot section 3.4)."""
    wl = small_workload(mode="prefill", length=24, k=32, H=3, D=10, Dv=6)
    oi = to_oracle(generate(wl, "cpu"))
    res = o.forward(oi)
    kv = oi.kv_cache[0].astype(float)
    for t in range(24):
        sel = res["idx"][t]
        assert sorted(sel[sel >= 0].tolist()) == list(range(t + 1)), f"row {t} selection"
        mask = np.arange(24) <= t
        want_out, want_lse = _sdpa(oi.q[t].astype(float), kv, 6, oi.sm_scale, mask)
        _close(res["out"][t], want_out, 1e-12, f"row {t} dense causal")
        _close(res["lse"][t], want_lse, 1e-12, f"row {t} lse")
    # the first query sees only itself
    assert res["idx"][0, 0] == 0 and np.all(res["idx"][0, 1:] == -1)
    assert np.array_equal(res["out"][0], np.tile(kv[0, :6], (3, 1)))


def pin_forward_mask_consistency(o):
    """k < n: the output equals dense attention masked to the oracle's own selection,
    and the selection passes the top-k certificate against the oracle's scores."""
    wl = small_workload(mode="prefill", length=50, k=9, H=2, D=12, Dv=8)
    oi = to_oracle(generate(wl, "cpu"))
    res = o.forward(oi, keep_scores=True)
    kv = oi.kv_cache[0].astype(float)
    for t in range(50):
        sel = res["idx"][t]
        sel = sel[sel >= 0]
        certificate(res["scores"][t], sel, 9)
        mask = np.zeros(50, bool)
        mask[sel] = True
        want_out, _ = _sdpa(oi.q[t].astype(float), kv, 8, oi.sm_scale, mask)
        _close(res["out"][t], want_out, 1e-12, f"row {t}")


def pin_causality_poison(o):
    """Cache slots past each sequence's length hold NaN (generator poison): the oracle
    must never read them, and replacing them by huge values changes nothing."""
    wl = small_workload(mode="decode", num_seqs=3, length=30, k=5)
    inp = generate(wl, "cpu", lengths=[7, 30, 18])
    oi = to_oracle(inp)
    assert np.isnan(oi.kv_cache[0, 7:]).all() and np.isnan(oi.k_cache[2, 18:]).all()
    a = o.forward(oi)
    oi.kv_cache = np.where(np.isnan(oi.kv_cache), np.float32(1e30), oi.kv_cache)
    oi.k_cache = np.where(np.isnan(oi.k_cache), np.float32(1e30), oi.k_cache)
    b = o.forward(oi)
    for key in ("idx", "out", "lse"):
        assert np.array_equal(a[key], b[key]), key
    assert np.all(a["idx"][0][a["idx"][0] >= 0] < 7)


def pin_paged_equals_contiguous(o):
    """The same logical data laid out in permuted 4-token blocks gives identical results."""
    rng = np.random.default_rng(14)
    wl = small_workload(mode="decode", num_seqs=3, length=29, k=6)
    oi = to_oracle(generate(wl, "cpu", lengths=[29, 13, 21]))
    a = o.forward(oi)
    bs = 4
    B, L = oi.kv_cache.shape[:2]
    nb = (L + bs - 1) // bs
    perm = rng.permutation(B * nb)
    table = perm.reshape(B, nb)
    kc = np.full((B * nb, bs) + oi.k_cache.shape[2:], np.nan, oi.k_cache.dtype)
    vc = np.full((B * nb, bs) + oi.kv_cache.shape[2:], np.nan, oi.kv_cache.dtype)
    for b in range(B):
        for s in range(L):
            kc[table[b, s // bs], s % bs] = oi.k_cache[b, s]
            vc[table[b, s // bs], s % bs] = oi.kv_cache[b, s]
    oi.block_table, oi.block_size, oi.k_cache, oi.kv_cache = table, bs, kc, vc
    b_ = o.forward(oi)
    for key in ("idx", "out", "lse"):
        assert np.array_equal(a[key], b_[key]), key


def pin_paged_fp8_equals_contiguous(o):
    """An e4m3fn indexer's key codes *and* their per-token fp32 scales re-laid into
    permuted 4-token blocks give identical scores, selections, outputs and lse.
    The scales are first spread over [1/4, 4] per token, so a scale read from the
    wrong slot, or not read, changes the scores."""
    rng = np.random.default_rng(16)
    wl = small_workload(mode="decode", num_seqs=3, length=37, k=5, index_dtype="fp8")
    oi = to_oracle(generate(wl, "cpu", lengths=[37, 11, 26]))
    assert oi.index_dtype == "fp8" and oi.k_scale is not None
    oi.k_scale = (oi.k_scale * rng.uniform(0.25, 4.0, oi.k_scale.shape)).astype(np.float32)
    a = o.forward(oi, keep_scores=True)
    bs = 4
    B, L = oi.kv_cache.shape[:2]
    nb = (L + bs - 1) // bs
    table = rng.permutation(B * nb).reshape(B, nb)
    kc = np.full((B * nb, bs) + oi.k_cache.shape[2:], 0x7F, oi.k_cache.dtype)     # e4m3fn NaN codes
    ks = np.full((B * nb, bs), np.nan, np.float32)
    vc = np.full((B * nb, bs) + oi.kv_cache.shape[2:], np.nan, oi.kv_cache.dtype)
    for b in range(B):
        for s in range(L):
            kc[table[b, s // bs], s % bs] = oi.k_cache[b, s]
            ks[table[b, s // bs], s % bs] = oi.k_scale[b, s]
            vc[table[b, s // bs], s % bs] = oi.kv_cache[b, s]
    oi.block_table, oi.block_size, oi.k_cache, oi.k_scale, oi.kv_cache = table, bs, kc, ks, vc
    b_ = o.forward(oi, keep_scores=True)
    for key in ("idx", "out", "lse"):
        assert np.array_equal(a[key], b_[key]), key
    for t in range(3):
        assert np.array_equal(a["scores"][t], b_["scores"][t]), f"scores of query {t}"


def pin_prefill_row_equals_decode(o):
    """Prefill row t equals a decode step whose context is the first t+1 tokens."""
    wl = small_workload(mode="prefill", length=30, k=7)
    oi = to_oracle(generate(wl, "cpu"))
    a = o.forward(oi)
    for t in (0, 6, 7, 8, 29):
        d = o.OracleInputs(
            mode="decode", q_pos=np.array([t]), block_table=None, block_size=oi.block_size,
            index_dtype=oi.index_dtype, q_idx=oi.q_idx[t:t + 1], q_scale=None, w=oi.w[t:t + 1],
            k_cache=oi.k_cache[:, : t + 1], k_scale=None, mla_dtype=oi.mla_dtype, q=oi.q[t:t + 1],
            kv_cache=oi.kv_cache[:, : t + 1], topk=oi.topk, sm_scale=oi.sm_scale, v_dim=oi.v_dim)
        b = o.forward(d)
        for key in ("idx", "out", "lse"):
            assert np.array_equal(a[key][t], b[key][0]), (t, key)


def pin_permutation_invariance(o):
    """Permuting a decode context (keys and latents together) permutes the selected
    positions and leaves the attention output unchanged."""
    rng = np.random.default_rng(15)
    wl = small_workload(mode="decode", num_seqs=1, length=31, k=8)
    oi = to_oracle(generate(wl, "cpu"))
    a = o.forward(oi)
    perm = rng.permutation(31)
    kc = np.empty_like(oi.k_cache)
    vc = np.empty_like(oi.kv_cache)
    kc[0, perm] = oi.k_cache[0]
    vc[0, perm] = oi.kv_cache[0]
    oi.k_cache, oi.kv_cache = kc, vc
    b = o.forward(oi)
    assert sorted(perm[a["idx"][0]].tolist()) == sorted(b["idx"][0].tolist())
    _close(a["out"], b["out"], 1e-12, "permuted out")
    _close(a["lse"], b["lse"], 1e-12, "permuted lse")


# ---------------------------------------------------------------- dense MLA

def pin_dense_causal_sdpa(o):
    """Dense MLA of a prefill equals torch's causal SDPA (diagonal included, the
    library's own mask) over the whole [T, T] problem, lse included."""
    T, H, D, Dv = 37, 3, 10, 6
    wl = small_workload(mode="prefill", length=T, k=4, H=H, D=D, Dv=Dv)
    oi = to_oracle(generate(wl, "cpu"))
    res = o.dense_forward(oi)
    kv = torch.from_numpy(oi.kv_cache[0, :T].astype(np.float64))
    q = torch.from_numpy(oi.q.astype(np.float64)).permute(1, 0, 2).reshape(1, H, T, D)
    k = kv.reshape(1, 1, T, D).expand(1, H, T, D)
    v = kv[:, :Dv].contiguous().reshape(1, 1, T, Dv).expand(1, H, T, Dv)
    want = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=True, scale=oi.sm_scale)
    _close(res["out"], want.reshape(H, T, Dv).permute(1, 0, 2).numpy(), 1e-12, "dense causal out")
    logits = (q @ k.transpose(-1, -2)) * oi.sm_scale
    causal = torch.ones(T, T, dtype=torch.bool).tril()
    want_lse = torch.logsumexp(logits.masked_fill(~causal, -math.inf), dim=-1)
    _close(res["lse"], want_lse.reshape(H, T).T.numpy(), 1e-12, "dense causal lse")


def pin_dense_ragged_paged(o):
    """Dense decode over ragged, paged contexts equals SDPA over each sequence's
    first n_t tokens, taken from a contiguous copy of the same data; slots past
    a sequence's length (NaN poison) are never read."""
    rng = np.random.default_rng(16)
    wl = small_workload(mode="decode", num_seqs=3, length=30, k=5, H=2, D=12, Dv=8)
    oi = to_oracle(generate(wl, "cpu", lengths=[7, 30, 18]))
    contiguous = oi.kv_cache.copy()
    bs = 4
    B, L = oi.kv_cache.shape[:2]
    nb = (L + bs - 1) // bs
    table = rng.permutation(B * nb).reshape(B, nb)
    vc = np.full((B * nb, bs) + oi.kv_cache.shape[2:], np.nan, oi.kv_cache.dtype)
    for b in range(B):
        for s in range(L):
            vc[table[b, s // bs], s % bs] = oi.kv_cache[b, s]
    oi.block_table, oi.block_size, oi.kv_cache = table, bs, vc
    res = o.dense_forward(oi)
    for t in range(3):
        n = int(oi.q_pos[t]) + 1
        want_out, want_lse = _sdpa(oi.q[t].astype(float), contiguous[t, :n].astype(float), 8, oi.sm_scale,
                                   np.ones(n, bool))
        _close(res["out"][t], want_out, 1e-12, f"query {t} out")
        _close(res["lse"][t], want_lse, 1e-12, f"query {t} lse")


def pin_dense_equals_short_prompt_dsa(o):
    """With k >= every n_t the DSA path selects every candidate, so its result is
    the dense one (short prompts, zeroshot section 3.4)."""
    wl = small_workload(mode="decode", num_seqs=4, length=20, k=32)
    oi = to_oracle(generate(wl, "cpu", lengths=[1, 9, 20, 14]))
    a = o.forward(oi)
    d = o.dense_forward(oi)
    _close(a["out"], d["out"], 1e-12, "short-prompt out")
    _close(a["lse"], d["lse"], 1e-12, "short-prompt lse")


# ---------------------------------------------------------------- indexer warm-up loss

def pin_attention_distribution_torch(o):
    """p_t equals the head mean of torch's float64 softmax over each query's causal
    candidates (ragged paged decode, NaN poison past each length), and sums to 1."""
    wl = small_workload(mode="decode", num_seqs=3, length=30, k=5, H=3, D=12, Dv=8)
    oi = to_oracle(generate(wl, "cpu", lengths=[7, 30, 18]))
    for t in range(3):
        n = int(oi.q_pos[t]) + 1
        q = torch.from_numpy(oi.q[t].astype(np.float64))
        kv = torch.from_numpy(oi.kv_cache[t, :n].astype(np.float64))
        want = torch.softmax(oi.sm_scale * (q @ kv.T), dim=-1).mean(dim=0).numpy()
        got = o.attention_distribution(oi, t)
        _close(got, want, 1e-12, f"query {t} distribution")
        assert abs(got.sum() - 1.0) < 1e-12


def pin_kl_rows_torch(o):
    """kl_rows equals torch's kl_div(log_softmax(I), p, sum) and its gradient equals
    torch autograd's, zeros in p included."""
    rng = np.random.default_rng(21)
    for n in (1, 2, 9, 40):
        I = rng.normal(size=n) * 3
        p = rng.random(n) ** 3
        p[rng.random(n) < 0.3] = 0.0
        if p.sum() == 0:
            p[0] = 1.0
        p /= p.sum()
        It = torch.tensor(I, dtype=torch.float64, requires_grad=True)
        lt = torch.nn.functional.kl_div(torch.log_softmax(It, dim=0), torch.tensor(p), reduction="sum")
        lt.backward()
        loss, g = o.kl_rows(I, p)
        _close(loss, lt.item(), 1e-12, f"n={n} loss")
        _close(g, It.grad.numpy(), 1e-12, f"n={n} grad")


def pin_kl_rows_zero_at_match(o):
    """I = log p + c (any c) is a perfect match: loss 0 and gradient 0."""
    rng = np.random.default_rng(22)
    p = rng.random(12)
    p /= p.sum()
    for c in (0.0, 5.0, -40.0):
        loss, g = o.kl_rows(np.log(p) + c, p)
        assert abs(loss) < 1e-12 and np.max(np.abs(g)) < 1e-12, c


def pin_index_scores_backward_autograd(o):
    """dq, dw, dk of eq. I equal torch autograd of sum_s g_s I_s (float64, mixed-sign
    weights)."""
    rng = np.random.default_rng(23)
    for H_I, d_I, n in ((1, 3, 4), (3, 5, 7), (4, 8, 33)):
        q = rng.normal(size=(H_I, d_I))
        w = rng.normal(size=H_I)
        k = rng.normal(size=(n, d_I))
        g = rng.normal(size=n)
        qt, wt, kt = (torch.tensor(x, requires_grad=True) for x in (q, w, k))
        I = (wt[:, None] * torch.relu(qt @ kt.T)).sum(dim=0)
        (I * torch.tensor(g)).sum().backward()
        dq, dw, dk = o.index_scores_backward(q, w, k, g)
        _close(dq, qt.grad.numpy(), 1e-12, "dq")
        _close(dw, wt.grad.numpy(), 1e-12, "dw")
        _close(dk, kt.grad.numpy(), 1e-12, "dk")


def _kl_workload():
    wl = small_workload(mode="prefill", length=14, k=4, H_I=3, d_I=8, H=2, D=12, Dv=8, w_high=1.0)
    return to_oracle(generate(wl, "cpu"))


def pin_indexer_kl_loss_finite_differences(o):
    """Central differences of the summed loss (inputs moved by 2^-10, exact in
    float32) match the analytic gradients into w, q_I and k_I; q/k entries are
    used only where no q.k term lies within reach of the ReLU kink."""
    oi = _kl_workload()
    res = o.indexer_kl_loss(oi)
    h = 2.0 ** -10

    def total(field, idx, delta):
        arr = getattr(oi, field)
        old = arr[idx]
        arr[idx] = np.float32(old + delta)
        try:
            return float(o.indexer_kl_loss(oi)["loss"].sum())
        finally:
            arr[idx] = old

    def fd(field, idx):
        return (total(field, idx, h) - total(field, idx, -h)) / (2 * h)

    rng = np.random.default_rng(24)
    for _ in range(6):                                     # w: eq. I is linear in w
        t, j = int(rng.integers(0, 14)), int(rng.integers(0, 3))
        _close(fd("w", (t, j)), res["dw"][t, j], 1e-5, f"dw[{t},{j}]")
    q = oi.q_idx.astype(np.float64)
    k = oi.k_cache[0].astype(np.float64)
    checked = 0
    for t in range(3, 14):
        for j in range(3):
            x = q[t, j] @ k[: t + 1].T
            if np.min(np.abs(x)) < 0.05:
                continue
            d = int(rng.integers(0, 8))
            _close(fd("q_idx", (t, j, d)), res["dq"][t, j, d], 1e-5, f"dq[{t},{j},{d}]")
            checked += 1
            break
    assert checked >= 4
    checked = 0
    for s in range(14):
        x = q[s:, :, :] @ k[s]
        if np.min(np.abs(x)) < 0.05:
            continue
        d = int(rng.integers(0, 8))
        _close(fd("k_cache", (0, s, d)), res["dk"][0, s, d], 1e-5, f"dk[{s},{d}]")
        checked += 1
    assert checked >= 4


def pin_indexer_kl_loss_autograd(o):
    """The whole objective against torch autograd in float64: p from torch's softmax
    over the latent rows, the loss from torch's kl_div, gradients by autograd."""
    oi = _kl_workload()
    res = o.indexer_kl_loss(oi)
    T = oi.num_q
    q = torch.tensor(oi.q_idx.astype(np.float64), requires_grad=True)
    w = torch.tensor(oi.w.astype(np.float64), requires_grad=True)
    k = torch.tensor(oi.k_cache[0].astype(np.float64), requires_grad=True)
    qm = torch.tensor(oi.q.astype(np.float64))
    kv = torch.tensor(oi.kv_cache[0].astype(np.float64))
    total = 0.0
    for t in range(T):
        n = t + 1
        p = torch.softmax(oi.sm_scale * (qm[t] @ kv[:n].T), dim=-1).mean(dim=0)
        I = (w[t][:, None] * torch.relu(q[t] @ k[:n].T)).sum(dim=0)
        lt = torch.nn.functional.kl_div(torch.log_softmax(I, dim=0), p, reduction="sum")
        _close(res["loss"][t], lt.item(), 1e-12, f"loss[{t}]")
        total = total + lt
    total.backward()
    _close(res["dq"], q.grad.numpy(), 1e-11, "dq")
    _close(res["dw"], w.grad.numpy(), 1e-11, "dw")
    _close(res["dk"][0, :T], k.grad.numpy(), 1e-11, "dk")


def pin_indexer_kl_paged_poison(o):
    """Ragged paged decode with NaN poison past each length: finite results, and the
    key gradients land only in slots the block table names for valid positions."""
    rng = np.random.default_rng(25)
    wl = small_workload(mode="decode", num_seqs=3, length=29, k=6)
    oi = to_oracle(generate(wl, "cpu", lengths=[29, 13, 21]))
    ref = o.indexer_kl_loss(oi)
    bs = 4
    B, L = oi.kv_cache.shape[:2]
    nb = (L + bs - 1) // bs
    table = rng.permutation(B * nb).reshape(B, nb)
    kc = np.full((B * nb, bs) + oi.k_cache.shape[2:], np.nan, oi.k_cache.dtype)
    vc = np.full((B * nb, bs) + oi.kv_cache.shape[2:], np.nan, oi.kv_cache.dtype)
    for b in range(B):
        for s in range(L):
            kc[table[b, s // bs], s % bs] = oi.k_cache[b, s]
            vc[table[b, s // bs], s % bs] = oi.kv_cache[b, s]
    oi.block_table, oi.block_size, oi.k_cache, oi.kv_cache = table, bs, kc, vc
    res = o.indexer_kl_loss(oi)
    for key in ("loss", "dq", "dw"):
        assert np.all(np.isfinite(res[key])), key
        _close(res[key], ref[key], 1e-12, key)
    for b, n in enumerate((29, 13, 21)):
        for s in range(L):
            got = res["dk"][table[b, s // bs], s % bs]
            if s < n:
                _close(got, ref["dk"][b, s], 1e-12, f"dk seq {b} pos {s}")
            else:
                assert np.all(got == 0), f"dk written past the length: seq {b} pos {s}"


# ---------------------------------------------------------------- fp8 quantisation and append

def pin_e4m3_encode_roundtrip(o):
    """Every finite e4m3fn value encodes back to its own code (signed zeros included)."""
    codes = np.arange(256, dtype=np.uint8)
    vals = o.decode_e4m3fn(codes)
    fin = np.isfinite(vals)
    assert np.array_equal(o.encode_e4m3fn(vals[fin]), codes[fin]), "round trip"


def pin_e4m3_encode_midpoints(o):
    """Halfway between neighbouring codes the even code wins; just off the midpoint the nearer one."""
    for c in range(0, 0x7E):
        a, b = float(o.decode_e4m3fn(c)), float(o.decode_e4m3fn(c + 1))
        mid = (a + b) / 2.0
        even = c if c % 2 == 0 else c + 1
        for sign, bit in ((1.0, 0), (-1.0, 0x80)):
            got = o.encode_e4m3fn(np.array([sign * mid]))[0]
            assert got == (even | bit), f"midpoint of codes {c:#x},{c + 1:#x}"
            lo = o.encode_e4m3fn(np.array([sign * np.nextafter(mid, a)]))[0]
            hi = o.encode_e4m3fn(np.array([sign * np.nextafter(mid, b)]))[0]
            assert lo == (c | bit) and hi == ((c + 1) | bit), f"near the midpoint of {c:#x}"


def pin_e4m3_encode_torch(o):
    """Random float32 values in [-448, 448] (all binades) against torch's float8_e4m3fn cast."""
    rng = np.random.default_rng(17)
    mag = np.exp2(rng.uniform(-12.0, np.log2(448.0), 200000)).astype(np.float32)
    y = np.where(rng.random(mag.shape) < 0.5, -mag, mag).astype(np.float32)
    ref = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(o.encode_e4m3fn(y), ref), "encoder vs torch cast"


def pin_quantize_golden(o):
    """Hand-derived rows (tests/golden/quantize_hand.json)."""
    g = _golden("quantize_hand.json")
    for case in g["cases"]:
        codes, scale = o.quantize_fp8(np.array([case["x"]], dtype=np.float32))
        assert codes[0].tolist() == case["codes"], case["name"]
        assert float(scale[0]) == case["scale"], case["name"]


def pin_quantize_bounds(o):
    """Per row: the largest magnitude maps to +-448, and dequantisation errs by at most half
    the spacing of e4m3fn values around the code (times the scale)."""
    rng = np.random.default_rng(23)
    x = (rng.standard_normal((64, 128)) * np.exp2(rng.uniform(-20, 20, (64, 1)))).astype(np.float32)
    codes, scale = o.quantize_fp8(x)
    vals = o.decode_e4m3fn(codes)
    assert np.all(np.max(np.abs(vals), axis=1) == 448.0)
    mags = o.decode_e4m3fn(np.arange(0x7F, dtype=np.uint8))
    y = x.astype(np.float64) / scale.astype(np.float64)[:, None]
    # spacing of e4m3fn values on the side of the code where y lies
    idx = np.searchsorted(mags, np.abs(vals))
    up = np.abs(y) > np.abs(vals)
    spacing = np.where(up, mags[np.minimum(idx + 1, 0x7E)] - mags[idx], mags[idx] - mags[np.maximum(idx - 1, 0)])
    # the quotient itself is a float32: allow its own rounding on top of the half spacing
    assert np.all(np.abs(vals - y) <= spacing / 2 + np.abs(y) * 2.0 ** -23), "rounding error bound"


def pin_append_index_keys(o):
    """Appending into a paged cache writes exactly the slots the block table names."""
    bs, d = 4, 8
    table = np.array([[2, 0, -1], [1, 3, 5]], dtype=np.int64)     # sequence 0: blocks 2, 0; sequence 1: 1, 3, 5
    cache = np.full((6, bs, d), 0x11, dtype=np.uint8)
    scale = np.full((6, bs), 7.0, dtype=np.float32)
    rng = np.random.default_rng(5)
    k_new = rng.standard_normal((2, d)).astype(np.float32)
    # decode: token 0 -> sequence 0 at position 5 (block 0, offset 1); token 1 -> sequence 1 at position 10
    # (table entry 2 = block 5, outside the 6-block pool? no: block 5 exists, offset 2)
    c2, s2 = o.append_index_keys("decode", [5, 10], table, bs, k_new, cache, scale)
    codes, sc = o.quantize_fp8(k_new)
    changed = np.argwhere(np.any(c2 != cache, axis=2) | (s2 != scale))
    assert sorted(map(tuple, changed.tolist())) == [(0, 1), (5, 2)], changed
    assert np.array_equal(c2[0, 1], codes[0]) and s2[0, 1] == sc[0]
    assert np.array_equal(c2[5, 2], codes[1]) and s2[5, 2] == sc[1]
    # a negative position and an absent block are skipped
    c3, s3 = o.append_index_keys("decode", [-1, 9], np.array([[2, 0, -1], [1, 3, -1]]), bs, k_new, cache, scale)
    assert np.array_equal(c3, cache) and np.array_equal(s3, scale)
    # contiguous cache [B, Lmax, d]: prefill tokens all belong to sequence 0
    cc = np.zeros((1, 6, d), dtype=np.uint8)
    cs = np.ones((1, 6), dtype=np.float32)
    c4, s4 = o.append_index_keys("prefill", [0, 3], None, bs, k_new, cc, cs)
    assert np.array_equal(c4[0, 0], codes[0]) and np.array_equal(c4[0, 3], codes[1])
    assert np.all(c4[0, [1, 2, 4, 5]] == 0) and s4[0, 3] == sc[1]




# ---------------------------------------------------------------- Stage 2: sparse training

def _mla_torch(q, rows, Dv, scale):
    """eq. U's attention written in torch ops (float64): K is the whole row, V its
    first Dv entries, both taken from the one leaf tensor `rows`."""
    p = torch.softmax(scale * (q @ rows.T), dim=-1)
    return p @ rows[:, :Dv]


def pin_sparse_mla_backward_autograd(o):
    """dq and the row gradients equal torch autograd of eq. U's attention (float64),
    key and value parts of a row summed because they are one leaf."""
    rng = np.random.default_rng(31)
    for H, D, Dv, m in ((1, 4, 3, 1), (2, 6, 4, 3), (3, 12, 8, 17), (4, 10, 10, 9)):
        q = rng.normal(size=(H, D))
        rows = rng.normal(size=(m, D))
        dout = rng.normal(size=(H, Dv))
        qt, rt = torch.tensor(q, requires_grad=True), torch.tensor(rows, requires_grad=True)
        (_mla_torch(qt, rt, Dv, 0.41) * torch.tensor(dout)).sum().backward()
        dq, dr = o.sparse_mla_backward(q, rows, Dv, 0.41, dout)
        _close(dq, qt.grad.numpy(), 1e-12, f"dq m={m}")
        _close(dr, rt.grad.numpy(), 1e-12, f"drows m={m}")
    # one selected row: the softmax is constant, so dq = 0 and the row gets dout
    q, rows, dout = rng.normal(size=(3, 6)), rng.normal(size=(1, 6)), rng.normal(size=(3, 4))
    dq, dr = o.sparse_mla_backward(q, rows, 4, 0.3, dout)
    assert np.all(np.abs(dq) < 1e-15)
    _close(dr[0, :4], dout.sum(axis=0), 1e-12, "single row value gradient")
    assert np.all(np.abs(dr[0, 4:]) < 1e-15)
    dq, dr = o.sparse_mla_backward(q, rows[:0], 4, 0.3, dout)       # empty selection
    assert dq.shape == (3, 6) and np.all(dq == 0) and dr.shape == (0, 6)


def pin_sparse_mla_backward_finite_differences(o):
    """Central differences (float64, h = 1e-6) of sum(dout * out) in q and in the
    selected rows match the analytic gradients."""
    rng = np.random.default_rng(32)
    H, D, Dv, m = 3, 7, 5, 6
    q, rows, dout = rng.normal(size=(H, D)), rng.normal(size=(m, D)), rng.normal(size=(H, Dv))
    f = lambda qq, rr: float(np.sum(dout * o.sparse_mla(qq, rr, Dv, 0.5)[0]))
    dq, dr = o.sparse_mla_backward(q, rows, Dv, 0.5, dout)
    h = 1e-6
    for _ in range(8):
        i, j = int(rng.integers(0, H)), int(rng.integers(0, D))
        qp, qm = q.copy(), q.copy()
        qp[i, j] += h
        qm[i, j] -= h
        _close((f(qp, rows) - f(qm, rows)) / (2 * h), dq[i, j], 1e-7, f"dq[{i},{j}]")
        i, j = int(rng.integers(0, m)), int(rng.integers(0, D))
        rp, rm = rows.copy(), rows.copy()
        rp[i, j] += h
        rm[i, j] -= h
        _close((f(q, rp) - f(q, rm)) / (2 * h), dr[i, j], 1e-7, f"drows[{i},{j}]")


def pin_sparse_backward_equals_masked_dense(o):
    """The sparse backward equals torch SDPA's backward over every candidate with a
    mask equal to the chosen set (float64): the same dq, the chosen rows' gradients,
    and zero gradient on every row outside the set."""
    rng = np.random.default_rng(33)
    for _ in range(6):
        H, D, Dv, n = 3, 12, 8, int(rng.integers(2, 30))
        q, rows, dout = rng.normal(size=(H, D)), rng.normal(size=(n, D)), rng.normal(size=(H, Dv))
        sel = np.sort(rng.choice(n, size=int(rng.integers(1, n + 1)), replace=False))
        mask = np.zeros(n, bool)
        mask[sel] = True
        qt = torch.tensor(q, requires_grad=True)
        rt = torch.tensor(rows, requires_grad=True)
        kt = rt.reshape(1, 1, n, D).expand(1, H, n, D)
        vt = rt[:, :Dv].reshape(1, 1, n, Dv).expand(1, H, n, Dv)
        out = torch.nn.functional.scaled_dot_product_attention(qt.reshape(1, H, 1, D), kt, vt,
                                                               attn_mask=torch.tensor(mask).reshape(1, 1, 1, n),
                                                               scale=0.29)
        (out.reshape(H, Dv) * torch.tensor(dout)).sum().backward()
        dq, dr = o.sparse_mla_backward(q, rows[sel], Dv, 0.29, dout)
        _close(dq, qt.grad.numpy(), 1e-12, "masked dense dq")
        _close(dr, rt.grad.numpy()[sel], 1e-12, "masked dense drows")
        assert np.all(np.abs(rt.grad.numpy()[~mask]) < 1e-15)


def pin_sparse_attention_backward_dense_causal(o):
    """With every candidate selected (k >= n) the Stage-2 attention gradient of a whole
    prefill equals torch's causal SDPA backward (float64): dq per query, and the
    cache-row gradients summed over all the queries that read each row."""
    wl = small_workload(mode="prefill", length=21, k=32, H=3, D=10, Dv=6)
    oi = to_oracle(generate(wl, "cpu"))
    T = oi.num_q
    idx = np.full((T, 32), -1)
    for t in range(T):
        idx[t, : t + 1] = np.arange(t + 1)
    dout = np.random.default_rng(34).normal(size=(T, 3, 6))
    res = o.sparse_attention_backward(oi, idx, dout)
    qt = torch.tensor(oi.q.astype(np.float64), requires_grad=True)           # [T, H, D]
    ct = torch.tensor(oi.kv_cache[0].astype(np.float64), requires_grad=True)  # [T, D]
    out = torch.nn.functional.scaled_dot_product_attention(
        qt.permute(1, 0, 2).unsqueeze(0), ct.reshape(1, 1, T, 10).expand(1, 3, T, 10),
        ct[:, :6].reshape(1, 1, T, 6).expand(1, 3, T, 6), is_causal=True, scale=oi.sm_scale)
    (out[0].permute(1, 0, 2) * torch.tensor(dout)).sum().backward()
    _close(res["dq"], qt.grad.numpy(), 1e-12, "causal dq")
    _close(res["dkv"][0, :T], ct.grad.numpy(), 1e-12, "causal dkv")


def pin_sparse_attention_backward_paged(o):
    """Paged caches (permuted 4-token blocks, NaN poison elsewhere) give the same dq,
    and each row gradient lands in the slot the block table names; slots of rows no
    query selected hold 0."""
    rng = np.random.default_rng(35)
    wl = small_workload(mode="decode", num_seqs=3, length=23, k=6)
    oi = to_oracle(generate(wl, "cpu", lengths=[23, 9, 16]))
    res = o.forward(oi)
    dout = rng.normal(size=(3, oi.q.shape[1], oi.v_dim))
    a = o.sparse_attention_backward(oi, res["idx"], dout)
    bs = 4
    B, L = oi.kv_cache.shape[:2]
    nb = (L + bs - 1) // bs
    table = rng.permutation(B * nb).reshape(B, nb)
    vc = np.full((B * nb, bs) + oi.kv_cache.shape[2:], np.nan, oi.kv_cache.dtype)
    for b in range(B):
        for s in range(L):
            vc[table[b, s // bs], s % bs] = oi.kv_cache[b, s]
    oi.block_table, oi.block_size, oi.kv_cache = table, bs, vc
    b_ = o.sparse_attention_backward(oi, res["idx"], dout)
    _close(b_["dq"], a["dq"], 1e-15, "paged dq")
    for b in range(B):
        for s in range(L):
            _close(b_["dkv"][table[b, s // bs], s % bs], a["dkv"][b, s], 1e-15, f"dkv seq {b} pos {s}")
    sel0 = set(res["idx"][0][res["idx"][0] >= 0].tolist())
    for s in range(23):
        if s not in sel0:
            assert np.all(a["dkv"][0, s] == 0), f"unselected row {s}"


def pin_sparse_distribution_torch(o):
    """The Stage-2 target is the head mean of torch's softmax over the selected rows;
    with every candidate selected it is the Stage-1 target."""
    wl = small_workload(mode="decode", num_seqs=2, length=30, k=5, H=3, D=12, Dv=8)
    oi = to_oracle(generate(wl, "cpu", lengths=[30, 17]))
    rng = np.random.default_rng(36)
    for t in range(2):
        n = int(oi.q_pos[t]) + 1
        sel = np.sort(rng.choice(n, size=7, replace=False))
        q = torch.from_numpy(oi.q[t].astype(np.float64))
        kv = torch.from_numpy(oi.kv_cache[t, sel].astype(np.float64))
        want = torch.softmax(oi.sm_scale * (q @ kv.T), dim=-1).mean(dim=0).numpy()
        _close(o.sparse_attention_distribution(oi, t, sel), want, 1e-12, f"query {t}")
        _close(o.sparse_attention_distribution(oi, t, np.arange(n)), o.attention_distribution(oi, t), 1e-12,
               f"query {t} full set")


def _stage2_workload():
    wl = small_workload(mode="prefill", length=16, k=5, H_I=3, d_I=8, H=2, D=12, Dv=8, w_high=1.0, w_low=-0.5)
    return to_oracle(generate(wl, "cpu"))


def pin_sparse_indexer_kl_autograd(o):
    """Stage 2's indexer objective against torch in float64: the selection from
    torch's stable descending sort, the target from torch's softmax over the selected
    latent rows, the loss from kl_div over the selection, gradients by autograd (mixed-
    sign weights)."""
    oi = _stage2_workload()
    res = o.sparse_indexer_kl_loss(oi)
    T, k = oi.num_q, oi.topk
    q = torch.tensor(oi.q_idx.astype(np.float64), requires_grad=True)
    w = torch.tensor(oi.w.astype(np.float64), requires_grad=True)
    kk = torch.tensor(oi.k_cache[0].astype(np.float64), requires_grad=True)
    qm = torch.tensor(oi.q.astype(np.float64))
    kv = torch.tensor(oi.kv_cache[0].astype(np.float64))
    total = 0.0
    for t in range(T):
        n = t + 1
        I = (w[t][:, None] * torch.relu(q[t] @ kk[:n].T)).sum(dim=0)
        sel = torch.sort(-I.detach(), stable=True).indices[: min(k, n)]
        assert sorted(sel.tolist()) == sorted(res["idx"][t][res["idx"][t] >= 0].tolist()), f"selection {t}"
        p = torch.softmax(oi.sm_scale * (qm[t] @ kv[sel].T), dim=-1).mean(dim=0)
        lt = torch.nn.functional.kl_div(torch.log_softmax(I[sel], dim=0), p, reduction="sum")
        _close(res["loss"][t], lt.item(), 1e-12, f"loss[{t}]")
        total = total + lt
    total.backward()
    _close(res["dq"], q.grad.numpy(), 1e-11, "dq")
    _close(res["dw"], w.grad.numpy(), 1e-11, "dw")
    _close(res["dk"][0, :T], kk.grad.numpy(), 1e-11, "dk")
    for t in range(T):                                   # no gradient outside the selection
        g = res["grad_scores"][t]
        off = np.ones(g.shape[0], bool)
        off[res["idx"][t][res["idx"][t] >= 0]] = False
        assert np.all(g[off] == 0), f"gradient outside S_{t}"


def pin_sparse_indexer_kl_full_selection(o):
    """k >= n: the selection is every candidate, and Stage 2's indexer objective is
    the Stage-1 warm-up objective (loss and every gradient)."""
    oi = _stage2_workload()
    oi.topk = 64
    a = o.sparse_indexer_kl_loss(oi)
    b = o.indexer_kl_loss(oi)
    for key in ("loss", "dq", "dw", "dk"):
        _close(a[key], b[key], 1e-12, key)


def pin_sparse_indexer_kl_finite_differences(o):
    """With the selections held fixed, central differences (2^-10, exact in float32)
    of the summed loss in w and in q_I (away from the ReLU kink) match the gradients."""
    oi = _stage2_workload()
    res = o.sparse_indexer_kl_loss(oi)
    sels = res["idx"]
    h = 2.0 ** -10

    def total(field, idx, delta):
        arr = getattr(oi, field)
        old = arr[idx]
        arr[idx] = np.float32(old + delta)
        try:
            return float(o.sparse_indexer_kl_loss(oi, selections=sels)["loss"].sum())
        finally:
            arr[idx] = old

    fd = lambda field, idx: (total(field, idx, h) - total(field, idx, -h)) / (2 * h)
    rng = np.random.default_rng(37)
    for _ in range(6):
        t, j = int(rng.integers(6, 16)), int(rng.integers(0, 3))
        _close(fd("w", (t, j)), res["dw"][t, j], 1e-5, f"dw[{t},{j}]")
    q = oi.q_idx.astype(np.float64)
    k = oi.k_cache[0].astype(np.float64)
    checked = 0
    for t in range(6, 16):
        for j in range(3):
            if np.min(np.abs(q[t, j] @ k[: t + 1].T)) < 0.05:
                continue
            d = int(rng.integers(0, 8))
            _close(fd("q_idx", (t, j, d)), res["dq"][t, j, d], 1e-5, f"dq[{t},{j},{d}]")
            checked += 1
            break
    assert checked >= 4


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
