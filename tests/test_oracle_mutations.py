"""Plants plausible mistakes in the oracle (on the CPU) and requires the pins to catch each.

A mutation replaces one function or table of the oracle module; the pins run
against the mutated module and at least one must fail."""
import math

import numpy as np
import pytest

import oracle.dsa_oracle as od
from tests import pins


def _no_relu(q, w, keys):
    return w @ (q @ keys.T)


def _relu_after_weight(q, w, keys):
    return np.maximum(w[:, None] * (q @ keys.T), 0.0).sum(axis=0)


def _no_weight(q, w, keys):
    return np.maximum(q @ keys.T, 0.0).sum(axis=0)


def _key_index_swapped(q, w, keys):
    return w @ np.maximum(q @ keys[::-1].T, 0.0)


def _ties_high(scores, k):
    s = np.asarray(scores, float) + 0.0
    n = s.shape[0]
    order = n - 1 - np.argsort(-s[::-1], kind="stable")
    return order[: min(k, n)].astype(np.int64)


def _k_minus_one(scores, k):
    s = np.asarray(scores, float) + 0.0
    return np.argsort(-s, kind="stable")[: max(min(k, s.shape[0]) - 1, 0)].astype(np.int64)


def _smallest(scores, k):
    s = np.asarray(scores, float) + 0.0
    return np.argsort(s, kind="stable")[: min(k, s.shape[0])].astype(np.int64)


def _mla_value_tail(q, rows, v_dim, sm):
    r = rows.copy()
    r[:, :v_dim] = rows[:, rows.shape[1] - v_dim:]
    return od.__dict__["_orig_sparse_mla"](q, r, v_dim, sm)


def _mla_no_rope(q, rows, v_dim, sm):
    q2 = q.copy()
    q2[:, v_dim:] = 0.0
    return od.__dict__["_orig_sparse_mla"](q2, rows, v_dim, sm)


def _mla_no_scale(q, rows, v_dim, sm):
    return od.__dict__["_orig_sparse_mla"](q, rows, v_dim, 1.0)


def _mla_lse_log2(q, rows, v_dim, sm):
    out, lse = od.__dict__["_orig_sparse_mla"](q, rows, v_dim, sm)
    return out, lse / math.log(2.0)


def _exclude_self(inp, t):
    return max(int(inp.q_pos[t]), 0)


def _bias8_table():
    t = od.E4M3FN_TABLE.copy()
    finite = np.isfinite(t)
    t[finite] = t[finite] / 2.0
    return t


def _fp8_no_kscale(inp, t):
    q_t, w_t, keys = od.__dict__["_orig_query_index_operands"](inp, t)
    if inp.index_dtype == "fp8":
        b = od.sequence_of(inp, t)
        n = od.candidate_count(inp, t)
        keys = od.decode(od.gather_rows(inp.k_cache, inp, b, np.arange(n)), "fp8")
    return q_t, w_t, keys


def _paged_ignores_table(cache, inp, b, positions):
    positions = np.asarray(positions, dtype=np.int64)
    if inp.block_table is None:
        return cache[b][positions]
    bs = inp.block_size
    nb = inp.block_table.shape[1]
    return cache[b * nb + positions // bs, positions % bs]


def _paged_scales_ignore_table(scale, inp, b, positions):
    positions = np.asarray(positions, dtype=np.int64)
    if inp.block_table is None:
        return scale[b][positions]
    bs = inp.block_size
    nb = inp.block_table.shape[1]
    return scale[b * nb + positions // bs, positions % bs]


def _paged_scales_all_one(scale, inp, b, positions):
    positions = np.asarray(positions, dtype=np.int64)
    if inp.block_table is None:
        return scale[b][positions]
    return np.ones(positions.shape[0], np.float32)


def _bf16_truncated_low(bits):
    b = np.asarray(bits).astype(np.uint16).astype(np.uint32) << np.uint32(15)
    return b.view(np.float32).astype(np.float64)


def _encode_ties_away(y):
    y = np.asarray(y, dtype=np.float64)
    pos = od.E4M3FN_TABLE[:0x7F]
    mag = np.abs(y)
    hi = np.minimum(np.searchsorted(pos, mag, side="left"), 0x7E)
    lo = np.maximum(hi - 1, 0)
    code = np.where((pos[hi] - mag) <= (mag - pos[lo]), hi, lo).astype(np.uint8)
    return np.where(np.signbit(y), code | np.uint8(0x80), code).astype(np.uint8)


def _encode_truncate(y):
    y = np.asarray(y, dtype=np.float64)
    pos = od.E4M3FN_TABLE[:0x7F]
    mag = np.abs(y)
    code = (np.searchsorted(pos, mag, side="right") - 1).astype(np.uint8)
    return np.where(np.signbit(y), code | np.uint8(0x80), code).astype(np.uint8)


def _append_block_offset_dropped(mode, q_pos, block_table, block_size, k_new, k_cache, k_scale):
    # stores every paged token at offset 0 of its block
    q_pos = np.asarray(q_pos, dtype=np.int64)
    if block_table is None:
        return od.__dict__["_orig_append"](mode, q_pos, block_table, block_size, k_new, k_cache, k_scale)
    return od.__dict__["_orig_append"](mode, q_pos - q_pos % block_size, block_table, block_size, k_new, k_cache,
                                       k_scale)


def _dense_with(shift):
    def f(inp, t):
        n = od.candidate_count(inp, t) + shift
        b = od.sequence_of(inp, t)
        q_t = od.decode(inp.q[t], inp.mla_dtype)
        rows = od.decode(od.gather_rows(inp.kv_cache, inp, b, np.arange(max(n, 0))), inp.mla_dtype)
        return od.sparse_mla(q_t, rows, inp.v_dim, inp.sm_scale)
    return f


def _dense_reversed_table(inp, t):
    # reads each sequence's blocks in reverse table order
    if inp.block_table is None:
        return od.__dict__["_orig_dense"](inp, t)
    saved = inp.block_table
    inp.block_table = saved[:, ::-1]
    try:
        return od.__dict__["_orig_dense"](inp, t)
    finally:
        inp.block_table = saved


def _dist_unnormalised(inp, t):
    return od.__dict__["_orig_dist"](inp, t) * inp.q.shape[1]


def _dist_first_head(inp, t):
    n = od.candidate_count(inp, t)
    b = od.sequence_of(inp, t)
    q_t = od.decode(inp.q[t], inp.mla_dtype)[:1]
    rows = od.decode(od.gather_rows(inp.kv_cache, inp, b, np.arange(n)), inp.mla_dtype)
    z = inp.sm_scale * (q_t @ rows.T)
    a = np.exp(z - z.max(axis=1, keepdims=True))
    return (a / a.sum(axis=1, keepdims=True))[0]


def _kl_grad_sign(scores, p):
    loss, g = od.__dict__["_orig_kl"](scores, p)
    return loss, -g


def _kl_reversed(scores, p):
    # KL(softmax(I) || p)
    I = np.asarray(scores, float)
    q = np.exp(I - I.max())
    q /= q.sum()
    p = np.asarray(p, float)
    loss = float(np.sum(q * (np.log(q) - np.log(np.maximum(p, 1e-300)))))
    return loss, od.__dict__["_orig_kl"](scores, p)[1]


def _bwd_relu_value(q, w, keys, grad):
    x = q @ keys.T
    gm = grad[None, :] * w[:, None] * np.maximum(x, 0.0)
    return gm @ keys, (grad[None, :] * np.maximum(x, 0.0)).sum(axis=1), gm.T @ q


def _bwd_dk_no_weight(q, w, keys, grad):
    dq, dw, _ = od.__dict__["_orig_bwd"](q, w, keys, grad)
    gm = grad[None, :] * (q @ keys.T > 0)
    return dq, dw, gm.T @ q


def _bwd_dw_unmasked(q, w, keys, grad):
    dq, _, dk = od.__dict__["_orig_bwd"](q, w, keys, grad)
    return dq, (grad[None, :] * (q @ keys.T)).sum(axis=1), dk


def _sbwd(drop_delta=False, no_value=False, no_scale=False, no_rope=False):
    def f(q, rows, v_dim, sm, dout):
        H, D = q.shape
        if rows.shape[0] == 0:
            return np.zeros((H, D)), np.zeros((0, D))
        z = sm * (q @ rows.T)
        p = np.exp(z - z.max(axis=1, keepdims=True))
        p /= p.sum(axis=1, keepdims=True)
        dp = dout @ rows[:, :v_dim].T
        dz = p * dp if drop_delta else p * (dp - (p * dp).sum(axis=1, keepdims=True))
        dq = (1.0 if no_scale else sm) * (dz @ rows)
        dr = sm * (dz.T @ q)
        if no_rope:
            dr[:, v_dim:] = 0.0
        if not no_value:
            dr[:, :v_dim] += p.T @ dout
        return dq, dr
    return f


def _add_rows_overwrite(acc, inp, b, positions, values):
    positions = np.asarray(positions, dtype=np.int64)
    if inp.block_table is None:
        acc[b, positions] = values
    else:
        blocks = np.asarray(inp.block_table[b], dtype=np.int64)[positions // inp.block_size]
        acc[blocks, positions % inp.block_size] = values


def _add_rows_ignore_table(acc, inp, b, positions, values):
    positions = np.asarray(positions, dtype=np.int64)
    if inp.block_table is None:
        np.add.at(acc, (np.full(positions.shape[0], b), positions), values)
    else:
        nb = inp.block_table.shape[1]
        np.add.at(acc, (b * nb + positions // inp.block_size, positions % inp.block_size), values)


def _sdist_dense_restricted(inp, t, selected):
    # the dense (all-candidate) target restricted to S and renormalised: not the
    # sparse attention's own distribution (heads are weighted differently)
    sel = np.asarray(selected, dtype=np.int64)
    sel = sel[sel >= 0]
    if sel.shape[0] == 0:
        return np.zeros(0)
    p = od.attention_distribution(inp, t)[sel]
    return p / p.sum()


def _skl(variant):
    def f(inp, rows=None, selections=None):
        res = od.__dict__["_orig_skl"](inp, rows, selections)
        if variant == "softmax_all":
            # softmax over every candidate, KL terms over S only
            for i, t in enumerate(res["rows"]):
                q_t, w_t, keys = od.query_index_operands(inp, t)
                I = od.index_scores(q_t, w_t, keys)
                sel = res["idx"][i][res["idx"][i] >= 0]
                p = od.sparse_attention_distribution(inp, t, sel)
                lq = I - (I.max() + np.log(np.exp(I - I.max()).sum()))
                res["loss"][i] = float(np.sum(p * (np.log(np.maximum(p, 1e-300)) - lq[sel])))
        elif variant == "grad_leaks":
            for i, t in enumerate(res["rows"]):
                q_t, w_t, keys = od.query_index_operands(inp, t)
                I = od.index_scores(q_t, w_t, keys)
                g = res["grad_scores"][i]
                off = np.ones(g.shape[0], bool)
                off[res["idx"][i][res["idx"][i] >= 0]] = False
                e = np.exp(I - I.max())
                g[off] = (e / e.sum())[off]
                res["dq"][i], res["dw"][i], _ = od.index_scores_backward(q_t, w_t, keys, g)
        return res
    return f


MUTATIONS = {
    "indexer_no_relu": ("index_scores", _no_relu),
    "indexer_relu_after_weight": ("index_scores", _relu_after_weight),
    "indexer_no_weight": ("index_scores", _no_weight),
    "indexer_key_index_swapped": ("index_scores", _key_index_swapped),
    "topk_ties_to_higher_position": ("topk", _ties_high),
    "topk_one_short": ("topk", _k_minus_one),
    "topk_smallest": ("topk", _smallest),
    "mla_value_from_tail": ("sparse_mla", _mla_value_tail),
    "mla_key_without_rope": ("sparse_mla", _mla_no_rope),
    "mla_missing_scale": ("sparse_mla", _mla_no_scale),
    "mla_lse_base2": ("sparse_mla", _mla_lse_log2),
    "candidates_exclude_self": ("candidate_count", _exclude_self),
    "e4m3_exponent_bias_8": ("E4M3FN_TABLE", _bias8_table()),
    "fp8_key_scale_dropped": ("query_index_operands", _fp8_no_kscale),
    "paged_ignores_block_table": ("gather_rows", _paged_ignores_table),
    "paged_scales_ignore_block_table": ("gather_scales", _paged_scales_ignore_table),
    "paged_scales_all_one": ("gather_scales", _paged_scales_all_one),
    "bf16_wrong_shift": ("decode_bf16", _bf16_truncated_low),
    "fp8_ties_away_from_zero": ("encode_e4m3fn", _encode_ties_away),
    "fp8_round_toward_zero": ("encode_e4m3fn", _encode_truncate),
    "fp8_scale_uses_fnuz_max": ("E4M3FN_MAX", 240.0),
    "append_block_offset_dropped": ("append_index_keys", _append_block_offset_dropped),
    "dense_excludes_self": ("dense_attention", _dense_with(-1)),
    "dense_one_past_self": ("dense_attention", _dense_with(+1)),
    "dense_reversed_block_table": ("dense_attention", _dense_reversed_table),
    "kl_target_not_normalised": ("attention_distribution", _dist_unnormalised),
    "kl_target_first_head_only": ("attention_distribution", _dist_first_head),
    "kl_gradient_sign_flipped": ("kl_rows", _kl_grad_sign),
    "kl_direction_reversed": ("kl_rows", _kl_reversed),
    "bwd_relu_value_as_mask": ("index_scores_backward", _bwd_relu_value),
    "bwd_dk_without_weight": ("index_scores_backward", _bwd_dk_no_weight),
    "bwd_dw_without_relu": ("index_scores_backward", _bwd_dw_unmasked),
    "sparse_bwd_no_softmax_delta": ("sparse_mla_backward", _sbwd(drop_delta=True)),
    "sparse_bwd_no_value_gradient": ("sparse_mla_backward", _sbwd(no_value=True)),
    "sparse_bwd_dq_without_scale": ("sparse_mla_backward", _sbwd(no_scale=True)),
    "sparse_bwd_key_gradient_without_rope": ("sparse_mla_backward", _sbwd(no_rope=True)),
    "sparse_dkv_overwrites_instead_of_adding": ("_add_rows", _add_rows_overwrite),
    "sparse_dkv_ignores_block_table": ("_add_rows", _add_rows_ignore_table),
    "sparse_target_from_dense_attention": ("sparse_attention_distribution", _sdist_dense_restricted),
    "sparse_kl_softmax_over_all_candidates": ("sparse_indexer_kl_loss", _skl("softmax_all")),
    "sparse_kl_gradient_outside_selection": ("sparse_indexer_kl_loss", _skl("grad_leaks")),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(name, monkeypatch):
    attr, repl = MUTATIONS[name]
    monkeypatch.setattr(od, "_orig_sparse_mla", od.sparse_mla, raising=False)
    monkeypatch.setattr(od, "_orig_query_index_operands", od.query_index_operands, raising=False)
    monkeypatch.setattr(od, "_orig_append", od.append_index_keys, raising=False)
    monkeypatch.setattr(od, "_orig_dense", od.dense_attention, raising=False)
    monkeypatch.setattr(od, "_orig_dist", od.attention_distribution, raising=False)
    monkeypatch.setattr(od, "_orig_kl", od.kl_rows, raising=False)
    monkeypatch.setattr(od, "_orig_bwd", od.index_scores_backward, raising=False)
    monkeypatch.setattr(od, "_orig_skl", od.sparse_indexer_kl_loss, raising=False)
    monkeypatch.setattr(od, attr, repl)
    caught = []
    for pin in pins.ALL_PINS:
        try:
            pin(od)
        except Exception as e:           # AssertionError or a crash both count as caught
            caught.append((pin.__name__, type(e).__name__))
    assert caught, f"mutation {name} passed every pin"
