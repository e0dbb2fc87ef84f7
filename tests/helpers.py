"""Test-side glue: converts generated inputs to the oracle's host form, builds small workloads."""
from __future__ import annotations

import math

import numpy as np

from oracle import OracleInputs
from workloads import Workload, generate, raw_numpy, dtype_tag


def to_oracle(inp) -> OracleInputs:
    """Host copies of the exact bytes in ``inp`` (a workloads.DSAInputs)."""
    return OracleInputs(
        mode=inp.mode,
        q_pos=raw_numpy(inp.q_pos).astype(np.int64),
        block_table=None if inp.block_table is None else raw_numpy(inp.block_table).astype(np.int64),
        block_size=inp.block_size,
        index_dtype=dtype_tag(inp.q_idx),
        q_idx=raw_numpy(inp.q_idx),
        q_scale=raw_numpy(inp.q_scale),
        w=raw_numpy(inp.w),
        k_cache=raw_numpy(inp.k_cache),
        k_scale=raw_numpy(inp.k_scale),
        mla_dtype=dtype_tag(inp.q),
        q=raw_numpy(inp.q),
        kv_cache=raw_numpy(inp.kv_cache),
        topk=inp.topk,
        sm_scale=inp.sm_scale,
        v_dim=inp.wl.v_dim,
    )


def small_workload(mode="prefill", length=40, num_seqs=1, H_I=3, d_I=8, k=6, H=2, D=12, Dv=8,
                   index_dtype="f32", mla_dtype="f32", paged=False, seed=11, length_range=None,
                   w_high=1.0, qkv_std=None, prefill_q_start=0, planted_frac=0.0,
                   block_size=64, w_low=0.0) -> Workload:
    return Workload(name="small", seed=seed, mode=mode, num_seqs=num_seqs, length=length,
                    length_range=length_range, paged=paged, block_size=block_size,
                    index_heads=H_I, index_dim=d_I, topk=k, heads=H, qk_dim=D, v_dim=Dv,
                    index_dtype=index_dtype, mla_dtype=mla_dtype, w_high=w_high, w_low=w_low,
                    qkv_std=(1.0 / math.sqrt(D)) if qkv_std is None else qkv_std,
                    sm_scale=1.0 / math.sqrt(D), prefill_q_start=prefill_q_start,
                    planted_frac=planted_frac)


def small_inputs(**kw):
    lengths = kw.pop("lengths", None)
    wl = small_workload(**kw)
    return generate(wl, "cpu", lengths=lengths)


# ---------------------------------------------------------------- GPU-vs-oracle checkers

import oracle as _oracle  # noqa: E402


def to_oracle_rows(inp, rows):
    """Oracle inputs restricted to query ``rows`` (prefill: row i of the result is query rows[i];
    decode keeps every query, since query t reads sequence t)."""
    if inp.mode == "decode":
        return to_oracle(inp), list(rows)
    rows = list(rows)
    sel = __import__("torch").tensor(rows, dtype=__import__("torch").long, device=inp.q_pos.device)
    oi = OracleInputs(
        mode=inp.mode,
        q_pos=raw_numpy(inp.q_pos.index_select(0, sel)).astype(np.int64),
        block_table=None if inp.block_table is None else raw_numpy(inp.block_table).astype(np.int64),
        block_size=inp.block_size,
        index_dtype=dtype_tag(inp.q_idx),
        q_idx=raw_numpy(inp.q_idx.index_select(0, sel)),
        q_scale=None if inp.q_scale is None else raw_numpy(inp.q_scale.index_select(0, sel)),
        w=raw_numpy(inp.w.index_select(0, sel)),
        k_cache=raw_numpy(inp.k_cache),
        k_scale=raw_numpy(inp.k_scale),
        mla_dtype=dtype_tag(inp.q),
        q=raw_numpy(inp.q.index_select(0, sel)),
        kv_cache=raw_numpy(inp.kv_cache),
        topk=inp.topk, sm_scale=inp.sm_scale, v_dim=inp.wl.v_dim)
    return oi, list(range(len(rows)))


SCORE_TOL = {"f32": 1e-4, "bf16": 1e-2, "fp8": 5e-2}
OUT_TOL = {"f32": 1e-4, "bf16": 2e-2}
NEAR_TIE = 1e-3


def score_magnitude(oi, t):
    """sum_j |w(t,j)| ReLU(q(t,j) . k(s)) over query t's candidates: the size of the
    terms whose signed sum is I(t,s).  It equals |I(t,s)| when every weight is
    non-negative; with mixed-sign weights the sum can cancel to far below its terms,
    and a relative tolerance is then taken against this magnitude instead."""
    q_t, w_t, keys = _oracle.query_index_operands(oi, t)
    return np.abs(w_t) @ np.maximum(q_t @ keys.T, 0.0)


def check_scores(gpu_row, ora_row, tol, what="", scale=None):
    """|I_gpu - I_oracle| <= tol * |I_oracle| (+ a 1e-6 * mean|I| floor for exact zeros);
    with ``scale`` (score_magnitude), tol * scale in place of tol * |I_oracle|."""
    g = np.asarray(gpu_row, dtype=np.float64)
    o = np.asarray(ora_row, dtype=np.float64)
    assert g.shape == o.shape, what
    ref = np.abs(o) if scale is None else np.asarray(scale, dtype=np.float64)
    floor = 1e-6 * (np.mean(ref) if o.size else 0.0)
    bad = np.abs(g - o) > tol * ref + floor
    assert not bad.any(), f"{what}: {bad.sum()} scores off, worst rel {np.max(np.abs(g - o) / (ref + floor + 1e-300)):.3e}"


def check_topk_row_exact(gpu_row, scores_f32, k, what=""):
    """Isolated top-k: bit-exact against the oracle rule run on the same fp32 values."""
    n = scores_f32.shape[0]
    m = min(k, n)
    want = np.sort(_oracle.topk(np.asarray(scores_f32, dtype=np.float64), k))
    got = np.asarray(gpu_row)
    assert np.all(got[m:] == -1), f"{what}: padding"
    assert np.array_equal(got[:m], want), f"{what}: selection differs ({np.setdiff1d(got[:m], want)[:5]})"


def check_topk_row_e2e(gpu_row, ora_scores, k, what="", scale=None):
    """End-to-end top-k: same size, ascending, in range; any swap against the oracle's
    selection lies within NEAR_TIE relative of the oracle's k-th score (with ``scale``,
    score_magnitude, relative to the k-th position's magnitude).  Returns #swaps."""
    n = ora_scores.shape[0]
    m = min(k, n)
    got = np.asarray(gpu_row)
    g = got[:m]
    assert np.all(got[m:] == -1), f"{what}: padding"
    assert np.all(g >= 0) and np.all(g < n), f"{what}: out of range"
    assert np.all(np.diff(g) > 0), f"{what}: not strictly ascending"
    o = _oracle.topk(ora_scores, k)
    if m == n:
        assert g.shape[0] == n
        return 0
    tau = ora_scores[o[-1]]
    band = NEAR_TIE * (abs(tau) if scale is None else float(scale[o[-1]]))
    diff = np.setxor1d(g, o)
    if diff.size:
        dev = np.abs(ora_scores[diff] - tau)
        assert np.all(dev <= band), f"{what}: swap outside the near-tie band ({dev.max():.3e} vs tau {tau:.4e})"
    return diff.size // 2


def check_attention(out_gpu, lse_gpu, out_ora, lse_ora, tol, what=""):
    og = np.asarray(out_gpu, dtype=np.float64)
    oo = np.asarray(out_ora, dtype=np.float64)
    err = np.abs(og - oo).max() if og.size else 0.0
    assert err <= tol, f"{what}: max abs err {err:.3e} > {tol}"
    nrm = np.linalg.norm(oo)
    if nrm > 0:
        rel = np.linalg.norm(og - oo) / nrm
        assert rel <= (1e-2 if tol >= 1e-2 else 1e-5), f"{what}: relative RMS err {rel:.3e}"
    if lse_gpu is not None:
        lg = np.asarray(lse_gpu, dtype=np.float64)
        lo = np.asarray(lse_ora, dtype=np.float64)
        both_inf = np.isneginf(lg) & np.isneginf(lo)
        assert np.array_equal(np.isneginf(lg), np.isneginf(lo)), f"{what}: lse -inf pattern"
        d = np.abs(lg[~both_inf] - lo[~both_inf])
        assert d.size == 0 or d.max() <= (2e-3 if tol >= 1e-2 else 1e-5), f"{what}: lse err {d.max():.3e}"
