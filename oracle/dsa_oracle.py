"""CPU oracle of the DeepSeek Sparse Attention (DSA) forward path, in float64 NumPy.

TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check and the
benchmark's CPU-baseline leg may import this module.  It shares no code with
the HIP library (its own bf16 and e4m3fn decoders, its own cache addressing)
and the library never calls it.

Sources (the pages this follows; cited below by tag):

* [ZS]  "DeepSeek V3.2: How Far Can Open Models Go If You Actually Try?"
        (zeroshot.it.com) -- section 3.1: the indexer score equation (eq. I),
        the selection-then-attention equation (eq. U) and the MQA-mode note;
        section 3.3: Stage 1, the dense warm-up in which the indexer is trained
        with a KL loss against the dense attention; section 3.4: short
        prompts behave like dense masked attention.
* [LD]  "DeepSeek-V3.2: Pushing the Frontier of Open Large Language Models"
        (papers.lunadong.com summary) -- System Modules (indexer scores the
        preceding tokens; a top-k operation selects; MLA in MQA mode attends),
        Key Hyperparameters (k = 2048).
* [BT]  baseten.co "DeepSeek-V3.2" -- section (1) DSA + MLA: the indexer and
        selector amount to an attention mask over past tokens.

Every step is the plain definition:

1. decode the input bytes to float64 exactly (bf16: bits << 16; e4m3fn: the
   OCP format, 1 sign, 4 exponent bits biased by 7, 3 mantissa bits,
   subnormals m * 2^-9, S.1111.111 NaN);
2. query t of sequence b at position p sees the candidates s = 0..p
   (the query's own position included);
3. eq. I:  I(t,s) = sum_j w(t,j) * ReLU(q(t,j) . k(s));  with an e4m3fn
   indexer the operands are dequantised first, q = q8 * q_scale(t,j),
   k = k8 * k_scale(s);
4. top-k: the first min(k, n) candidates in the order (score descending,
   position ascending);
5. eq. U in MQA mode: every head h attends over the selected latent rows c(s)
   with logits sm_scale * q(t,h) . c(s) over all D dims and values c(s)[:Dv];
   softmax; lse = max + ln(sum exp(z - max)).
6. upstream of the indexer ("runs in FP8" [ZS 3.1]): per-row e4m3fn
   quantisation with an fp32 scale, and the append of a new token's quantised
   index key into the (paged) key cache.
7. the dense MLA that DSA is measured against [ZS 3.4]: eq. U's attention
   over every candidate s = 0..p, no indexer and no selection.
8. the indexer's warm-up objective [ZS 3.3 Stage 1; LD Objective Functions]: the KL divergence
   between the head-aggregated, L1-normalised dense attention distribution
   and softmax(I), and its gradient into q_I, w and k_I.
9. Stage 2, sparse training [ZS 3.3 Stage 2]: the gradient of eq. U's
   attention over the selected rows (dq, and the latent-row gradients summed
   into the cache rows), and the indexer's KL loss restricted to the selected
   subset S_t with its gradient.

Readings where the pages are silent are stated at each function.
"""
from __future__ import annotations

import math
from dataclasses import dataclass
from typing import Optional

import numpy as np


# --------------------------------------------------------------------------
# 1. exact decoding of the element types
# --------------------------------------------------------------------------

def decode_bf16(bits) -> np.ndarray:
    """bfloat16 bit patterns -> float64.  A bf16 value is the top half of an fp32."""
    b = np.asarray(bits).astype(np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):                 # signalling-NaN patterns stay NaN
        return b.view(np.float32).astype(np.float64)


def _build_e4m3fn_table() -> np.ndarray:
    """All 256 OCP FP8 E4M3 ("fn": no infinities, one NaN mantissa) values."""
    table = np.empty(256, dtype=np.float64)
    for code in range(256):
        sign = -1.0 if (code >> 7) & 1 else 1.0
        exp = (code >> 3) & 0xF
        man = code & 0x7
        if exp == 0xF and man == 0x7:
            table[code] = math.nan
        elif exp == 0:
            table[code] = sign * man * 2.0 ** -9          # subnormal: (m/8) * 2^(1-7)
        else:
            table[code] = sign * (1.0 + man / 8.0) * 2.0 ** (exp - 7)
    return table


E4M3FN_TABLE = _build_e4m3fn_table()


def decode_e4m3fn(codes) -> np.ndarray:
    return E4M3FN_TABLE[np.asarray(codes).astype(np.uint8)]


def decode(raw, dtype: str) -> np.ndarray:
    """Raw element bytes of type ``dtype`` ("f32" | "bf16" | "fp8") -> float64."""
    if dtype == "bf16":
        return decode_bf16(raw)
    if dtype == "fp8":
        return decode_e4m3fn(raw)
    if dtype == "f32":
        return np.asarray(raw, dtype=np.float32).astype(np.float64)
    raise ValueError(dtype)


def _finite(x: np.ndarray, what: str) -> np.ndarray:
    if not np.all(np.isfinite(x)):
        raise ValueError(f"oracle read a non-finite {what}: inputs must be finite")
    return x


# --------------------------------------------------------------------------
# 2. inputs and cache addressing
# --------------------------------------------------------------------------

@dataclass
class OracleInputs:
    """Host copies of the bytes the library receives (see workloads.raw_numpy)."""
    mode: str                       # "prefill": every query reads sequence 0; "decode": query t reads sequence t
    q_pos: np.ndarray               # int [T]
    block_table: Optional[np.ndarray]   # int [B, max_blocks] or None (contiguous)
    block_size: int
    index_dtype: str
    q_idx: np.ndarray               # raw [T, H_I, d_I]
    q_scale: Optional[np.ndarray]   # f32 [T, H_I] (fp8 only)
    w: np.ndarray                   # f32 [T, H_I]
    k_cache: np.ndarray             # raw [B, Lmax, d_I] or [N_blk, bs, d_I]
    k_scale: Optional[np.ndarray]   # f32 [B, Lmax] or [N_blk, bs] (fp8 only)
    mla_dtype: str
    q: np.ndarray                   # raw [T, H, D]
    kv_cache: np.ndarray            # raw [B, Lmax, D] or [N_blk, bs, D]
    topk: int
    sm_scale: float
    v_dim: int

    @property
    def num_q(self) -> int:
        return int(self.q_pos.shape[0])


def sequence_of(inp: OracleInputs, t: int) -> int:
    return t if inp.mode == "decode" else 0


def candidate_count(inp: OracleInputs, t: int) -> int:
    """Reading: a query sees every earlier token and itself, s = 0..pos (n = pos + 1)."""
    return max(int(inp.q_pos[t]) + 1, 0)


def gather_rows(cache: np.ndarray, inp: OracleInputs, b: int, positions: np.ndarray) -> np.ndarray:
    """Raw cache rows of sequence ``b`` at logical ``positions``.

    Contiguous cache: ``cache[b, s]``.  Paged cache: logical position s lives in
    physical block ``block_table[b, s // bs]`` at offset ``s % bs``.
    """
    positions = np.asarray(positions, dtype=np.int64)
    if inp.block_table is None:
        return cache[b][positions]
    bs = inp.block_size
    blocks = np.asarray(inp.block_table[b], dtype=np.int64)[positions // bs]
    if np.any(blocks < 0) or np.any(blocks >= cache.shape[0]):
        raise ValueError("block table entry out of range for a candidate position")
    return cache[blocks, positions % bs]


def gather_scales(scale: np.ndarray, inp: OracleInputs, b: int, positions: np.ndarray) -> np.ndarray:
    """fp32 key scales of sequence ``b`` at logical ``positions``: one scale per
    cache slot, addressed exactly like the key rows (``gather_rows``)."""
    positions = np.asarray(positions, dtype=np.int64)
    if inp.block_table is None:
        return scale[b][positions]
    bs = inp.block_size
    blocks = np.asarray(inp.block_table[b], dtype=np.int64)[positions // bs]
    if np.any(blocks < 0) or np.any(blocks >= scale.shape[0]):
        raise ValueError("block table entry out of range for a candidate position")
    return scale[blocks, positions % bs]


# --------------------------------------------------------------------------
# 3. the lightning indexer, eq. I  [ZS 3.1; LD System Modules]
# --------------------------------------------------------------------------

def index_scores(q_t: np.ndarray, w_t: np.ndarray, keys: np.ndarray) -> np.ndarray:
    """eq. I for one query: I(s) = sum_j w_j * ReLU(q_j . k_s).

    q_t [H_I, d_I], w_t [H_I], keys [n, d_I], all float64 -> I [n].
    Reading: no extra scale or normalisation inside the sum; w may have any sign.
    """
    dots = q_t @ keys.T                      # [H_I, n]: q(t,j) . k(s)
    return w_t @ np.maximum(dots, 0.0)       # sum over heads of w * ReLU


def query_index_operands(inp: OracleInputs, t: int):
    """Dequantised float64 (q_t [H_I,d_I], w_t [H_I], keys [n,d_I]) for query t."""
    b = sequence_of(inp, t)
    n = candidate_count(inp, t)
    pos = np.arange(n)
    q_t = decode(inp.q_idx[t], inp.index_dtype)
    keys = decode(gather_rows(inp.k_cache, inp, b, pos), inp.index_dtype)
    w_t = np.asarray(inp.w[t], dtype=np.float64)
    if inp.index_dtype == "fp8":
        # "runs in FP8" [ZS 3.1]: e4m3fn operands with per-row fp32 scales; dequantise, then eq. I.
        q_t = q_t * np.asarray(inp.q_scale[t], dtype=np.float64)[:, None]
        keys = keys * gather_scales(inp.k_scale, inp, b, pos).astype(np.float64)[:, None]
    _finite(q_t, "indexer query")
    _finite(keys, "indexer key")
    _finite(w_t, "head weight")
    return q_t, w_t, keys


def query_index_scores(inp: OracleInputs, t: int) -> np.ndarray:
    """I(t, s) for s = 0..pos_t (float64 [n_t])."""
    q_t, w_t, keys = query_index_operands(inp, t)
    return index_scores(q_t, w_t, keys)


# --------------------------------------------------------------------------
# 4. fine-grained top-k selection  [ZS 3.1 eq. U; LD "Top-k operation"]
# --------------------------------------------------------------------------

def topk(scores: np.ndarray, k: int) -> np.ndarray:
    """Positions of the min(k, n) largest scores, in order (score desc, position asc).

    Readings: exactly min(k, n) positions even when scores tie (ties go to the
    lower position); -0.0 counts as equal to +0.0; when n <= k every candidate
    is selected (dense behaviour for short prompts, [ZS 3.4]).
    """
    s = np.asarray(scores, dtype=np.float64) + 0.0          # -0.0 + 0.0 == +0.0
    _finite(s, "score")
    m = min(int(k), s.shape[0])
    order = np.argsort(-s, kind="stable")                    # stable: equal keys keep position order
    return order[:m].astype(np.int64)


def topk_padded(scores: np.ndarray, k: int) -> np.ndarray:
    """``topk`` written into a length-k int row padded with -1."""
    out = np.full(int(k), -1, dtype=np.int64)
    sel = topk(scores, k)
    out[: sel.shape[0]] = sel
    return out


# --------------------------------------------------------------------------
# 5. sparse MLA in MQA mode, eq. U  [ZS 3.1; LD Novel Architectural Elements]
# --------------------------------------------------------------------------

def sparse_mla(q_t: np.ndarray, rows: np.ndarray, v_dim: int, sm_scale: float):
    """Attention of every head of one query over the selected latent rows.

    q_t [H, D], rows [m, D] float64.  Every head shares the same rows (MQA
    mode): the key is the whole D-wide row, the value its first ``v_dim``
    entries.  Returns (out [H, v_dim], lse [H]).  An empty selection gives a
    zero output and lse = -inf.
    """
    H = q_t.shape[0]
    m = rows.shape[0]
    if m == 0:
        return np.zeros((H, v_dim)), np.full(H, -np.inf)
    z = sm_scale * (q_t @ rows.T)                  # [H, m] logits
    zmax = z.max(axis=1, keepdims=True)
    e = np.exp(z - zmax)
    denom = e.sum(axis=1, keepdims=True)
    p = e / denom                                  # softmax over the selected rows
    out = p @ rows[:, :v_dim]
    lse = zmax[:, 0] + np.log(denom[:, 0])
    return out, lse


def query_attention(inp: OracleInputs, t: int, selected) -> tuple:
    """eq. U for query t over the given selected positions (entries < 0 ignored)."""
    sel = np.asarray(selected, dtype=np.int64)
    sel = sel[sel >= 0]
    n = candidate_count(inp, t)
    if np.any(sel >= n):
        raise ValueError("selected position outside the causal candidates")
    b = sequence_of(inp, t)
    q_t = _finite(decode(inp.q[t], inp.mla_dtype), "MLA query")
    rows = _finite(decode(gather_rows(inp.kv_cache, inp, b, sel), inp.mla_dtype), "latent row")
    return sparse_mla(q_t, rows, inp.v_dim, inp.sm_scale)


# --------------------------------------------------------------------------
# the whole path
# --------------------------------------------------------------------------

def forward(inp: OracleInputs, rows=None, keep_scores: bool = False) -> dict:
    """Indexer -> top-k -> sparse MLA for the query rows ``rows`` (default: all).

    Returns a dict with ``rows``, ``idx`` [R, k] (selection order, -1 padded),
    ``out`` [R, H, Dv], ``lse`` [R, H] and, when asked, ``scores`` (list of [n_t]).
    """
    rows = list(range(inp.num_q)) if rows is None else [int(r) for r in rows]
    k = inp.topk
    H = inp.q.shape[1]
    idx = np.full((len(rows), k), -1, dtype=np.int64)
    out = np.zeros((len(rows), H, inp.v_dim))
    lse = np.zeros((len(rows), H))
    scores = []
    for i, t in enumerate(rows):
        s = query_index_scores(inp, t)
        sel = topk(s, k)
        idx[i, : sel.shape[0]] = sel
        out[i], lse[i] = query_attention(inp, t, sel)
        if keep_scores:
            scores.append(s)
    res = {"rows": rows, "idx": idx, "out": out, "lse": lse}
    if keep_scores:
        res["scores"] = scores
    return res


# --------------------------------------------------------------------------
# 6. fp8 quantisation and key-cache append  ("runs in FP8" [ZS 3.1; BT (1)])
# --------------------------------------------------------------------------

E4M3FN_MAX = 448.0
# codes 0x00..0x7E are the non-negative finite values, in increasing order
_E4M3_POSITIVE = E4M3FN_TABLE[:0x7F]


def encode_e4m3fn(y) -> np.ndarray:
    """Nearest e4m3fn code to each finite value (|y| <= 448), ties to the even code.

    Round to nearest, ties to even, is the IEEE default and the reading for a
    format conversion the pages leave unstated.  The sign bit follows the sign
    of y (-0.0 encodes as 0x80).  Works in float64, where every float32 input,
    every e4m3fn value and every midpoint between neighbours is exact.
    """
    y = np.asarray(y, dtype=np.float64)
    if not np.all(np.isfinite(y)) or np.any(np.abs(y) > E4M3FN_MAX):
        raise ValueError("encode_e4m3fn: inputs must be finite and within +-448 (clamp first)")
    mag = np.abs(y)
    hi = np.searchsorted(_E4M3_POSITIVE, mag, side="left")       # first value >= mag
    hi = np.minimum(hi, 0x7E)
    lo = np.maximum(hi - 1, 0)
    d_lo = mag - _E4M3_POSITIVE[lo]
    d_hi = _E4M3_POSITIVE[hi] - mag
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(mag == _E4M3_POSITIVE[hi], hi, np.where(pick_hi, hi, lo)).astype(np.uint8)
    return np.where(np.signbit(y), code | np.uint8(0x80), code).astype(np.uint8)


def quantize_fp8(x) -> tuple:
    """Per-row e4m3fn quantisation of x [rows, n] (float32 values).

    Reading (per-token fp32 scales): scale = amax(|x|) / 448, or 1 when the row
    is all zeros; code = RNE(clamp(x / scale, -448, 448)).  The scale and the
    quotient are float32 IEEE operations, the precision the quantised codes are
    decided in.  Returns (codes uint8 [rows, n], scale float32 [rows]).
    """
    x = np.asarray(x, dtype=np.float32)
    _finite(x.astype(np.float64), "value to quantise")
    amax = np.max(np.abs(x), axis=1) if x.shape[1] else np.zeros(x.shape[0], np.float32)
    scale = np.where(amax > 0, amax / np.float32(E4M3FN_MAX), np.float32(1.0)).astype(np.float32)
    y = (x / scale[:, None]).astype(np.float32)
    y = np.clip(y, np.float32(-E4M3FN_MAX), np.float32(E4M3FN_MAX))
    return encode_e4m3fn(y), scale


def append_index_keys(mode: str, q_pos, block_table, block_size: int, k_new, k_cache, k_scale) -> tuple:
    """Quantise the new index key of every query token and store it in the cache.

    Token t belongs to sequence sequence_of(t) at position q_pos[t]; its key
    k_new[t] (float32 values) is quantised per row as in quantize_fp8 and
    written, with its scale, to that position's cache slot (through the block
    table when paged).  Tokens whose position is negative or whose block is
    outside the pool are skipped.  Returns updated copies (codes, scales).
    """
    cache = np.array(k_cache, copy=True)
    scales = np.array(k_scale, copy=True)
    codes, sc = quantize_fp8(k_new)
    q_pos = np.asarray(q_pos, dtype=np.int64)
    for t in range(q_pos.shape[0]):
        b = t if mode == "decode" else 0
        pos = int(q_pos[t])
        if pos < 0:
            continue
        if block_table is None:
            if pos >= cache.shape[1]:
                continue
            cache[b, pos] = codes[t]
            scales[b, pos] = sc[t]
        else:
            j = pos // block_size
            if j >= block_table.shape[1]:
                continue
            blk = int(block_table[b, j])
            if blk < 0 or blk >= cache.shape[0]:
                continue
            cache[blk, pos % block_size] = codes[t]
            scales[blk, pos % block_size] = sc[t]
    return cache, scales


# --------------------------------------------------------------------------
# 7. dense MLA, the attention DSA is compared against  [ZS 3.4; LD, dense
#    warm-up stage]
# --------------------------------------------------------------------------

def dense_attention(inp: OracleInputs, t: int) -> tuple:
    """Dense MLA in MQA mode for query t: every head attends over every candidate.

    The comparison the pages draw ([ZS 3.4]: DSA decodes a 128K context about
    twice as cheaply as dense MLA; for short prompts DSA behaves as dense
    attention) is against attention over all preceding tokens and the token
    itself, s = 0..pos_t, with the same logits, softmax and values as eq. U.
    Returns (out [H, v_dim], lse [H]).
    """
    n = candidate_count(inp, t)
    b = sequence_of(inp, t)
    q_t = _finite(decode(inp.q[t], inp.mla_dtype), "MLA query")
    rows = _finite(decode(gather_rows(inp.kv_cache, inp, b, np.arange(n)), inp.mla_dtype), "latent row")
    return sparse_mla(q_t, rows, inp.v_dim, inp.sm_scale)


def dense_forward(inp: OracleInputs, rows=None) -> dict:
    """dense_attention for the query rows ``rows`` (default: all): ``out`` [R, H, Dv], ``lse`` [R, H]."""
    rows = list(range(inp.num_q)) if rows is None else [int(r) for r in rows]
    H = inp.q.shape[1]
    out = np.zeros((len(rows), H, inp.v_dim))
    lse = np.zeros((len(rows), H))
    for i, t in enumerate(rows):
        out[i], lse[i] = dense_attention(inp, t)
    return {"rows": rows, "out": out, "lse": lse}


# --------------------------------------------------------------------------
# 8. the indexer's warm-up loss, L_I = sum_t KL(p_t || softmax(I_t)), and its
#    gradient into the indexer's inputs  [ZS 3.3, Stage 1 (dense warm-up);
#    LD Modeling, Objective Functions]
# --------------------------------------------------------------------------

def attention_distribution(inp: OracleInputs, t: int) -> np.ndarray:
    """p_t over the candidates s = 0..pos_t: the dense attention probabilities of
    every head, summed over heads and L1-normalised.

    Reading of the target [LD Objective Functions]: the main attention's
    softmax weights (eq. U over every candidate) are added over the H heads
    and divided by their total, which is H; float64 [n_t].
    """
    n = candidate_count(inp, t)
    if n == 0:
        return np.zeros(0)
    b = sequence_of(inp, t)
    q_t = _finite(decode(inp.q[t], inp.mla_dtype), "MLA query")
    rows = _finite(decode(gather_rows(inp.kv_cache, inp, b, np.arange(n)), inp.mla_dtype), "latent row")
    z = inp.sm_scale * (q_t @ rows.T)                          # [H, n]
    a = np.exp(z - z.max(axis=1, keepdims=True))
    a /= a.sum(axis=1, keepdims=True)                          # softmax per head
    agg = a.sum(axis=0)                                        # aggregate over heads
    return agg / agg.sum()                                     # L1 normalisation


def kl_rows(scores: np.ndarray, p: np.ndarray) -> tuple:
    """KL(p || softmax(I)) of one query and its gradient with respect to I.

    scores I [n] and target p [n] (sums to 1).  loss = sum_s p_s (log p_s -
    log softmax(I)_s), a term with p_s = 0 contributing 0; dloss/dI =
    softmax(I) - p (p does not depend on I).  Returns (loss, grad [n]).
    """
    I = np.asarray(scores, dtype=np.float64)
    p = np.asarray(p, dtype=np.float64)
    if I.shape[0] == 0:
        return 0.0, np.zeros(0)
    m = I.max()
    lse = m + math.log(np.exp(I - m).sum())
    log_q = I - lse
    nz = p > 0
    loss = float(np.sum(p[nz] * (np.log(p[nz]) - log_q[nz])))
    return loss, np.exp(log_q) - p


def index_scores_backward(q_t: np.ndarray, w_t: np.ndarray, keys: np.ndarray, grad: np.ndarray) -> tuple:
    """Gradient of eq. I for one query, given dL/dI(s) for its candidates.

    With x_js = q_j . k_s and I_s = sum_j w_j ReLU(x_js):
      dL/dw_j = sum_s g_s ReLU(x_js)
      dL/dq_j = sum_s g_s w_j [x_js > 0] k_s
      dL/dk_s = sum_j g_s w_j [x_js > 0] q_j
    Reading: ReLU'(0) = 0.  Returns (dq [H_I, d_I], dw [H_I], dk [n, d_I]).
    """
    x = q_t @ keys.T                                           # [H_I, n]
    on = x > 0
    gm = grad[None, :] * w_t[:, None] * on                     # [H_I, n]
    dw = (grad[None, :] * np.maximum(x, 0.0)).sum(axis=1)
    dq = gm @ keys
    dk = gm.T @ q_t
    return dq, dw, dk


def indexer_kl_loss(inp: OracleInputs, rows=None) -> dict:
    """Loss and gradients of the warm-up objective over query rows ``rows``.

    Per query: I_t from eq. I over its candidates, p_t from
    attention_distribution, (loss_t, g_t) from kl_rows, then
    index_scores_backward.  Key gradients of every query are added into
    ``dk``, shaped like the key cache (one row per cache slot).  Returns
    ``loss`` [R] (the per-query terms; L_I is their sum), ``grad_scores``
    (list of g_t), ``dq`` [R, H_I, d_I], ``dw`` [R, H_I] and ``dk``.
    """
    rows = list(range(inp.num_q)) if rows is None else [int(r) for r in rows]
    H_I, d_I = inp.q_idx.shape[1], inp.q_idx.shape[2]
    loss = np.zeros(len(rows))
    dq = np.zeros((len(rows), H_I, d_I))
    dw = np.zeros((len(rows), H_I))
    dk = np.zeros(inp.k_cache.shape[:-1] + (d_I,))
    grads = []
    for i, t in enumerate(rows):
        q_t, w_t, keys = query_index_operands(inp, t)
        I = index_scores(q_t, w_t, keys)
        p = attention_distribution(inp, t)
        loss[i], g = kl_rows(I, p)
        grads.append(g)
        dq[i], dw[i], dk_t = index_scores_backward(q_t, w_t, keys, g)
        b = sequence_of(inp, t)
        n = candidate_count(inp, t)
        pos = np.arange(n)
        if inp.block_table is None:
            dk[b, pos] += dk_t
        else:
            blocks = np.asarray(inp.block_table[b], dtype=np.int64)[pos // inp.block_size]
            np.add.at(dk, (blocks, pos % inp.block_size), dk_t)
    return {"rows": rows, "loss": loss, "grad_scores": grads, "dq": dq, "dw": dw, "dk": dk}


# --------------------------------------------------------------------------
# 9. Stage 2, sparse training [ZS 3.3 Stage 2: the main attention switches to
#    top-k, every parameter trains, and the indexer keeps learning from a loss
#    taken on the selected subset S_t; NH DSA section: 2048 key-value pairs
#    per query in this stage]
# --------------------------------------------------------------------------

def sparse_mla_backward(q_t: np.ndarray, rows: np.ndarray, v_dim: int, sm_scale: float, dout: np.ndarray) -> tuple:
    """Gradient of eq. U's attention for one query over its selected rows.

    Forward (sparse_mla): z = sm_scale q c^T [H, m], p = softmax_rows(z),
    out = p c[:, :Dv].  Given dL/dout [H, Dv], the chain rule gives
      dp  = dout c[:, :Dv]^T                       [H, m]
      dz  = p * (dp - sum_s p_s dp_s)              [H, m]   (softmax backward)
      dq  = sm_scale dz c                          [H, D]
      dc  = sm_scale dz^T q  (+ p^T dout in the first Dv columns)   [m, D]
    The key and the value of a selected token are the same latent row (MQA
    mode), so its row gradient adds both parts.  An empty selection gives
    zeros.  Returns (dq [H, D], drows [m, D])."""
    H, D = q_t.shape
    m = rows.shape[0]
    if m == 0:
        return np.zeros((H, D)), np.zeros((0, D))
    z = sm_scale * (q_t @ rows.T)
    p = np.exp(z - z.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    dp = dout @ rows[:, :v_dim].T
    dz = p * (dp - (p * dp).sum(axis=1, keepdims=True))
    dq = sm_scale * (dz @ rows)
    drows = sm_scale * (dz.T @ q_t)
    drows[:, :v_dim] += p.T @ dout
    return dq, drows


def _add_rows(acc: np.ndarray, inp: OracleInputs, b: int, positions: np.ndarray, values: np.ndarray) -> None:
    """acc[slot(b, s)] += values for each logical position s (cache layout; a
    position selected twice adds twice)."""
    positions = np.asarray(positions, dtype=np.int64)
    if inp.block_table is None:
        np.add.at(acc, (np.full(positions.shape[0], b), positions), values)
    else:
        blocks = np.asarray(inp.block_table[b], dtype=np.int64)[positions // inp.block_size]
        if np.any(blocks < 0) or np.any(blocks >= acc.shape[0]):
            raise ValueError("block table entry out of range for a selected position")
        np.add.at(acc, (blocks, positions % inp.block_size), values)


def sparse_attention_backward(inp: OracleInputs, idx: np.ndarray, dout: np.ndarray, rows=None) -> dict:
    """The main attention's gradient in Stage 2, for query rows ``rows``.

    Query t attends over its selected positions idx[t] (entries < 0 ignored);
    dout [R, H, Dv] is dL/dout of those rows.  Returns ``dq`` [R, H, D] and
    ``dkv``, shaped like the latent cache, holding for every cache row the sum
    over all queries that selected its token of that query's row gradient (0
    for rows no query selected).  The selection itself has no gradient."""
    rows = list(range(inp.num_q)) if rows is None else [int(r) for r in rows]
    H, D = inp.q.shape[1], inp.q.shape[2]
    dq = np.zeros((len(rows), H, D))
    dkv = np.zeros(inp.kv_cache.shape[:-1] + (D,))
    for i, t in enumerate(rows):
        sel = np.asarray(idx[i], dtype=np.int64)
        sel = sel[sel >= 0]
        if np.any(sel >= candidate_count(inp, t)):
            raise ValueError("selected position outside the causal candidates")
        b = sequence_of(inp, t)
        q_t = _finite(decode(inp.q[t], inp.mla_dtype), "MLA query")
        crow = _finite(decode(gather_rows(inp.kv_cache, inp, b, sel), inp.mla_dtype), "latent row")
        dq[i], dr = sparse_mla_backward(q_t, crow, inp.v_dim, inp.sm_scale, np.asarray(dout[i], dtype=np.float64))
        _add_rows(dkv, inp, b, sel, dr)
    return {"rows": rows, "dq": dq, "dkv": dkv}


def sparse_attention_distribution(inp: OracleInputs, t: int, selected) -> np.ndarray:
    """p_t over the selected positions (order of ``selected``, entries < 0 ignored):
    the Stage-2 main attention's softmax weights over S_t, summed over the heads
    and L1-normalised (each head's weights sum to 1 over S_t, so this is their
    mean).  Reading of the pages' "loss on the selected subset": the target of
    the warm-up objective, taken from the attention that now runs over S_t."""
    sel = np.asarray(selected, dtype=np.int64)
    sel = sel[sel >= 0]
    if sel.shape[0] == 0:
        return np.zeros(0)
    b = sequence_of(inp, t)
    q_t = _finite(decode(inp.q[t], inp.mla_dtype), "MLA query")
    crow = _finite(decode(gather_rows(inp.kv_cache, inp, b, sel), inp.mla_dtype), "latent row")
    z = inp.sm_scale * (q_t @ crow.T)
    a = np.exp(z - z.max(axis=1, keepdims=True))
    a /= a.sum(axis=1, keepdims=True)
    agg = a.sum(axis=0)
    return agg / agg.sum()


def sparse_indexer_kl_loss(inp: OracleInputs, rows=None, selections=None) -> dict:
    """Stage 2's indexer objective over query rows ``rows``: per query
    L_t = KL(p_t,S || softmax(I_t,S)) with S = S_t the query's selection (the
    top-k of its current scores, or ``selections[i]`` when given), p from
    sparse_attention_distribution and the softmax taken over S_t only.  Its
    gradient with respect to I(t, s) is softmax(I_S)_s - p_s for s in S_t and 0
    for every other candidate, back-propagated through eq. I.  Returns
    ``loss`` [R], ``idx`` [R, k] (the selections, -1 padded), ``grad_scores``
    (list of dense [n_t] gradients), ``dq`` [R, H_I, d_I], ``dw`` [R, H_I] and
    ``dk`` (key cache layout)."""
    rows = list(range(inp.num_q)) if rows is None else [int(r) for r in rows]
    H_I, d_I = inp.q_idx.shape[1], inp.q_idx.shape[2]
    k = inp.topk
    loss = np.zeros(len(rows))
    idx = np.full((len(rows), k), -1, dtype=np.int64)
    dq = np.zeros((len(rows), H_I, d_I))
    dw = np.zeros((len(rows), H_I))
    dk = np.zeros(inp.k_cache.shape[:-1] + (d_I,))
    grads = []
    for i, t in enumerate(rows):
        q_t, w_t, keys = query_index_operands(inp, t)
        I = index_scores(q_t, w_t, keys)
        if selections is None:
            sel = topk(I, k)
        else:
            sel = np.asarray(selections[i], dtype=np.int64)
            sel = sel[sel >= 0]
        idx[i, : sel.shape[0]] = sel
        p = sparse_attention_distribution(inp, t, sel)
        loss[i], g_sel = kl_rows(I[sel], p)
        g = np.zeros(I.shape[0])
        g[sel] = g_sel
        grads.append(g)
        dq[i], dw[i], dk_t = index_scores_backward(q_t, w_t, keys, g)
        b = sequence_of(inp, t)
        n = candidate_count(inp, t)
        pos = np.arange(n)
        if inp.block_table is None:
            dk[b, pos] += dk_t
        else:
            blocks = np.asarray(inp.block_table[b], dtype=np.int64)[pos // inp.block_size]
            np.add.at(dk, (blocks, pos % inp.block_size), dk_t)
    return {"rows": rows, "loss": loss, "idx": idx, "grad_scores": grads, "dq": dq, "dw": dw, "dk": dk}
