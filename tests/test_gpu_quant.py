"""fp8 quantisation and key-cache append on the GPU against the CPU oracle,
through the C ABI: codes and scales bit for bit (the codes are decided in fp32
on both sides), then quantise -> append -> fused forward end to end."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
from tests.helpers import OUT_TOL, SCORE_TOL, check_attention, check_scores, check_topk_row_e2e, to_oracle
from tests.test_gpu_ops import B, DEV, _say, big_dims
from workloads import generate, raw_numpy

pytestmark = pytest.mark.gpu


def _rows(rows, n, dtype, seed):
    """Rows spanning many binades, an all-zero row and (fp32) a row of subnormals."""
    g = torch.Generator().manual_seed(seed)
    x = torch.randn((rows, n), generator=g, dtype=torch.float32)
    span = 30.0 if dtype == torch.float32 else 20.0
    x *= torch.exp2(torch.empty((rows, 1)).uniform_(-span, span, generator=g))
    x[0] = 0.0
    if rows > 2 and dtype == torch.float32:
        x[2] = torch.randn(n, generator=g) * 1e-40          # fp32 subnormals
    return x.to(dtype)


def _check_quant(x, codes, scale, rep, what):
    ref_codes, ref_scale = oracle.quantize_fp8(x.float().cpu().numpy().reshape(-1, x.shape[-1]))
    got = codes.view(torch.uint8).cpu().numpy().reshape(ref_codes.shape)
    bad = np.argwhere(got != ref_codes)
    assert bad.shape[0] == 0, f"{what}: {bad.shape[0]} codes differ, first at {bad[0].tolist()}"
    s = scale.cpu().numpy()
    assert s.shape == (ref_scale.shape[0], rep)
    assert np.array_equal(s.view(np.int32), np.repeat(ref_scale[:, None], rep, axis=1).view(np.int32)), what


QUANT_CASES = [
    ("keys_bf16", 1003, 128, torch.bfloat16, 1),      # one wave per row, ragged last workgroup
    ("keys_f32", 77, 128, torch.float32, 1),
    ("queries_bf16", 37, 64 * 128, torch.bfloat16, 64),  # one workgroup per row, scale per head
    ("wide_f32", 5, 2052, torch.float32, 3),
    ("short_f32", 9, 4, torch.float32, 2),
]


@pytest.mark.parametrize("name,rows,n,dtype,rep", QUANT_CASES, ids=[c[0] for c in QUANT_CASES])
def test_quantize_matches_oracle(name, rows, n, dtype, rep):
    _say("quantize_fp8", name)
    x = _rows(rows, n, dtype, seed=rows + n).to(DEV)
    codes, scale = B().quantize_fp8(x, scale_repeat=rep)
    torch.cuda.synchronize()
    _check_quant(x, codes, scale, rep, name)


def test_quantize_ties_and_edges():
    """Rows at scale 1 (amax 448): every midpoint between neighbouring codes, values just
    off them, signed zeros, underflow to zero, and the largest codes."""
    _say("quantize_fp8 ties")
    vals = oracle.decode_e4m3fn(np.arange(0x7F, dtype=np.uint8))
    mids = (vals[:-1] + vals[1:]) / 2.0
    pts = np.concatenate([mids, np.nextafter(mids, 0.0), np.nextafter(mids, 1e9), vals,
                          [0.0, 1e-4, 2.0 ** -11, 3 * 2.0 ** -11, 447.0, 440.0]]).astype(np.float32)
    pts = np.concatenate([pts, -pts, np.array([-0.0], np.float32)])
    per = 124                                    # values per row, plus 448 to fix the scale at 1
    pad = (-len(pts)) % per
    pts = np.concatenate([pts, np.zeros(pad, np.float32)]).reshape(-1, per)
    x = np.concatenate([np.full((pts.shape[0], 4), 448.0, np.float32), pts], axis=1)
    xt = torch.from_numpy(x).to(DEV)
    codes, scale = B().quantize_fp8(xt)
    torch.cuda.synchronize()
    _check_quant(xt, codes, scale, 1, "ties")
    assert np.all(scale.cpu().numpy() == 1.0)


APPEND_CASES = [
    ("decode_paged", dict(mode="decode", num_seqs=5, length=600, k=64, paged=True, index_dtype="fp8"),
     [600, 1, 65, 64, 300]),
    ("decode_contig", dict(mode="decode", num_seqs=4, length=200, k=64, index_dtype="fp8"), [200, 7, 64, 1]),
    ("prefill_contig", dict(mode="prefill", length=130, k=64, index_dtype="fp8"), None),
]


@pytest.mark.parametrize("name,kw,lengths", APPEND_CASES, ids=[c[0] for c in APPEND_CASES])
def test_append_matches_oracle(name, kw, lengths):
    _say("append_index_keys", name)
    inp = generate(big_dims(**kw), DEV, lengths=lengths)
    T = inp.num_q
    g = torch.Generator().manual_seed(7)
    k_new = (torch.randn((T, 128), generator=g) * torch.exp2(torch.randn((T, 1), generator=g) * 4)).to(torch.bfloat16)
    q_pos = inp.q_pos.clone()
    table = None if inp.block_table is None else inp.block_table.clone()
    if T > 2:
        q_pos[1] = -1                                # skipped: no position
    if table is not None and T > 3:
        table[3, int(q_pos[3]) // 64] = -1           # skipped: block outside the pool
    inp2 = dataclasses.replace(inp, q_pos=q_pos.to(DEV), block_table=None if table is None else table.to(DEV))
    pb = B().problem_from_inputs(inp2)
    cache, scale = inp.k_cache.clone(), inp.k_scale.clone()
    B().append_index_keys(pb, k_new.to(DEV), cache, scale)
    torch.cuda.synchronize()
    ref_c, ref_s = oracle.append_index_keys(inp.mode, raw_numpy(q_pos).astype(np.int64),
                                            None if table is None else raw_numpy(table).astype(np.int64),
                                            inp.block_size, k_new.float().numpy(), raw_numpy(inp.k_cache),
                                            raw_numpy(inp.k_scale))
    got_c, got_s = raw_numpy(cache), raw_numpy(scale)
    assert np.array_equal(got_c, ref_c), f"{name}: cache bytes differ at {np.argwhere(got_c != ref_c)[:3].tolist()}"
    assert np.array_equal(got_s.view(np.int32), ref_s.view(np.int32)), name


def test_quantize_append_forward():
    """A decode step with fp8 indexing: the new queries and keys arrive in bf16, are
    quantised and appended, and the fused forward runs on the result; the oracle
    quantises and appends on its own and runs its own path."""
    _say("quantise -> append -> forward")
    lengths = [3000, 129, 2048, 700]
    inp = generate(big_dims(mode="decode", num_seqs=4, length=3000, k=2048, paged=True, index_dtype="fp8"),
                   DEV, lengths=lengths)
    T = inp.num_q
    g = torch.Generator().manual_seed(11)
    q_new = torch.randn((T, 64, 128), generator=g).to(torch.bfloat16)
    k_new = torch.randn((T, 128), generator=g).to(torch.bfloat16)
    # GPU: quantise the queries (one scale per token, repeated over the heads), append the keys
    q8, qs = B().quantize_fp8(q_new.to(DEV).reshape(T, 64 * 128), scale_repeat=64)
    cache, kscale = inp.k_cache.clone(), inp.k_scale.clone()
    pb = B().problem_from_inputs(inp)
    B().append_index_keys(pb, k_new.to(DEV), cache, kscale)
    gpu_inp = dataclasses.replace(inp, q_idx=q8.reshape(T, 64, 128), q_scale=qs, k_cache=cache, k_scale=kscale)
    out, lse, idx = B().forward_inputs(gpu_inp)
    pb2 = B().problem_from_inputs(gpu_inp)
    scores = B().index_scores(pb2, gpu_inp.q_idx, gpu_inp.q_scale, gpu_inp.w, gpu_inp.k_cache, gpu_inp.k_scale)
    torch.cuda.synchronize()
    # oracle: its own quantisation and append of the same bf16 values
    oi = to_oracle(inp)
    oq, os_ = oracle.quantize_fp8(q_new.float().numpy().reshape(T, -1))
    oc, osc = oracle.append_index_keys("decode", oi.q_pos, oi.block_table, inp.block_size, k_new.float().numpy(),
                                       oi.k_cache, oi.k_scale)
    oi = dataclasses.replace(oi, q_idx=oq.reshape(T, 64, 128), q_scale=np.repeat(os_[:, None], 64, axis=1),
                             k_cache=oc, k_scale=osc)
    sc_h, ig, og, lg = scores.cpu().numpy(), idx.cpu().numpy(), out.float().cpu().numpy(), lse.cpu().numpy()
    for t in range(T):
        ref = oracle.query_index_scores(oi, t)
        n = ref.shape[0]
        check_scores(sc_h[t][:n], ref, SCORE_TOL["fp8"], f"row {t}")
        check_topk_row_e2e(ig[t], ref, inp.topk, f"row {t}")
        o_ref, l_ref = oracle.query_attention(oi, t, ig[t, :min(inp.topk, n)])
        check_attention(og[t], lg[t], o_ref, l_ref, OUT_TOL["bf16"], f"row {t}")
