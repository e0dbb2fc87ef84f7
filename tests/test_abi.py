"""The C ABI on the CPU: the library loads, exports what include/dsa.h declares,
its structs match the C layout, and invalid arguments are rejected on the host
before any launch (no GPU is touched by these calls)."""
import ctypes
import os
import re
import subprocess

import pytest
import torch

from sparse_long_context_relu_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    text = open(B.HEADER_PATH).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dsa_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_function():
    names = declared_functions()
    assert set(names) == set(B.EXPORTS), names
    for n in names:
        assert hasattr(B.LIB, n), n


def test_only_api_symbols_exported():
    out = subprocess.run(["nm", "-D", "--defined-only", B.LIB_PATH], capture_output=True, text=True).stdout
    dsa = sorted(l.split()[-1] for l in out.splitlines() if l.split()[-1].startswith("dsa_"))
    assert dsa == sorted(B.EXPORTS)


def test_struct_layout_matches_c(tmp_path):
    src = tmp_path / "layout.c"
    src.write_text("""
#include <stdio.h>
#include <stddef.h>
#include "dsa.h"
#define P(T, f) printf(#T "." #f " %zu\\n", offsetof(T, f));
int main(void) {
  printf("dsa_seqs %zu\\n", sizeof(dsa_seqs));
  printf("dsa_dims %zu\\n", sizeof(dsa_dims));
  printf("dsa_forward_args %zu\\n", sizeof(dsa_forward_args));
  printf("dsa_kl_args %zu\\n", sizeof(dsa_kl_args));
  P(dsa_seqs, q_pos) P(dsa_seqs, block_table) P(dsa_seqs, max_blocks) P(dsa_seqs, max_seq_len)
  P(dsa_dims, mla_dtype)
  P(dsa_forward_args, sm_scale) P(dsa_forward_args, topk_idx) P(dsa_forward_args, stage_events)
  P(dsa_kl_args, sm_scale) P(dsa_kl_args, lse) P(dsa_kl_args, loss) P(dsa_kl_args, dk)
  P(dsa_kl_args, stage_events)
  return 0;
}
""")
    exe = tmp_path / "layout"
    r = subprocess.run(["gcc", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
                        "-I", "/opt/rocm/include", str(src), "-o", str(exe)], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    got = dict(l.split() for l in subprocess.run([str(exe)], capture_output=True, text=True).stdout.splitlines())
    assert int(got["dsa_seqs"]) == ctypes.sizeof(B.DsaSeqs)
    assert int(got["dsa_dims"]) == ctypes.sizeof(B.DsaDims)
    assert int(got["dsa_forward_args"]) == ctypes.sizeof(B.DsaForwardArgs)
    assert int(got["dsa_kl_args"]) == ctypes.sizeof(B.DsaKlArgs)
    for key, v in got.items():
        if "." in key:
            struct, field = key.split(".")
            cls = {"dsa_seqs": B.DsaSeqs, "dsa_dims": B.DsaDims, "dsa_forward_args": B.DsaForwardArgs,
                   "dsa_kl_args": B.DsaKlArgs}[struct]
            assert getattr(cls, field).offset == int(v), key


def _problem(**kw):
    base = dict(mode="decode", q_pos=torch.tensor([8191, 8191], dtype=torch.int32), max_ctx=8192, num_seqs=2,
                max_seq_len=8192)
    base.update(kw)
    return B.make_problem(**base)


FAKE = 0x1000  # never dereferenced: every call below fails validation first


def _index(pb, scores_ld=8192, **ptrs):
    p = dict(q_idx=FAKE, q_scale=None, w=FAKE, k_cache=FAKE, k_scale=None, scores=FAKE)
    p.update(ptrs)
    return B.LIB.dsa_index_scores(ctypes.byref(pb.seqs), ctypes.byref(pb.dims), p["q_idx"], p["q_scale"], p["w"],
                                  p["k_cache"], p["k_scale"], p["scores"], scores_ld, None)


def test_index_scores_validation():
    pb = _problem()
    assert _index(pb, q_idx=None) == B.ERR_INVALID_ARG
    assert _index(pb, scores=None) == B.ERR_INVALID_ARG
    assert _index(pb, scores_ld=100) == B.ERR_INVALID_ARG
    pb.dims.index_heads = 32
    assert _index(pb) == B.ERR_UNSUPPORTED
    pb = _problem(index_dtype=B.FP8_E4M3FN)
    assert _index(pb) == B.ERR_INVALID_ARG            # fp8 needs both scale arrays
    pb = _problem()
    pb.seqs.mode = 7
    assert _index(pb) == B.ERR_INVALID_ARG
    pb = _problem(max_seq_len=100)
    assert _index(pb) == B.ERR_INVALID_ARG            # cache shorter than the context bound
    pb = _problem(max_ctx=300000, max_seq_len=300000)
    assert _index(pb) == B.ERR_UNSUPPORTED
    pb = _problem()
    pb.seqs.num_q = 3                                  # decode: more queries than sequences
    assert _index(pb) == B.ERR_INVALID_ARG
    pb = _problem()
    pb.seqs.reserved = 1
    assert _index(pb) == B.ERR_INVALID_ARG
    bt = torch.zeros((2, 10), dtype=torch.int32)
    pb = _problem(block_table=bt, num_blocks=20)
    assert _index(pb) == B.ERR_INVALID_ARG            # too few block-table columns for max_ctx
    pb = _problem(q_pos=torch.zeros(0, dtype=torch.int32))
    assert _index(pb) == B.OK                          # nothing to do, nothing launched


def test_topk_validation():
    pb = _problem()
    need = B.workspace_size(B.OP_TOPK, pb)
    assert need > 0
    call = lambda k, ws, nb, ld=8192, sc=FAKE, idx=FAKE: B.LIB.dsa_topk(
        ctypes.byref(pb.seqs), k, sc, ld, idx, ws, nb, None)
    assert call(0, FAKE, need) == B.ERR_INVALID_ARG
    assert call(4096, FAKE, need) == B.ERR_UNSUPPORTED
    assert call(2048, None, 0) == B.ERR_WORKSPACE
    assert call(2048, FAKE, need - 1) == B.ERR_WORKSPACE
    assert call(2048, FAKE + 16, need) == B.ERR_WORKSPACE     # base not 256-byte aligned
    assert call(2048, FAKE, need, sc=None) == B.ERR_INVALID_ARG
    assert call(2048, FAKE, need, idx=None) == B.ERR_INVALID_ARG


def test_sparse_mla_validation():
    pb = _problem()
    need = B.workspace_size(B.OP_SPARSE_MLA, pb)
    assert need == 2 * 32 * 128 * (512 * 2 + 8)           # 2 queries x 32 splits: bf16 outputs, fp32 (max, sum)
    call = lambda pbx, ws=FAKE, nb=1 << 40, q=FAKE, sm=0.04: B.LIB.dsa_sparse_mla(
        ctypes.byref(pbx.seqs), ctypes.byref(pbx.dims), sm, q, FAKE, FAKE, FAKE, None, ws, nb, None)
    assert call(pb, q=None) == B.ERR_INVALID_ARG
    assert call(pb, sm=float("nan")) == B.ERR_INVALID_ARG
    if need:
        assert call(pb, ws=None, nb=0) == B.ERR_WORKSPACE
    pb2 = _problem(heads=64)
    assert call(pb2) == B.ERR_UNSUPPORTED
    pb3 = _problem(mla_dtype=B.FP8_E4M3FN)
    assert call(pb3) == B.ERR_UNSUPPORTED
    pb4 = _problem(v_dim=600)
    assert call(pb4) == B.ERR_INVALID_ARG


def test_dense_mla_validation_and_workspace():
    """Dense MLA: host checks and the split / chunk workspace (no launch)."""
    call = lambda pbx, ws=FAKE, nb=1 << 40, q=FAKE, sm=0.04: B.LIB.dsa_dense_mla(
        ctypes.byref(pbx.seqs), ctypes.byref(pbx.dims), sm, q, FAKE, FAKE, None, ws, nb, None)
    per_split = 128 * (512 * 2 + 8)                      # bf16 head outputs + fp32 (max, sum) per split
    # decode, 32 x 128K: 64 splits of 2048 rows, one chunk
    pb = _problem(q_pos=torch.full((32,), 131071, dtype=torch.int32), max_ctx=131072, num_seqs=32,
                  max_seq_len=131072)
    need = B.workspace_size(B.OP_DENSE_MLA, pb)
    assert need == 32 * 64 * per_split
    assert call(pb, q=None) == B.ERR_INVALID_ARG
    assert call(pb, sm=float("nan")) == B.ERR_INVALID_ARG
    assert call(pb, ws=None, nb=0) == B.ERR_WORKSPACE
    assert call(pb, nb=need - 1) == B.ERR_WORKSPACE
    # the top-k size is not read
    pb.dims.topk = 0
    assert B.workspace_size(B.OP_DENSE_MLA, pb) == need
    # prefill, 16K: 8 splits per query, query chunks bounded by 1 GiB of partials
    pf = B.make_problem(mode="prefill", q_pos=torch.arange(16384, dtype=torch.int32), max_ctx=16384, num_seqs=1,
                        max_seq_len=16384)
    ws16k = B.workspace_size(B.OP_DENSE_MLA, pf)
    assert ws16k == (1 << 30) // (8 * per_split) * (8 * per_split)
    # short contexts with many queries need no splits
    short = B.make_problem(mode="prefill", q_pos=torch.arange(512, dtype=torch.int32), max_ctx=512, num_seqs=1,
                           max_seq_len=512)
    assert B.workspace_size(B.OP_DENSE_MLA, short) == 0
    assert call(_problem(heads=64)) == B.ERR_UNSUPPORTED
    assert call(_problem(mla_dtype=B.FP8_E4M3FN)) == B.ERR_UNSUPPORTED
    f32 = dict(mla_dtype=B.F32, heads=8, qk_dim=80, v_dim=64)
    assert call(_problem(**f32)) == B.ERR_UNSUPPORTED     # fp32 lists are limited to 1024 candidates
    small = _problem(q_pos=torch.tensor([255, 100], dtype=torch.int32), max_ctx=256, max_seq_len=256, **f32)
    assert B.workspace_size(B.OP_DENSE_MLA, small) == 0


def test_warmup_objective_validation_and_workspace():
    """Host checks and workspace sizes of the indexer warm-up entry points (no launch)."""
    L = B.LIB
    qp = torch.arange(4096, dtype=torch.int32)
    pf = B.make_problem(mode="prefill", q_pos=qp, max_ctx=4096, num_seqs=1, max_seq_len=4096)
    sp, dp = ctypes.byref(pf.seqs), ctypes.byref(pf.dims)
    # probs: lse of every (query, head) + the lse pass's 2 splits of (max, sum) pairs
    assert B.workspace_size(B.OP_ATTENTION_PROBS, pf) == 4096 * 128 * 4 + 4096 * 2 * 128 * 8
    assert L.dsa_attention_probs(sp, dp, 0.04, None, FAKE, FAKE, 4096, None, 0, FAKE, 1 << 40, None) == B.ERR_INVALID_ARG
    assert L.dsa_attention_probs(sp, dp, 0.04, FAKE, FAKE, FAKE, 4000, None, 0, FAKE, 1 << 40, None) == B.ERR_INVALID_ARG
    assert L.dsa_attention_probs(sp, dp, 0.04, FAKE, FAKE, FAKE, 4096, None, 1, FAKE, 1 << 40, None) == B.ERR_INVALID_ARG
    assert L.dsa_attention_probs(sp, dp, 0.04, FAKE, FAKE, FAKE, 4096, None, 0, None, 0, None) == B.ERR_WORKSPACE
    f32 = B.make_problem(mode="prefill", q_pos=qp[:256], max_ctx=256, num_seqs=1, max_seq_len=256,
                         mla_dtype=B.F32, heads=8, qk_dim=80, v_dim=64)
    assert L.dsa_attention_probs(ctypes.byref(f32.seqs), ctypes.byref(f32.dims), 0.04, FAKE, FAKE, FAKE, 256, None,
                                 0, FAKE, 1 << 40, None) == B.ERR_UNSUPPORTED
    # KL rows: no workspace
    assert L.dsa_indexer_kl(sp, None, FAKE, 4096, FAKE, None) == B.ERR_INVALID_ARG
    assert L.dsa_indexer_kl(sp, FAKE, FAKE, 100, FAKE, None) == B.ERR_INVALID_ARG
    # backward: dk partials of 8 query splits (512 queries each) x 32 key blocks x 128 keys x 128 dims
    assert B.workspace_size(B.OP_INDEXER_BACKWARD, pf) == 8 * 32 * 128 * 128 * 4
    bw = lambda **kw: L.dsa_indexer_backward(sp, dp, *[kw.get(k, FAKE) for k in ("q", "w", "k", "g")], 4096,
                                             *[kw.get(k, FAKE) for k in ("dq", "dw", "dk")], FAKE, 1 << 40, None)
    assert bw(dk=None) == B.ERR_INVALID_ARG and bw(g=None) == B.ERR_INVALID_ARG
    # the same over a selection: the list is required and k is checked like dsa_topk's
    bs = lambda sel=FAKE, k=2048, **kw: L.dsa_indexer_backward_selected(
        sp, dp, *[kw.get(n, FAKE) for n in ("q", "w", "k", "g")], 4096, sel, k,
        *[kw.get(n, FAKE) for n in ("dq", "dw", "dk")], FAKE, 1 << 40, None)
    assert bs(sel=None) == B.ERR_INVALID_ARG and bs(dq=None) == B.ERR_INVALID_ARG and bs(g=None) == B.ERR_INVALID_ARG
    assert bs(k=0) != B.OK and bs(k=-16) != B.OK
    fp8 = B.make_problem(mode="prefill", q_pos=qp, max_ctx=4096, num_seqs=1, max_seq_len=4096,
                         index_dtype=B.FP8_E4M3FN)
    assert L.dsa_indexer_backward(ctypes.byref(fp8.seqs), ctypes.byref(fp8.dims), FAKE, FAKE, FAKE, FAKE, 4096, FAKE,
                                  FAKE, FAKE, FAKE, 1 << 40, None) == B.ERR_UNSUPPORTED
    # decode: dq key splits (2 per query at 4096 candidates), no dk partials
    dc = B.make_problem(mode="decode", q_pos=torch.full((4,), 4095, dtype=torch.int32), max_ctx=4096, num_seqs=4,
                        max_seq_len=4096)
    assert B.workspace_size(B.OP_INDEXER_BACKWARD, dc) == 4 * 2 * (64 * 128 + 64) * 4
    # the fused objective: scores and target rows, then the larger of the two sub-workspaces
    need = B.workspace_size(B.OP_INDEXER_KL_LOSS, pf)
    assert need == 2 * 4096 * 4096 * 4 + max(B.workspace_size(B.OP_ATTENTION_PROBS, pf),
                                             B.workspace_size(B.OP_INDEXER_BACKWARD, pf))
    args = B.DsaKlArgs(q_idx=FAKE, w=FAKE, k_cache=FAKE, q=FAKE, kv_cache=FAKE, sm_scale=0.04, loss=FAKE, dq_idx=FAKE,
                       dw=FAKE, dk=None)
    call = lambda nb: L.dsa_indexer_kl_loss(sp, dp, ctypes.byref(args), FAKE, nb, None)
    assert call(need) == B.ERR_INVALID_ARG                      # dq without dk
    args.dk = FAKE
    assert call(need - 1) == B.ERR_WORKSPACE
    args.reserved = 1
    assert call(need) == B.ERR_INVALID_ARG


def test_forward_validation_and_workspace():
    pb = _problem()
    need = B.workspace_size(B.OP_FORWARD, pb)
    # scores (2 x 8192 fp32) + idx + top-k rows + split partials, each 256-byte aligned
    assert need >= 2 * 8192 * 4 + 2 * 2048 * 4
    args = B.DsaForwardArgs(q_idx=FAKE, w=FAKE, k_cache=FAKE, q=FAKE, kv_cache=FAKE, sm_scale=0.04, out=FAKE)
    call = lambda ws, nb: B.LIB.dsa_forward(ctypes.byref(pb.seqs), ctypes.byref(pb.dims), ctypes.byref(args),
                                            ws, nb, None)
    assert call(None, 0) == B.ERR_WORKSPACE
    assert call(FAKE, need - 1) == B.ERR_WORKSPACE
    assert call(FAKE + 4, need) == B.ERR_WORKSPACE            # base not 256-byte aligned
    args.out = None
    assert call(FAKE, need) == B.ERR_INVALID_ARG
    args.out = FAKE
    args.reserved = 3
    assert call(FAKE, need) == B.ERR_INVALID_ARG
    # prefill workspaces are bounded by query chunking, not by T x L scores
    qp = torch.arange(65536, dtype=torch.int32)
    pf = B.make_problem(mode="prefill", q_pos=qp, max_ctx=65536, num_seqs=1, max_seq_len=65536,
                        index_dtype=B.FP8_E4M3FN)
    ws64k = B.workspace_size(B.OP_FORWARD, pf)
    assert (2 << 30) <= ws64k < (5 << 29)          # 8192-row chunks of 256 KiB score rows, not 16 GiB
    assert B.forward_chunk_rows(pf) == 8192
    assert B.forward_chunk_rows(pb) == 2           # decode: every query in one chunk


def test_quantize_and_append_validation():
    """Host-side checks of the fp8 quantisation and key-append entry points (no launch)."""
    L, P = B.LIB, ctypes.c_void_p
    fake = P(0x1000)
    assert L.dsa_quantize_fp8(-1, 128, B.BF16, fake, fake, fake, 1, None) == B.ERR_INVALID_ARG
    assert L.dsa_quantize_fp8(4, 0, B.BF16, fake, fake, fake, 1, None) == B.ERR_INVALID_ARG
    assert L.dsa_quantize_fp8(4, 128, B.FP8_E4M3FN, fake, fake, fake, 1, None) == B.ERR_INVALID_ARG
    assert L.dsa_quantize_fp8(4, 130, B.BF16, fake, fake, fake, 1, None) == B.ERR_UNSUPPORTED
    assert L.dsa_quantize_fp8(4, 128, B.BF16, fake, fake, fake, 2000, None) == B.ERR_UNSUPPORTED
    assert L.dsa_quantize_fp8(4, 128, B.BF16, None, fake, fake, 1, None) == B.ERR_INVALID_ARG
    assert L.dsa_quantize_fp8(0, 128, B.BF16, None, None, None, 1, None) == B.OK
    q_pos = torch.zeros(2, dtype=torch.int32)
    pb = B.make_problem(mode="decode", q_pos=q_pos, max_ctx=64, num_seqs=2, max_seq_len=64,
                        index_dtype=B.FP8_E4M3FN, topk=64)
    sp = ctypes.byref(pb.seqs)
    assert L.dsa_append_index_keys(sp, 128, B.BF16, fake, fake, None, None) == B.ERR_INVALID_ARG
    assert L.dsa_append_index_keys(sp, 126, B.BF16, fake, fake, fake, None) == B.ERR_UNSUPPORTED
    assert L.dsa_append_index_keys(sp, 128, B.FP8_E4M3FN, fake, fake, fake, None) == B.ERR_INVALID_ARG
    assert L.dsa_append_index_keys(None, 128, B.BF16, fake, fake, fake, None) == B.ERR_INVALID_ARG


def test_read_ceiling_validation():
    """Host-side checks of the read-rate measurement entry point (no launch)."""
    L, P = B.LIB, ctypes.c_void_p
    fake = P(0x1000)
    chunk = 512 * 1024
    assert L.dsa_read_ceiling(None, chunk, 0, fake, None) == B.ERR_INVALID_ARG
    assert L.dsa_read_ceiling(fake, chunk, 0, None, None) == B.ERR_INVALID_ARG
    assert L.dsa_read_ceiling(P(0x1008), chunk, 0, fake, None) == B.ERR_INVALID_ARG   # src not 16-byte aligned
    assert L.dsa_read_ceiling(fake, 0, 0, fake, None) == B.ERR_INVALID_ARG
    assert L.dsa_read_ceiling(fake, chunk + 16, 0, fake, None) == B.ERR_UNSUPPORTED
    assert L.dsa_read_ceiling(fake, 3 * chunk, 1, fake, None) == B.ERR_UNSUPPORTED    # 96 blocks: not a power of two
    assert L.dsa_read_ceiling(fake, 3 * chunk, 3, fake, None) == B.ERR_UNSUPPORTED    # paged + cached: same check
    assert L.dsa_read_ceiling(fake, chunk, 4, fake, None) == B.ERR_INVALID_ARG        # unknown flag bit
    assert L.dsa_read_ceiling(fake, chunk, -1, fake, None) == B.ERR_INVALID_ARG


def test_status_strings():
    for s in (B.OK, B.ERR_INVALID_ARG, B.ERR_UNSUPPORTED, B.ERR_WORKSPACE, B.ERR_HIP):
        assert B.status_string(s).startswith("DSA_")
    assert "unknown" in B.status_string(12345)


@pytest.mark.parametrize("T", [8292, 8192 + 255, 65791, 131327, 16384 + 1])
def test_forward_workspace_covers_ragged_tail_chunk(T):
    """A prefill whose last query chunk is short (T mod chunk in [1, 255]) runs that
    chunk with the sliced top-k layout and split attention rows, both larger per row
    than a full chunk's.  Every chunk starts its regions at the same offsets, so the
    forward workspace must hold, after the score and index regions of a full chunk,
    the larger top-k region and the larger split-partial region of the two chunk
    sizes (each taken from the standalone ops' workspace sizes, which use the same
    layouts)."""
    a256 = lambda x: (x + 255) // 256 * 256
    qp = torch.arange(T, dtype=torch.int32)
    pf = B.make_problem(mode="prefill", q_pos=qp, max_ctx=T, num_seqs=1, max_seq_len=T)
    chunk = B.forward_chunk_rows(pf)
    tail = T % chunk
    assert chunk == 8192 and 0 < tail < 256
    need = B.workspace_size(B.OP_FORWARD, pf)

    def part(rows):
        p = B.make_problem(mode="prefill", q_pos=qp[T - rows:], max_ctx=T, num_seqs=1, max_seq_len=T)
        return B.workspace_size(B.OP_TOPK, p), B.workspace_size(B.OP_SPARSE_MLA, p)

    (tk_full, ml_full), (tk_tail, ml_tail) = part(chunk), part(tail)
    assert ml_tail > ml_full == 0          # only the short chunk splits its attention rows
    ld = (T + 63) // 64 * 64
    want = a256(ld * chunk * 4) + a256(chunk * 2048 * 4) + a256(max(tk_full, tk_tail)) + a256(max(ml_full, ml_tail))
    assert need >= want, (need, want)


def test_forward_noalloc_rejects_problems_over_its_scratch():
    """dsa_forward_noalloc checks its arguments like dsa_forward, then rejects on the
    host a problem whose forward workspace exceeds the 128 MiB static scratch (no
    launch; no device is touched by these calls)."""
    assert B.status_string(B.ERR_SCRATCH_LIMIT).startswith("DSA_ERR_SCRATCH_LIMIT")
    big = B.make_problem(mode="decode", q_pos=torch.full((128,), 131071, dtype=torch.int32), max_ctx=131072,
                         num_seqs=128, max_seq_len=131072)
    assert B.workspace_size(B.OP_FORWARD, big) > (128 << 20)
    args = B.DsaForwardArgs(q_idx=FAKE, w=FAKE, k_cache=FAKE, q=FAKE, kv_cache=FAKE, sm_scale=0.04, out=FAKE)
    call = lambda pb: B.LIB.dsa_forward_noalloc(ctypes.byref(pb.seqs), ctypes.byref(pb.dims), ctypes.byref(args), None)
    assert call(big) == B.ERR_SCRATCH_LIMIT
    args.out = None
    assert call(big) == B.ERR_INVALID_ARG                 # argument checks come first
    args.out = FAKE
    pb = _problem(q_pos=torch.zeros(0, dtype=torch.int32))
    assert call(pb) == B.OK                               # nothing to do, nothing launched
    fits = B.make_problem(mode="decode", q_pos=torch.full((32,), 131071, dtype=torch.int32), max_ctx=131072,
                          num_seqs=32, max_seq_len=131072)
    assert B.workspace_size(B.OP_FORWARD, fits) <= (128 << 20)   # the 128K decode batch fits


def test_stage2_validation_and_workspace():
    """Host checks of the Stage-2 entry points and the backward's chunked workspace (no launch)."""
    L = B.LIB
    qp = torch.arange(16384, dtype=torch.int32)
    pf = B.make_problem(mode="prefill", q_pos=qp, max_ctx=16384, num_seqs=1, max_seq_len=16384)
    sp, dp = ctypes.byref(pf.seqs), ctypes.byref(pf.dims)
    a256 = lambda x: (x + 255) // 256 * 256
    # chunks of 256 query rows: Delta, per-tile dS, per-row P | dS, bf16 row gradients, the key map
    want = (a256(256 * 128 * 4) + a256(256 * 64 * 128 * 32 * 2) + a256(256 * 2048 * 2 * 128 * 2)
            + a256(256 * 2048 * 576 * 2) + a256(16384 * 256 * 2))
    need = B.workspace_size(B.OP_SPARSE_MLA_BACKWARD, pf)
    assert need == want
    call = lambda pb, **kw: L.dsa_sparse_mla_backward(
        ctypes.byref(pb.seqs), ctypes.byref(pb.dims), 0.04, *[kw.get(k, FAKE) for k in
                                                              ("q", "kv", "idx", "out", "lse", "dout", "dq", "dkv")],
        None, kw.get("ws", FAKE), kw.get("nb", 1 << 40), None)
    assert call(pf, dkv=None) == B.ERR_INVALID_ARG and call(pf, lse=None) == B.ERR_INVALID_ARG
    assert call(pf, ws=None, nb=0) == B.ERR_WORKSPACE and call(pf, nb=need - 1) == B.ERR_WORKSPACE
    dec = _problem()
    assert call(dec) == B.ERR_UNSUPPORTED                         # training runs over whole sequences
    odd = B.make_problem(mode="prefill", q_pos=qp[:100], max_ctx=100, num_seqs=1, max_seq_len=100, topk=40)
    assert call(odd) == B.ERR_UNSUPPORTED                         # k not a multiple of 16
    f32 = B.make_problem(mode="prefill", q_pos=qp[:100], max_ctx=100, num_seqs=1, max_seq_len=100,
                         mla_dtype=B.F32, heads=8, qk_dim=80, v_dim=64, topk=32)
    assert call(f32) == B.ERR_UNSUPPORTED
    few = B.make_problem(mode="prefill", q_pos=qp[:44], max_ctx=300, num_seqs=1, max_seq_len=300, topk=64)
    assert B.workspace_size(B.OP_SPARSE_MLA_BACKWARD, few) == (
        a256(44 * 128 * 4) + a256(44 * 2 * 128 * 32 * 2) + a256(44 * 64 * 2 * 128 * 2) + a256(44 * 64 * 576 * 2)
        + a256(300 * 48 * 2))
    kl = lambda pb, sc=FAKE, ld=16384, idx=FAKE, k=2048, pr=FAKE, loss=FAKE: L.dsa_sparse_indexer_kl(
        ctypes.byref(pb.seqs), sc, ld, idx, k, pr, loss, None)
    assert kl(pf, sc=None) == B.ERR_INVALID_ARG and kl(pf, pr=None) == B.ERR_INVALID_ARG
    assert kl(pf, ld=100) == B.ERR_INVALID_ARG and kl(pf, k=0) == B.ERR_INVALID_ARG
    assert kl(pf, k=4096) == B.ERR_UNSUPPORTED
