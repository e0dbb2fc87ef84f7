"""ctypes binding of libdsa.so: argument marshalling only.

Every step of the DSA path runs in the library's HIP kernels; PyTorch supplies
device memory and the current stream.  Importing this module loads the
library and raises if it is missing -- there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
# DSA_LIBRARY_PATH selects another build of the same library (e.g. one whose
# host code is compiled with sanitizers); by default the in-tree build.
LIB_PATH = os.environ.get("DSA_LIBRARY_PATH") or os.path.join(_PKG, "libdsa.so")
HEADER_PATH = os.path.join(os.path.dirname(_PKG), "include", "dsa.h")

F32, BF16, FP8_E4M3FN = 0, 1, 2
PREFILL, DECODE = 0, 1
(OP_INDEX_SCORES, OP_TOPK, OP_SPARSE_MLA, OP_FORWARD, OP_DENSE_MLA, OP_ATTENTION_PROBS,
 OP_INDEXER_BACKWARD, OP_INDEXER_KL_LOSS, OP_SPARSE_MLA_BACKWARD) = 0, 1, 2, 3, 4, 5, 6, 7, 8
OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_HIP, ERR_SCRATCH_LIMIT = 0, -1, -2, -3, -4, -5

EXPORTS = ("dsa_workspace_size", "dsa_index_scores", "dsa_topk", "dsa_sparse_mla", "dsa_forward",
           "dsa_forward_noalloc",
           "dsa_dense_mla", "dsa_attention_probs", "dsa_indexer_kl", "dsa_indexer_backward", "dsa_indexer_backward_selected", "dsa_indexer_kl_loss", "dsa_forward_chunk_rows",
           "dsa_quantize_fp8", "dsa_append_index_keys", "dsa_sparse_mla_backward", "dsa_sparse_indexer_kl",
           "dsa_read_ceiling", "dsa_status_string")


class DsaSeqs(ctypes.Structure):
    _fields_ = [("mode", ctypes.c_int32), ("num_seqs", ctypes.c_int32), ("num_q", ctypes.c_int32),
                ("max_ctx", ctypes.c_int32), ("q_pos", ctypes.c_void_p), ("block_table", ctypes.c_void_p),
                ("max_blocks", ctypes.c_int32), ("num_blocks", ctypes.c_int32),
                ("block_size", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("max_seq_len", ctypes.c_int64)]


class DsaDims(ctypes.Structure):
    _fields_ = [("index_heads", ctypes.c_int32), ("index_dim", ctypes.c_int32), ("topk", ctypes.c_int32),
                ("heads", ctypes.c_int32), ("qk_dim", ctypes.c_int32), ("v_dim", ctypes.c_int32),
                ("index_dtype", ctypes.c_int32), ("mla_dtype", ctypes.c_int32)]


class DsaForwardArgs(ctypes.Structure):
    _fields_ = [("q_idx", ctypes.c_void_p), ("q_scale", ctypes.c_void_p), ("w", ctypes.c_void_p),
                ("k_cache", ctypes.c_void_p), ("k_scale", ctypes.c_void_p), ("q", ctypes.c_void_p),
                ("kv_cache", ctypes.c_void_p), ("sm_scale", ctypes.c_float), ("reserved", ctypes.c_int32),
                ("topk_idx", ctypes.c_void_p), ("out", ctypes.c_void_p), ("lse", ctypes.c_void_p),
                ("stage_events", ctypes.c_void_p)]


class DsaKlArgs(ctypes.Structure):
    _fields_ = [("q_idx", ctypes.c_void_p), ("w", ctypes.c_void_p), ("k_cache", ctypes.c_void_p),
                ("q", ctypes.c_void_p), ("kv_cache", ctypes.c_void_p), ("sm_scale", ctypes.c_float),
                ("reserved", ctypes.c_int32), ("lse", ctypes.c_void_p), ("loss", ctypes.c_void_p),
                ("dq_idx", ctypes.c_void_p),
                ("dw", ctypes.c_void_p), ("dk", ctypes.c_void_p), ("stage_events", ctypes.c_void_p)]


class DsaError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {status_string(status)} ({status})")
        self.status = status


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python -m sparse_long_context_relu_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    P, I32, I64, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    sp, dp = ctypes.POINTER(DsaSeqs), ctypes.POINTER(DsaDims)
    lib.dsa_workspace_size.argtypes = [ctypes.c_int, sp, dp]
    lib.dsa_workspace_size.restype = SZ
    lib.dsa_index_scores.argtypes = [sp, dp, P, P, P, P, P, P, I64, P]
    lib.dsa_index_scores.restype = ctypes.c_int
    lib.dsa_topk.argtypes = [sp, I32, P, I64, P, P, SZ, P]
    lib.dsa_topk.restype = ctypes.c_int
    lib.dsa_sparse_mla.argtypes = [sp, dp, ctypes.c_float, P, P, P, P, P, P, SZ, P]
    lib.dsa_sparse_mla.restype = ctypes.c_int
    lib.dsa_forward.argtypes = [sp, dp, ctypes.POINTER(DsaForwardArgs), P, SZ, P]
    lib.dsa_forward.restype = ctypes.c_int
    lib.dsa_forward_noalloc.argtypes = [sp, dp, ctypes.POINTER(DsaForwardArgs), P]
    lib.dsa_forward_noalloc.restype = ctypes.c_int
    lib.dsa_dense_mla.argtypes = [sp, dp, ctypes.c_float, P, P, P, P, P, SZ, P]
    lib.dsa_dense_mla.restype = ctypes.c_int
    lib.dsa_attention_probs.argtypes = [sp, dp, ctypes.c_float, P, P, P, I64, P, I32, P, SZ, P]
    lib.dsa_attention_probs.restype = ctypes.c_int
    lib.dsa_indexer_kl.argtypes = [sp, P, P, I64, P, P]
    lib.dsa_indexer_kl.restype = ctypes.c_int
    lib.dsa_indexer_backward.argtypes = [sp, dp, P, P, P, P, I64, P, P, P, P, SZ, P]
    lib.dsa_indexer_backward.restype = ctypes.c_int
    lib.dsa_indexer_backward_selected.argtypes = [sp, dp, P, P, P, P, I64, P, ctypes.c_int32, P, P, P, P, SZ, P]
    lib.dsa_indexer_backward_selected.restype = ctypes.c_int
    lib.dsa_indexer_kl_loss.argtypes = [sp, dp, ctypes.POINTER(DsaKlArgs), P, SZ, P]
    lib.dsa_indexer_kl_loss.restype = ctypes.c_int
    lib.dsa_forward_chunk_rows.argtypes = [sp, dp]
    lib.dsa_forward_chunk_rows.restype = ctypes.c_int64
    lib.dsa_quantize_fp8.argtypes = [I64, I32, I32, P, P, P, I32, P]
    lib.dsa_quantize_fp8.restype = ctypes.c_int
    lib.dsa_append_index_keys.argtypes = [sp, I32, I32, P, P, P, P]
    lib.dsa_append_index_keys.restype = ctypes.c_int
    lib.dsa_sparse_mla_backward.argtypes = [sp, dp, ctypes.c_float, P, P, P, P, P, P, P, P, P, P, SZ, P]
    lib.dsa_sparse_mla_backward.restype = ctypes.c_int
    lib.dsa_sparse_indexer_kl.argtypes = [sp, P, I64, P, I32, P, P, P]
    lib.dsa_sparse_indexer_kl.restype = ctypes.c_int
    lib.dsa_read_ceiling.argtypes = [P, I64, I32, P, P]
    lib.dsa_read_ceiling.restype = ctypes.c_int
    lib.dsa_status_string.argtypes = [ctypes.c_int]
    lib.dsa_status_string.restype = ctypes.c_char_p
    return lib


LIB = _load()


def status_string(status: int) -> str:
    return LIB.dsa_status_string(int(status)).decode()


def _check(status: int, what: str):
    if status != OK:
        raise DsaError(status, what)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _stream(stream=None):
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


_DTYPES = {torch.float32: F32, torch.bfloat16: BF16, torch.float8_e4m3fn: FP8_E4M3FN}


def dtype_code(t: torch.Tensor) -> int:
    return _DTYPES[t.dtype]


@dataclass
class Problem:
    """Host-side description of one call: C structs plus the tensors they point into."""
    seqs: DsaSeqs
    dims: DsaDims
    keep: tuple           # tensors whose device pointers the structs hold

    @property
    def num_q(self) -> int:
        return self.seqs.num_q


def make_problem(*, mode: str, q_pos: torch.Tensor, max_ctx: int, num_seqs: int,
                 block_table: Optional[torch.Tensor] = None, num_blocks: int = 0,
                 max_seq_len: int = 0, index_heads: int = 64, index_dim: int = 128, topk: int = 2048,
                 heads: int = 128, qk_dim: int = 576, v_dim: int = 512, index_dtype: int = BF16,
                 mla_dtype: int = BF16) -> Problem:
    assert q_pos.dtype == torch.int32 and q_pos.is_contiguous()
    if block_table is not None:
        assert block_table.dtype == torch.int32 and block_table.is_contiguous()
    seqs = DsaSeqs(mode=PREFILL if mode == "prefill" else DECODE, num_seqs=num_seqs,
                   num_q=q_pos.shape[0], max_ctx=max_ctx, q_pos=_ptr(q_pos),
                   block_table=_ptr(block_table),
                   max_blocks=0 if block_table is None else block_table.shape[1],
                   num_blocks=num_blocks, block_size=64 if block_table is not None else 0,
                   reserved=0, max_seq_len=max_seq_len)
    dims = DsaDims(index_heads=index_heads, index_dim=index_dim, topk=topk, heads=heads, qk_dim=qk_dim,
                   v_dim=v_dim, index_dtype=index_dtype, mla_dtype=mla_dtype)
    return Problem(seqs, dims, (q_pos, block_table))


def problem_from_inputs(inp, topk: Optional[int] = None) -> Problem:
    """Problem for an object shaped like workloads.DSAInputs (duck-typed)."""
    wl = inp.wl
    return make_problem(mode=inp.mode, q_pos=inp.q_pos, max_ctx=inp.max_ctx, num_seqs=inp.num_seqs,
                        block_table=inp.block_table, num_blocks=inp.num_blocks,
                        max_seq_len=inp.max_seq_len, index_heads=wl.index_heads, index_dim=wl.index_dim,
                        topk=inp.topk if topk is None else topk, heads=wl.heads, qk_dim=wl.qk_dim,
                        v_dim=wl.v_dim, index_dtype=dtype_code(inp.q_idx), mla_dtype=dtype_code(inp.q))


def forward_chunk_rows(pb: Problem) -> int:
    """Query rows per chunk of dsa_forward for this problem."""
    return int(LIB.dsa_forward_chunk_rows(ctypes.byref(pb.seqs), ctypes.byref(pb.dims)))


def workspace_size(op: int, pb: Problem) -> int:
    return int(LIB.dsa_workspace_size(op, ctypes.byref(pb.seqs), ctypes.byref(pb.dims)))


def _workspace(op: int, pb: Problem, ws: Optional[torch.Tensor], device) -> Optional[torch.Tensor]:
    need = workspace_size(op, pb)
    if need == 0:
        return ws
    if ws is None or ws.numel() * ws.element_size() < need:
        ws = torch.empty(need, dtype=torch.uint8, device=device)
    return ws


def _nbytes(t: Optional[torch.Tensor]) -> int:
    return 0 if t is None else t.numel() * t.element_size()


def index_scores(pb: Problem, q_idx, q_scale, w, k_cache, k_scale, scores=None, ld: Optional[int] = None,
                 stream=None) -> torch.Tensor:
    """scores[t, s] for s <= q_pos[t]; -inf beyond (fp32 [T, ld])."""
    ld = pb.seqs.max_ctx if ld is None else ld
    if scores is None:
        scores = torch.empty((pb.num_q, ld), dtype=torch.float32, device=q_idx.device)
    assert scores.dtype == torch.float32 and scores.is_contiguous() and scores.shape[-1] == ld
    st = LIB.dsa_index_scores(ctypes.byref(pb.seqs), ctypes.byref(pb.dims), _ptr(q_idx), _ptr(q_scale),
                              _ptr(w), _ptr(k_cache), _ptr(k_scale), _ptr(scores), ld, _stream(stream))
    _check(st, "dsa_index_scores")
    return scores


def topk(pb: Problem, scores: torch.Tensor, k: Optional[int] = None, idx=None, ws=None,
         stream=None) -> torch.Tensor:
    """Selected positions, ascending, -1 padded (int32 [T, k])."""
    k = pb.dims.topk if k is None else k
    assert scores.dtype == torch.float32 and scores.is_contiguous()
    if idx is None:
        idx = torch.empty((pb.num_q, k), dtype=torch.int32, device=scores.device)
    d = DsaDims.from_buffer_copy(pb.dims)
    d.topk = k
    pk = Problem(pb.seqs, d, pb.keep)
    ws = _workspace(OP_TOPK, pk, ws, scores.device)
    st = LIB.dsa_topk(ctypes.byref(pb.seqs), k, _ptr(scores), scores.shape[-1], _ptr(idx), _ptr(ws),
                      _nbytes(ws), _stream(stream))
    _check(st, "dsa_topk")
    return idx


def sparse_mla(pb: Problem, sm_scale: float, q, kv_cache, topk_idx, out=None, lse=None, ws=None,
               want_lse: bool = True, stream=None):
    """(out [T, H, Dv] in q's dtype, lse [T, H] fp32 or None)."""
    assert topk_idx.dtype == torch.int32 and topk_idx.is_contiguous()
    if out is None:
        out = torch.empty((pb.num_q, pb.dims.heads, pb.dims.v_dim), dtype=q.dtype, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((pb.num_q, pb.dims.heads), dtype=torch.float32, device=q.device)
    ws = _workspace(OP_SPARSE_MLA, pb, ws, q.device)
    st = LIB.dsa_sparse_mla(ctypes.byref(pb.seqs), ctypes.byref(pb.dims), float(sm_scale), _ptr(q),
                            _ptr(kv_cache), _ptr(topk_idx), _ptr(out), _ptr(lse), _ptr(ws), _nbytes(ws),
                            _stream(stream))
    _check(st, "dsa_sparse_mla")
    return out, lse


def dense_mla(pb: Problem, sm_scale: float, q, kv_cache, out=None, lse=None, ws=None, want_lse: bool = True,
              stream=None):
    """Dense MLA over every candidate of each query: (out [T, H, Dv] in q's dtype, lse [T, H] fp32 or None)."""
    if out is None:
        out = torch.empty((pb.num_q, pb.dims.heads, pb.dims.v_dim), dtype=q.dtype, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((pb.num_q, pb.dims.heads), dtype=torch.float32, device=q.device)
    ws = _workspace(OP_DENSE_MLA, pb, ws, q.device)
    st = LIB.dsa_dense_mla(ctypes.byref(pb.seqs), ctypes.byref(pb.dims), float(sm_scale), _ptr(q),
                           _ptr(kv_cache), _ptr(out), _ptr(lse), _ptr(ws), _nbytes(ws), _stream(stream))
    _check(st, "dsa_dense_mla")
    return out, lse


def attention_probs(pb: Problem, sm_scale: float, q, kv_cache, probs=None, ld: Optional[int] = None, lse=None,
                    lse_given: bool = False, ws=None, stream=None):
    """Head-aggregated dense attention distribution: (probs [T, ld] fp32, lse [T, H] fp32 or None).
    With lse_given, lse holds the per-head log-sum-exp already (e.g. from dense_mla)."""
    ld = pb.seqs.max_ctx if ld is None else ld
    if probs is None:
        probs = torch.empty((pb.num_q, ld), dtype=torch.float32, device=q.device)
    ws = _workspace(OP_ATTENTION_PROBS, pb, ws, q.device)
    st = LIB.dsa_attention_probs(ctypes.byref(pb.seqs), ctypes.byref(pb.dims), float(sm_scale), _ptr(q),
                                 _ptr(kv_cache), _ptr(probs), int(probs.stride(0)), _ptr(lse), int(lse_given),
                                 _ptr(ws), _nbytes(ws),
                                 _stream(stream))
    _check(st, "dsa_attention_probs")
    return probs, lse


def indexer_kl(pb: Problem, scores: torch.Tensor, probs: torch.Tensor, loss=None, stream=None):
    """KL rows: scores (I) is overwritten by dL/dI; returns loss [T] fp32."""
    assert scores.stride(0) == probs.stride(0) and scores.stride(1) == 1 and probs.stride(1) == 1
    if loss is None:
        loss = torch.empty(pb.num_q, dtype=torch.float32, device=scores.device)
    st = LIB.dsa_indexer_kl(ctypes.byref(pb.seqs), _ptr(scores), _ptr(probs), int(scores.stride(0)), _ptr(loss),
                            _stream(stream))
    _check(st, "dsa_indexer_kl")
    return loss


def indexer_backward(pb: Problem, q_idx, w, k_cache, grad_scores, dq=None, dw=None, dk=None, ws=None, stream=None):
    """Gradients of the indexer scores: (dq [T, H_I, d_I], dw [T, H_I], dk like k_cache) in fp32.
    dk defaults to zeros (rows no query sees stay 0)."""
    dev = q_idx.device
    T, HI, DI = q_idx.shape
    if dq is None:
        dq = torch.empty((T, HI, DI), dtype=torch.float32, device=dev)
    if dw is None:
        dw = torch.empty((T, HI), dtype=torch.float32, device=dev)
    if dk is None:
        dk = torch.zeros(tuple(k_cache.shape), dtype=torch.float32, device=dev)
    ws = _workspace(OP_INDEXER_BACKWARD, pb, ws, dev)
    st = LIB.dsa_indexer_backward(ctypes.byref(pb.seqs), ctypes.byref(pb.dims), _ptr(q_idx), _ptr(w), _ptr(k_cache),
                                  _ptr(grad_scores), int(grad_scores.stride(0)), _ptr(dq), _ptr(dw), _ptr(dk),
                                  _ptr(ws), _nbytes(ws), _stream(stream))
    _check(st, "dsa_indexer_backward")
    return dq, dw, dk


def indexer_backward_selected(pb: Problem, q_idx, w, k_cache, grad_scores, topk_idx, dq=None, dw=None, dk=None,
                              ws=None, stream=None):
    """indexer_backward for a score gradient that is zero outside the selection
    topk_idx [T, k]: dq, dw summed over the selected keys only; dk as indexer_backward."""
    dev = q_idx.device
    T, HI, DI = q_idx.shape
    if dq is None:
        dq = torch.empty((T, HI, DI), dtype=torch.float32, device=dev)
    if dw is None:
        dw = torch.empty((T, HI), dtype=torch.float32, device=dev)
    if dk is None:
        dk = torch.zeros(tuple(k_cache.shape), dtype=torch.float32, device=dev)
    ws = _workspace(OP_INDEXER_BACKWARD, pb, ws, dev)
    st = LIB.dsa_indexer_backward_selected(ctypes.byref(pb.seqs), ctypes.byref(pb.dims), _ptr(q_idx), _ptr(w),
                                           _ptr(k_cache), _ptr(grad_scores), int(grad_scores.stride(0)),
                                           _ptr(topk_idx), int(topk_idx.shape[1]), _ptr(dq), _ptr(dw), _ptr(dk),
                                           _ptr(ws), _nbytes(ws), _stream(stream))
    _check(st, "dsa_indexer_backward_selected")
    return dq, dw, dk


def indexer_kl_loss(pb: Problem, q_idx, w, k_cache, q, kv_cache, sm_scale: float, backward: bool = True,
                    lse=None, loss=None, dq=None, dw=None, dk=None, ws=None, stage_events=None, stream=None):
    """The warm-up objective in one call: (loss [T], dq, dw, dk), the gradients None when backward is False."""
    dev = q_idx.device
    T, HI, DI = q_idx.shape
    if loss is None:
        loss = torch.empty(T, dtype=torch.float32, device=dev)
    if backward:
        dq = torch.empty((T, HI, DI), dtype=torch.float32, device=dev) if dq is None else dq
        dw = torch.empty((T, HI), dtype=torch.float32, device=dev) if dw is None else dw
        dk = torch.zeros(tuple(k_cache.shape), dtype=torch.float32, device=dev) if dk is None else dk
    ws = _workspace(OP_INDEXER_KL_LOSS, pb, ws, dev)
    ev_arr = None
    if stage_events is not None:
        assert len(stage_events) == 5
        if any(e.cuda_event == 0 for e in stage_events):
            raise ValueError("stage_events: record each event once first (torch creates the HIP event then)")
        ev_arr = (ctypes.c_void_p * 5)(*[e.cuda_event for e in stage_events])
    args = DsaKlArgs(q_idx=_ptr(q_idx), w=_ptr(w), k_cache=_ptr(k_cache), q=_ptr(q), kv_cache=_ptr(kv_cache),
                     sm_scale=float(sm_scale), reserved=0, lse=_ptr(lse), loss=_ptr(loss), dq_idx=_ptr(dq) if backward else None,
                     dw=_ptr(dw) if backward else None, dk=_ptr(dk) if backward else None,
                     stage_events=None if ev_arr is None else ctypes.cast(ev_arr, ctypes.c_void_p))
    st = LIB.dsa_indexer_kl_loss(ctypes.byref(pb.seqs), ctypes.byref(pb.dims), ctypes.byref(args), _ptr(ws),
                                 _nbytes(ws), _stream(stream))
    _check(st, "dsa_indexer_kl_loss")
    return (loss, dq, dw, dk) if backward else (loss, None, None, None)


def forward(pb: Problem, q_idx, q_scale, w, k_cache, k_scale, q, kv_cache, sm_scale: float, out=None,
            lse=None, topk_idx=None, want_idx: bool = True, want_lse: bool = True, ws=None,
            stage_events=None, stream=None):
    """Indexer -> top-k -> sparse MLA in one call; returns (out, lse, topk_idx)."""
    dev = q.device
    if out is None:
        out = torch.empty((pb.num_q, pb.dims.heads, pb.dims.v_dim), dtype=q.dtype, device=dev)
    if lse is None and want_lse:
        lse = torch.empty((pb.num_q, pb.dims.heads), dtype=torch.float32, device=dev)
    if topk_idx is None and want_idx:
        topk_idx = torch.empty((pb.num_q, pb.dims.topk), dtype=torch.int32, device=dev)
    ws = _workspace(OP_FORWARD, pb, ws, dev)
    ev_arr = None
    if stage_events is not None:
        assert len(stage_events) == 4
        if any(e.cuda_event == 0 for e in stage_events):
            raise ValueError("stage_events: record each event once first (torch creates the HIP event then)")
        ev_arr = (ctypes.c_void_p * 4)(*[e.cuda_event for e in stage_events])
    args = DsaForwardArgs(q_idx=_ptr(q_idx), q_scale=_ptr(q_scale), w=_ptr(w), k_cache=_ptr(k_cache),
                          k_scale=_ptr(k_scale), q=_ptr(q), kv_cache=_ptr(kv_cache),
                          sm_scale=float(sm_scale), reserved=0, topk_idx=_ptr(topk_idx), out=_ptr(out),
                          lse=_ptr(lse),
                          stage_events=None if ev_arr is None else ctypes.cast(ev_arr, ctypes.c_void_p))
    st = LIB.dsa_forward(ctypes.byref(pb.seqs), ctypes.byref(pb.dims), ctypes.byref(args), _ptr(ws),
                         _nbytes(ws), _stream(stream))
    _check(st, "dsa_forward")
    return out, lse, topk_idx


def forward_noalloc(pb: Problem, q_idx, q_scale, w, k_cache, k_scale, q, kv_cache, sm_scale: float, out, lse=None,
                    topk_idx=None, stream=None):
    """dsa_forward_noalloc: dsa_forward with the library's static scratch (no workspace
    argument; the caller passes every output)."""
    args = DsaForwardArgs(q_idx=_ptr(q_idx), q_scale=_ptr(q_scale), w=_ptr(w), k_cache=_ptr(k_cache),
                          k_scale=_ptr(k_scale), q=_ptr(q), kv_cache=_ptr(kv_cache),
                          sm_scale=float(sm_scale), reserved=0, topk_idx=_ptr(topk_idx), out=_ptr(out),
                          lse=_ptr(lse), stage_events=None)
    st = LIB.dsa_forward_noalloc(ctypes.byref(pb.seqs), ctypes.byref(pb.dims), ctypes.byref(args), _stream(stream))
    _check(st, "dsa_forward_noalloc")
    return out, lse, topk_idx


def forward_inputs(inp, ws=None, stage_events=None, **kw):
    """dsa_forward on an object shaped like workloads.DSAInputs."""
    pb = problem_from_inputs(inp)
    return forward(pb, inp.q_idx, inp.q_scale, inp.w, inp.k_cache, inp.k_scale, inp.q, inp.kv_cache,
                   inp.sm_scale, ws=ws, stage_events=stage_events, **kw)


def quantize_fp8(src: torch.Tensor, scale_repeat: int = 1, dst=None, scale=None, stream=None):
    """Per-row e4m3fn quantisation of src [..., len] (bf16 / fp32): returns (codes, scales).

    codes has src's shape (torch.float8_e4m3fn); scales is [rows, scale_repeat] fp32."""
    src = src.contiguous()
    n = src.shape[-1]
    rows = src.numel() // n if n else 0
    if dst is None:
        dst = torch.empty(src.shape, dtype=torch.float8_e4m3fn, device=src.device)
    if scale is None:
        scale = torch.empty((rows, scale_repeat), dtype=torch.float32, device=src.device)
    st = LIB.dsa_quantize_fp8(rows, n, dtype_code(src), _ptr(src), _ptr(dst), _ptr(scale), scale_repeat,
                              _stream(stream))
    _check(st, "dsa_quantize_fp8")
    return dst, scale


def read_ceiling(src: torch.Tensor, paged: bool, sink=None, stream=None, cached: bool = False) -> torch.Tensor:
    """Stream src's bytes with the decode indexer's read shape (a measurement aid;
    `cached`: default-policy loads instead of streaming ones); returns the
    per-wave XOR words [nbytes / 131072] (uint32 as int32)."""
    assert src.is_contiguous()
    nbytes = src.numel() * src.element_size()
    if sink is None:
        sink = torch.empty(max(nbytes // 131072, 1), dtype=torch.int32, device=src.device)
    st = LIB.dsa_read_ceiling(_ptr(src), nbytes, (1 if paged else 0) | (2 if cached else 0), _ptr(sink),
                              _stream(stream))
    _check(st, "dsa_read_ceiling")
    return sink


def append_index_keys(pb: Problem, k_new: torch.Tensor, k_cache: torch.Tensor, k_scale: torch.Tensor, stream=None):
    """Quantise each query token's new index key and store it in the e4m3fn key cache (in place)."""
    k_new = k_new.contiguous()
    st = LIB.dsa_append_index_keys(ctypes.byref(pb.seqs), k_new.shape[-1], dtype_code(k_new), _ptr(k_new),
                                   _ptr(k_cache), _ptr(k_scale), _stream(stream))
    _check(st, "dsa_append_index_keys")


def sparse_mla_backward(pb: Problem, sm_scale: float, q, kv_cache, topk_idx, out, lse, dout, dq=None, dkv=None,
                        probs=None, want_probs: bool = True, ws=None, stream=None):
    """dsa_sparse_mla_backward: returns (dq [T, H, D] fp32, dkv (latent cache layout, fp32), probs [T, k] or None).
    dkv defaults to zeros (rows outside the prefill's positions are not written)."""
    dev = q.device
    T, H, D = pb.num_q, pb.dims.heads, pb.dims.qk_dim
    if dq is None:
        dq = torch.empty((T, H, D), dtype=torch.float32, device=dev)
    if dkv is None:
        dkv = torch.zeros(tuple(kv_cache.shape[:-1]) + (D,), dtype=torch.float32, device=dev)
    if probs is None and want_probs:
        probs = torch.empty((T, pb.dims.topk), dtype=torch.float32, device=dev)
    ws = _workspace(OP_SPARSE_MLA_BACKWARD, pb, ws, dev)
    st = LIB.dsa_sparse_mla_backward(ctypes.byref(pb.seqs), ctypes.byref(pb.dims), float(sm_scale), _ptr(q),
                                     _ptr(kv_cache), _ptr(topk_idx), _ptr(out), _ptr(lse), _ptr(dout), _ptr(dq),
                                     _ptr(dkv), _ptr(probs), _ptr(ws), _nbytes(ws), _stream(stream))
    _check(st, "dsa_sparse_mla_backward")
    return dq, dkv, probs


def sparse_indexer_kl(pb: Problem, scores: torch.Tensor, topk_idx: torch.Tensor, probs: torch.Tensor, loss=None,
                      stream=None):
    """dsa_sparse_indexer_kl: per-query KL on the selection; dL/dI is written over `scores` (in place)."""
    if loss is None:
        loss = torch.empty(pb.num_q, dtype=torch.float32, device=scores.device)
    st = LIB.dsa_sparse_indexer_kl(ctypes.byref(pb.seqs), _ptr(scores), scores.stride(0), _ptr(topk_idx),
                                   topk_idx.shape[1], _ptr(probs), _ptr(loss), _stream(stream))
    _check(st, "dsa_sparse_indexer_kl")
    return loss
