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
                   block_size=64) -> Workload:
    return Workload(name="small", seed=seed, mode=mode, num_seqs=num_seqs, length=length,
                    length_range=length_range, paged=paged, block_size=block_size,
                    index_heads=H_I, index_dim=d_I, topk=k, heads=H, qk_dim=D, v_dim=Dv,
                    index_dtype=index_dtype, mla_dtype=mla_dtype, w_high=w_high,
                    qkv_std=(1.0 / math.sqrt(D)) if qkv_std is None else qkv_std,
                    sm_scale=1.0 / math.sqrt(D), prefill_q_start=prefill_q_start,
                    planted_frac=planted_frac)


def small_inputs(**kw):
    lengths = kw.pop("lengths", None)
    wl = small_workload(**kw)
    return generate(wl, "cpu", lengths=lengths)
