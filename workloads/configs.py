"""Seeded synthetic workloads for the DeepSeek Sparse Attention forward path.

Each workload is a frozen description of shapes, element types, value
distributions and structure (causal prefill, single-token decode, paged cache,
planted keys).  The pages measure nothing on a public dataset for this path;
these recipes stand in for "128K context, k = 2048" (lunadong "DeepSeek-V3.2:
Pushing the Frontier of Open Large Language Models", Key Hyperparameters;
baseten "DeepSeek-V3.2", section (1) DSA + MLA).

This module holds no arithmetic of the method.  Both the CPU oracle side and
the HIP side consume the bytes that ``workloads.generate`` produces.
"""
from __future__ import annotations

import dataclasses
import math
from dataclasses import dataclass
from typing import Optional, Tuple


@dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    mode: str                      # "prefill" (one sequence, T = L queries) or "decode" (one query per sequence)
    num_seqs: int                  # B
    length: int                    # prefill: L; decode: fixed context when length_range is None
    length_range: Optional[Tuple[int, int]] = None   # decode: per-sequence context ~ U_int[lo, hi]
    paged: bool = False
    block_size: int = 64
    index_heads: int = 64          # H_I
    index_dim: int = 128           # d_I
    topk: int = 2048               # k
    heads: int = 128               # H
    qk_dim: int = 576              # D = latent 512 + rope 64
    v_dim: int = 512               # Dv
    index_dtype: str = "bf16"      # "f32" | "bf16" | "fp8"
    mla_dtype: str = "bf16"        # "f32" | "bf16"
    w_high: float = 1.0 / 8.0      # w ~ U(w_low, w_high)
    w_low: float = 0.0             # below 0: mixed-sign head weights (the indexer accepts any real w)
    qkv_std: float = 1.0 / 24.0    # q and latent cache ~ N(0, 1) * qkv_std
    sm_scale: float = 1.0 / math.sqrt(576.0)
    planted_frac: float = 0.0      # fraction of key positions shifted along one shared direction
    planted_sigma: float = 3.0
    prefill_q_start: int = 0       # prefill: queries cover positions [q_start, L)

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)

    @property
    def num_q(self) -> int:
        return self.num_seqs if self.mode == "decode" else self.length - self.prefill_q_start


WORKLOADS = {
    # Tiny causal prefill in fp32.
    "tiny_prefill_f32": Workload(
        name="tiny_prefill_f32", seed=1, mode="prefill", num_seqs=1, length=256,
        index_heads=4, index_dim=32, topk=32, heads=8, qk_dim=80, v_dim=64,
        index_dtype="f32", mla_dtype="f32", w_high=1.0,
        qkv_std=1.0 / math.sqrt(80.0), sm_scale=1.0 / math.sqrt(80.0)),
    # Decode, 16 sequences of 8192 tokens, contiguous caches, bf16.
    "decode_8k_bf16": Workload(
        name="decode_8k_bf16", seed=2, mode="decode", num_seqs=16, length=8192),
    # Causal prefill of 16384 tokens with 5% planted keys, bf16.
    "prefill_16k_bf16": Workload(
        name="prefill_16k_bf16", seed=3, mode="prefill", num_seqs=1, length=16384,
        planted_frac=0.05),
    # Long-context decode: 32 sequences, lengths ~ U[32768, 131072], paged 64-token blocks.
    "decode_128k_paged_bf16": Workload(
        name="decode_128k_paged_bf16", seed=4, mode="decode", num_seqs=32, length=131072,
        length_range=(32768, 131072), paged=True),
    # Same, every sequence exactly 131072 tokens.
    "decode_128k_exact_paged_bf16": Workload(
        name="decode_128k_exact_paged_bf16", seed=4, mode="decode", num_seqs=32, length=131072,
        paged=True),
    # The long-context decode with the indexer in e4m3fn (keys and queries with per-token fp32 scales).
    "decode_128k_paged_fp8": Workload(
        name="decode_128k_paged_fp8", seed=4, mode="decode", num_seqs=32, length=131072,
        length_range=(32768, 131072), paged=True, index_dtype="fp8"),
    # Causal prefill of 65536 tokens, indexer in e4m3fn with per-token fp32 scales.
    "prefill_64k_fp8": Workload(
        name="prefill_64k_fp8", seed=5, mode="prefill", num_seqs=1, length=65536,
        index_dtype="fp8"),
}

# The workload the decode throughput headline is quoted on.
BENCH_DEFAULT = "decode_128k_paged_bf16"
