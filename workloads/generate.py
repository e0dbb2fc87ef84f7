"""Seeded input generation for the DSA forward path.

Recipe (the same bytes feed the HIP library and the CPU oracle):

1. Structure first: decode context lengths (``U_int[lo, hi]`` when a range is
   given), query positions (decode: the last position of each sequence;
   prefill: ``q_start .. L-1``) and, for a paged cache, a random permutation
   of the block pool assigned to the sequences in order.
2. Then, in this order: indexer queries ``q_I ~ N(0,1)``, indexer keys
   ``k_I ~ N(0,1)``, head weights ``w ~ U(w_low, w_high)`` (``w_low`` is 0
   unless a test asks for mixed signs), MLA queries
   ``q ~ N(0,1)*std``, latent cache ``c ~ N(0,1)*std`` -- all drawn in fp32
   from one ``torch.Generator`` seeded with the workload seed.
3. Planted keys (prefill only): ``round(frac*L)`` positions drawn without
   replacement get ``sigma * u`` added, ``u`` a unit vector along a random
   Gaussian direction, before any cast.
4. Casts: bf16 by round-to-nearest-even (torch ``.to``); e4m3fn with a
   per-token fp32 scale ``amax/448`` (``1`` when ``amax == 0``), the scaled
   values clamped to +-448 and rounded to nearest even.
5. Poison: cache slots that no sequence owns (tails past a sequence's length,
   including the tail of its last paged block) are set to NaN, and unused
   block-table entries to -1, so any read outside the causal set shows up.

Nothing here computes any part of the method.
"""
from __future__ import annotations

import math
from dataclasses import dataclass
from typing import Optional, Sequence

import numpy as np
import torch

from .configs import Workload

E4M3_MAX = 448.0


@dataclass
class DSAInputs:
    wl: Workload
    mode: str                 # "prefill" | "decode"
    num_seqs: int             # B
    lengths: list             # host: context length of each sequence
    q_pos: torch.Tensor       # int32 [T]
    max_ctx: int              # max over queries of q_pos + 1
    block_table: Optional[torch.Tensor]   # int32 [B, max_blocks] or None
    num_blocks: int           # paged pool size (0 when contiguous)
    block_size: int
    max_seq_len: int          # contiguous slots per sequence (0 when paged)
    q_idx: torch.Tensor       # [T, H_I, d_I]   f32 | bf16 | float8_e4m3fn
    q_scale: Optional[torch.Tensor]       # f32 [T, H_I] (fp8 only)
    w: torch.Tensor           # f32 [T, H_I]
    k_cache: torch.Tensor     # [B, Lmax, d_I] or [N_blk, bs, d_I]
    k_scale: Optional[torch.Tensor]       # f32 [B, Lmax] or [N_blk, bs] (fp8 only)
    q: torch.Tensor           # [T, H, D]  f32 | bf16
    kv_cache: torch.Tensor    # [B, Lmax, D] or [N_blk, bs, D]
    topk: int
    sm_scale: float
    planted: Optional[torch.Tensor] = None  # int64 positions carrying the planted shift

    @property
    def num_q(self) -> int:
        return int(self.q_pos.shape[0])

    @property
    def paged(self) -> bool:
        return self.block_table is not None


def _torch_dtype(name: str):
    return {"f32": torch.float32, "bf16": torch.bfloat16, "fp8": torch.float8_e4m3fn}[name]


def _quantise_e4m3(x: torch.Tensor, token_dims: int):
    """Per-token e4m3fn quantisation; returns (codes, scale) with scale over the last ``token_dims`` dims."""
    red = tuple(range(x.dim() - token_dims, x.dim()))
    amax = x.abs().amax(dim=red)
    scale = torch.where(amax > 0, amax / E4M3_MAX, torch.ones_like(amax))
    shape = scale.shape + (1,) * token_dims
    codes = (x / scale.reshape(shape)).clamp(-E4M3_MAX, E4M3_MAX).to(torch.float8_e4m3fn)
    return codes, scale.to(torch.float32)


def generate(wl: Workload, device="cpu", seed: Optional[int] = None,
             lengths: Optional[Sequence[int]] = None) -> DSAInputs:
    """Build the inputs of workload ``wl`` on ``device``.

    ``lengths`` overrides the decode context lengths (one per sequence).
    """
    device = torch.device(device)
    g = torch.Generator(device=device)
    g.manual_seed(wl.seed if seed is None else seed)
    B = wl.num_seqs
    bs = wl.block_size

    # 1. structure
    if wl.mode == "decode":
        if lengths is not None:
            assert len(lengths) == B
            lens = torch.tensor(list(lengths), dtype=torch.int64, device=device)
        elif wl.length_range is not None:
            lo, hi = wl.length_range
            lens = torch.randint(lo, hi + 1, (B,), generator=g, device=device, dtype=torch.int64)
        else:
            lens = torch.full((B,), wl.length, dtype=torch.int64, device=device)
        q_pos = (lens - 1).to(torch.int32)
    else:
        assert B == 1, "a prefill workload holds one sequence"
        lens = torch.tensor([wl.length], dtype=torch.int64, device=device)
        q_pos = torch.arange(wl.prefill_q_start, wl.length, dtype=torch.int32, device=device)
    lens_host = [int(v) for v in lens.cpu().tolist()]
    assert all(v >= 1 for v in lens_host)
    max_len = max(lens_host)
    max_ctx = int(q_pos.max().item()) + 1 if q_pos.numel() else 0

    block_table = None
    num_blocks = 0
    max_seq_len = 0
    if wl.paged:
        nblk = [(v + bs - 1) // bs for v in lens_host]
        num_blocks = sum(nblk)
        max_blocks = (max_len + bs - 1) // bs
        perm = torch.randperm(num_blocks, generator=g, device=device).to(torch.int32)
        block_table = torch.full((B, max_blocks), -1, dtype=torch.int32, device=device)
        off = 0
        for b in range(B):
            block_table[b, : nblk[b]] = perm[off: off + nblk[b]]
            off += nblk[b]
        slots = num_blocks * bs
    else:
        max_seq_len = max_len
        slots = B * max_len

    T = int(q_pos.shape[0])
    H_I, d_I, H, D = wl.index_heads, wl.index_dim, wl.heads, wl.qk_dim

    # 2. values, fixed order
    q_idx = torch.randn((T, H_I, d_I), generator=g, device=device, dtype=torch.float32)
    k_idx = torch.randn((slots, d_I), generator=g, device=device, dtype=torch.float32)
    u = torch.rand((T, H_I), generator=g, device=device, dtype=torch.float32)
    w = u * wl.w_high if wl.w_low == 0.0 else wl.w_low + u * (wl.w_high - wl.w_low)
    q = torch.randn((T, H, D), generator=g, device=device, dtype=torch.float32) * wl.qkv_std
    kv = torch.randn((slots, D), generator=g, device=device, dtype=torch.float32) * wl.qkv_std

    # 3. planted keys (slot == position for a one-sequence contiguous cache)
    planted = None
    if wl.planted_frac > 0:
        assert wl.mode == "prefill" and not wl.paged
        n_pl = int(round(wl.planted_frac * wl.length))
        planted = torch.randperm(wl.length, generator=g, device=device)[:n_pl]
        u = torch.randn((d_I,), generator=g, device=device, dtype=torch.float32)
        u = u / torch.linalg.vector_norm(u)
        k_idx[planted] += wl.planted_sigma * u

    # 5 (before casts). poison slots that no sequence owns
    owned = torch.zeros(slots, dtype=torch.bool, device=device)
    if wl.paged:
        for b in range(B):
            nb = (lens_host[b] + bs - 1) // bs
            blk = block_table[b, :nb].to(torch.int64)
            tok = torch.arange(nb * bs, device=device)
            valid = tok < lens_host[b]
            owned[(blk[tok // bs] * bs + tok % bs)[valid]] = True
    else:
        for b in range(B):
            owned[b * max_len: b * max_len + lens_host[b]] = True
    k_idx[~owned] = float("nan")
    kv[~owned] = float("nan")

    # 4. casts
    q_scale = k_scale = None
    if wl.index_dtype == "fp8":
        q_idx_c, qs = _quantise_e4m3(q_idx, 2)
        q_scale = qs[:, None].expand(T, H_I).contiguous()
        k_idx_c, k_scale = _quantise_e4m3(k_idx, 1)
        k_idx_c = k_idx_c.view(torch.uint8)
        k_idx_c[~owned] = 0x7F            # e4m3fn NaN
        k_idx_c = k_idx_c.view(torch.float8_e4m3fn)
        k_scale[~owned] = float("nan")
    else:
        dt = _torch_dtype(wl.index_dtype)
        q_idx_c = q_idx.to(dt)
        k_idx_c = k_idx.to(dt)
    mdt = _torch_dtype(wl.mla_dtype)
    q_c = q.to(mdt)
    kv_c = kv.to(mdt)

    if wl.paged:
        k_cache = k_idx_c.reshape(num_blocks, bs, d_I)
        kv_cache = kv_c.reshape(num_blocks, bs, D)
        if k_scale is not None:
            k_scale = k_scale.reshape(num_blocks, bs)
    else:
        k_cache = k_idx_c.reshape(B, max_len, d_I)
        kv_cache = kv_c.reshape(B, max_len, D)
        if k_scale is not None:
            k_scale = k_scale.reshape(B, max_len)

    return DSAInputs(
        wl=wl, mode=wl.mode, num_seqs=B, lengths=lens_host, q_pos=q_pos.contiguous(),
        max_ctx=max_ctx, block_table=block_table, num_blocks=num_blocks, block_size=bs,
        max_seq_len=max_seq_len, q_idx=q_idx_c.contiguous(),
        q_scale=None if q_scale is None else q_scale.contiguous(), w=w.contiguous(),
        k_cache=k_cache.contiguous(), k_scale=None if k_scale is None else k_scale.contiguous(),
        q=q_c.contiguous(), kv_cache=kv_cache.contiguous(), topk=wl.topk, sm_scale=wl.sm_scale,
        planted=planted)


def raw_numpy(t: Optional[torch.Tensor]):
    """Host copy of a tensor's bytes as numpy: bf16 -> uint16 bits, e4m3fn -> uint8 codes."""
    if t is None:
        return None
    t = t.detach()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    if t.dtype == torch.float8_e4m3fn:
        return t.view(torch.uint8).cpu().numpy()
    return t.cpu().numpy()


def dtype_tag(t: torch.Tensor) -> str:
    return {torch.float32: "f32", torch.bfloat16: "bf16", torch.float8_e4m3fn: "fp8"}[t.dtype]


def to_device(inp: DSAInputs, device) -> DSAInputs:
    """Copy every tensor of ``inp`` to ``device`` (bytes unchanged)."""
    import dataclasses
    kw = {}
    for f in dataclasses.fields(inp):
        v = getattr(inp, f.name)
        kw[f.name] = v.to(device) if isinstance(v, torch.Tensor) else v
    return DSAInputs(**kw)
