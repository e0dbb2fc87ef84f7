#!/usr/bin/env python3
"""Throughput of the DSA forward path (indexer -> top-k -> sparse MLA) on one MI355X.

A step is one dsa_forward call over one batch of seeded synthetic inputs that
are resident in HBM before timing starts.  The default workload is the
long-context decode batch: 32 sequences, context ~ U[32768, 131072], paged
64-token blocks, k = 2048, H_I = 64, d_I = 128, H = 128, D = 576, Dv = 512,
bf16.  Prints one JSON line (stdout); progress goes to stderr.

Every timed region cycles through several seeded input sets, enough that two
steps on the same set are separated by at least twice the 256 MB MALL of other
inputs: no step reads what an earlier step left in the last-level cache.
Secondary lines: every context exactly 128K, the e4m3fn indexer (quantise +
append + forward), 16 x 8K contiguous decode, the 16K bf16 prefill and the 64K
prefill with the e4m3fn indexer, dense MLA on the same inputs, the indexer's
warm-up objective, measured ceilings, and the float64 oracle on the host.

    python bench.py [--steps K] [--warmup W] [--workload NAME]
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "DSA decode tokens/s + prefill tokens/s at L=128K, k=2048; % HBM/MFMA roofline"
HBM_PEAK_GBS = 8000.0                                  # MI355X HBM3E, published
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "fp8": 5000.0, "f32": 157.3}
ELEM = {"f32": 4, "bf16": 2, "fp8": 1}


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def algorithmic_bytes(inp):
    """Bytes the method must move per step, and per indexer launch (score and index
    round trips through HBM are overhead and not counted)."""
    wl = inp.wl
    n = inp.q_pos.to("cpu").long() + 1
    T = inp.num_q
    e_i = ELEM[wl.index_dtype]
    e_m = ELEM[wl.mla_dtype]
    keys = int(n.sum()) * wl.index_dim * e_i
    if wl.index_dtype == "fp8":
        keys += int(n.sum()) * 4 + T * wl.index_heads * 4
    idx_bytes = keys + T * wl.index_heads * (wl.index_dim * e_i + 4)
    rows = int(n.clamp(max=wl.topk).sum())
    mla_bytes = rows * wl.qk_dim * e_m + T * wl.heads * (wl.qk_dim + wl.v_dim) * e_m
    return idx_bytes, idx_bytes + mla_bytes


def algorithmic_flops(inp):
    wl = inp.wl
    n = inp.q_pos.to("cpu").long() + 1
    idx = int(n.sum()) * wl.index_heads * 2 * wl.index_dim
    mla = int(n.clamp(max=wl.topk).sum()) * wl.heads * 2 * (wl.qk_dim + wl.v_dim)
    return idx, mla


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
KERNEL_ISA_FILE = os.path.join(ROOT, "sparse_long_context_relu_amd", "kernel_isa.json")


def kernel_fingerprint(kernel):
    """SHA-256 of the kernel's gfx950 assembly in the library as built (written by the build)."""
    try:
        with open(KERNEL_ISA_FILE) as f:
            return json.load(f).get(kernel)
    except (OSError, ValueError):
        return None


def measured_traffic(kernel, workload):
    """HBM bytes per launch of `kernel` on `workload` from the committed counter
    runs (FETCH_SIZE and WRITE_SIZE, each scaled by what the counter reads for a
    plain copy of known size), or None when there are none or the kernel's
    machine code differs from the one the counters were taken on."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    fp = kernel_fingerprint(kernel + "<bf16>")
    for e in rec.get("entries", []):
        if e.get("kernel") == kernel and e.get("workload") == workload:
            if fp is None or e.get("isa_sha256") != fp:
                return None
            return int(e["traffic_bytes"])
    return None


def make_events(torch, count):
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(count)]
    for e in evs:            # torch creates the HIP event on first record
        e.record()
    torch.cuda.synchronize()
    return evs


def settle(torch, call, ms):
    """Run `call` untimed for about `ms` of wall time.  The GPU raises its shader
    clock over tens of milliseconds of sustained work; timing right after an
    idle gap (input generation, a sync) would measure the ramp, not the step."""
    if ms <= 0:
        return
    t0 = time.perf_counter()
    while (time.perf_counter() - t0) * 1e3 < ms:
        for _ in range(4):
            call()
        torch.cuda.synchronize()


MALL_BYTES = 256 << 20          # MI355X Infinity Cache (last-level, shared by the XCDs)


def rotation_sets(step_bytes):
    """Input sets a timed region cycles through, so that between two steps on the same
    set at least twice the MALL's capacity of other inputs has been read: no step
    finds its inputs left in the last-level cache by the step before it."""
    return int(min(8, max(2, 1 + math.ceil(2 * MALL_BYTES / max(step_bytes, 1)))))


def make_sets(generate, wl, n, first=None):
    """n seeded input sets of workload wl: set 0 is the canonical seed (`first`,
    when already generated); the others draw new values and a new block order
    for the same decode context lengths, so every timed step has one shape and
    the same algorithmic bytes."""
    s0 = first if first is not None else generate(wl, "cuda")
    lens = (s0.q_pos.to("cpu").long() + 1).tolist() if wl.mode == "decode" else None
    return [s0] + [generate(wl, "cuda", seed=wl.seed + 7919 * j, lengths=lens) for j in range(1, n)]


def time_forward(B, torch, inps, steps, warmup, settle_ms=0, preps=None):
    """Step time and stage times of dsa_forward, cycling through the input sets
    `inps` (step i uses set i mod len(inps)); `preps[j]` is work upstream of the
    forward on set j that belongs to the step."""
    inps = inps if isinstance(inps, (list, tuple)) else [inps]
    inp0 = inps[0]
    pbs = [B.problem_from_inputs(x) for x in inps]
    ws = torch.empty(max(B.workspace_size(B.OP_FORWARD, pb) for pb in pbs), dtype=torch.uint8, device="cuda")
    T, H, Dv, k = inp0.num_q, inp0.wl.heads, inp0.wl.v_dim, inp0.topk
    out = torch.empty((T, H, Dv), dtype=inp0.q.dtype, device="cuda")
    lse = torch.empty((T, H), dtype=torch.float32, device="cuda")
    idx = torch.empty((T, k), dtype=torch.int32, device="cuda")

    def call(i=0, ev=None):
        j = i % len(inps)
        x = inps[j]
        if preps is not None and preps[j] is not None:    # work upstream of the forward that belongs to the step
            preps[j]()
        B.forward(pbs[j], x.q_idx, x.q_scale, x.w, x.k_cache, x.k_scale, x.q, x.kv_cache, x.sm_scale, out=out,
                  lse=lse, topk_idx=idx, ws=ws, stage_events=ev)

    n_settle = [0]

    def settle_call():
        call(n_settle[0])
        n_settle[0] += 1

    settle(torch, settle_call, settle_ms)
    for i in range(warmup):
        call(i)
    # Timed region 1, the step time: K steps back to back, nothing recorded in between.
    start, end = make_events(torch, 2)
    torch.cuda.synchronize()
    start.record()
    for i in range(steps):
        call(i)
    end.record()
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(end)
    # Timed region 2, the stages: the same K steps with HIP events recorded by the
    # library on its stream between the kernels (indexer | top-k | attention).
    # Each event record costs a few microseconds, which is why region 1 has none.
    stage = [make_events(torch, 4) for _ in range(steps)]
    torch.cuda.synchronize()
    for i in range(steps):
        call(i, stage[i])
    torch.cuda.synchronize()
    st = [[stage[i][j].elapsed_time(stage[i][j + 1]) for j in range(3)] for i in range(steps)]
    mean = [sum(s[j] for s in st) / steps for j in range(3)]
    return total_ms / steps, mean


def decode_stage_rooflines(inp, stages):
    """Achieved HBM GB/s of the decode stages against 8 TB/s: the indexer on its key
    scan (+ q_I, w), the attention on the selected latent rows (+ q, out); the top-k
    on the fp32 score rows it reads (overhead of the path, not algorithmic bytes)."""
    wl = inp.wl
    n = inp.q_pos.to("cpu").long() + 1
    T = inp.num_q
    idx_b, _ = algorithmic_bytes(inp)
    rows = int(n.clamp(max=wl.topk).sum())
    e = ELEM[wl.mla_dtype]
    att_b = rows * wl.qk_dim * e + T * wl.heads * (wl.qk_dim + wl.v_dim) * e
    sc_b = int(n.sum()) * 4
    gbs = lambda b, ms: b / (ms * 1e-3) / 1e9
    return {"indexer": {"bytes": idx_b, "gbs": round(gbs(idx_b, stages[0]), 1),
                        "frac": round(gbs(idx_b, stages[0]) / HBM_PEAK_GBS, 4)},
            "attention_gather": {"bytes": att_b, "rows": rows, "gbs": round(gbs(att_b, stages[2]), 1),
                                 "frac": round(gbs(att_b, stages[2]) / HBM_PEAK_GBS, 4)},
            "topk_select": {"score_bytes_read": sc_b, "gbs": round(gbs(sc_b, stages[1]), 1),
                            "frac": round(gbs(sc_b, stages[1]) / HBM_PEAK_GBS, 4)}}


def env_info():
    """Host and software the numbers were taken on (read before the GPU is touched)."""
    import platform
    info = {"cpu_count": os.cpu_count(), "cpu_model": None, "rocm": None, "hipcc": None,
            "python": platform.python_version()}
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    info["cpu_model"] = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        with open("/opt/rocm/.info/version") as f:
            info["rocm"] = f.read().strip()
    except OSError:
        pass
    try:
        # recorded by the library's build (no child process here: under a profiler the
        # GPU is initialised before this program starts)
        with open(KERNEL_ISA_FILE) as f:
            info["hipcc"] = json.load(f).get("hipcc_version")
    except (OSError, ValueError):
        pass
    return info


def fused_prefill_stages(B, torch, pin, settle_ms, reps=2):
    """The stages of a prefill dsa_forward as the call runs them: one call per query
    chunk of the full call (dsa_forward_chunk_rows), each bracketed by its stage
    events, summed over the chunks ([indexer, top-k, attention] ms).  Unlike the
    standalone ops, the fused path writes no -inf over the masked upper triangle
    and keeps a chunk's scores in its workspace."""
    pb = B.problem_from_inputs(pin)
    piece = B.forward_chunk_rows(pb)
    T = pin.num_q
    fws = torch.empty(B.workspace_size(B.OP_FORWARD, pb), dtype=torch.uint8, device="cuda")
    pout = torch.empty((T, pin.wl.heads, pin.wl.v_dim), dtype=pin.q.dtype, device="cuda")
    pidx = torch.empty((T, pin.topk), dtype=torch.int32, device="cuda")
    pieces = []
    for c0 in range(0, T, piece):
        c1 = min(T, c0 + piece)
        pbc = B.make_problem(mode="prefill", q_pos=pin.q_pos[c0:c1], max_ctx=pin.max_ctx, num_seqs=pin.num_seqs,
                             block_table=pin.block_table, num_blocks=pin.num_blocks, max_seq_len=pin.max_seq_len,
                             index_heads=pin.wl.index_heads, index_dim=pin.wl.index_dim, topk=pin.topk,
                             heads=pin.wl.heads, qk_dim=pin.wl.qk_dim, v_dim=pin.wl.v_dim,
                             index_dtype=B.dtype_code(pin.q_idx), mla_dtype=B.dtype_code(pin.q))
        pieces.append((pbc, c0, c1))
    run_piece = lambda pbc, c0, c1, ev=None: B.forward(
        pbc, pin.q_idx[c0:c1], None if pin.q_scale is None else pin.q_scale[c0:c1], pin.w[c0:c1], pin.k_cache,
        pin.k_scale, pin.q[c0:c1], pin.kv_cache, pin.sm_scale, out=pout[c0:c1], topk_idx=pidx[c0:c1],
        want_lse=False, ws=fws, stage_events=ev)
    settle(torch, lambda: [run_piece(*pc) for pc in pieces], settle_ms)
    fused = [0.0, 0.0, 0.0]
    for _ in range(reps):
        evs = [make_events(torch, 4) for _ in pieces]
        torch.cuda.synchronize()
        for pc, ev in zip(pieces, evs):
            run_piece(*pc, ev=ev)
        torch.cuda.synchronize()
        for ev in evs:
            for j in range(3):
                fused[j] += ev[j].elapsed_time(ev[j + 1]) / reps
    del fws, pout, pidx
    return fused


def measured_ceilings(B, torch):
    """Ceilings measured next to the vendor peaks: streaming reads (a reduction over
    4 GiB, and the library's read-only kernel with the decode indexer's tiling over
    the same 4 GiB, contiguous and as scattered 16 KB blocks), a device copy and a
    large bf16 GEMM (8192^3)."""
    x = torch.ones(1 << 30, dtype=torch.float32, device="cuda")
    a = torch.randn((8192, 8192), device="cuda").to(torch.bfloat16)
    b = torch.randn((8192, 8192), device="cuda").to(torch.bfloat16)
    y = torch.empty_like(x)
    sink = torch.empty(x.numel() * 4 // 131072, dtype=torch.int32, device="cuda")
    read_ms = time_op(torch, lambda: x.sum(), 10, 3, 100)
    shape_ms = time_op(torch, lambda: B.read_ceiling(x, False, sink), 10, 3, 100)
    paged_ms = time_op(torch, lambda: B.read_ceiling(x, True, sink), 10, 3, 100)
    cached_ms = time_op(torch, lambda: B.read_ceiling(x, False, sink, cached=True), 10, 3, 100)
    cached_paged_ms = time_op(torch, lambda: B.read_ceiling(x, True, sink, cached=True), 10, 3, 100)
    copy_ms = time_op(torch, lambda: y.copy_(x), 10, 3, 100)
    gemm_ms = time_op(torch, lambda: torch.matmul(a, b), 10, 3, 200)
    gbs = lambda nbytes, ms: nbytes / (ms * 1e-3) / 1e9
    nb = x.numel() * 4
    res = {"hbm_copy_gbs": round(gbs(2 * nb, copy_ms), 1),
           "hbm_copy_frac_of_spec": round(gbs(2 * nb, copy_ms) / HBM_PEAK_GBS, 4),
           "hbm_reduce_read_gbs": round(gbs(nb, read_ms), 1),
           "indexer_shape_read_gbs": round(gbs(nb, shape_ms), 1),
           "indexer_shape_paged_read_gbs": round(gbs(nb, paged_ms), 1),
           "indexer_shape_paged_read_frac_of_spec": round(gbs(nb, paged_ms) / HBM_PEAK_GBS, 4),
           "indexer_shape_cached_loads_read_gbs": round(gbs(nb, cached_ms), 1),
           "indexer_shape_cached_loads_paged_read_gbs": round(gbs(nb, cached_paged_ms), 1),
           "bf16_gemm_tflops": round(2 * 8192 ** 3 / (gemm_ms * 1e-3) / 1e12, 1),
           "bf16_gemm_frac_of_spec": round(2 * 8192 ** 3 / (gemm_ms * 1e-3) / 1e12 / MFMA_PEAK_TFLOPS["bf16"], 4),
           "how": "device copy of 4 GiB (read + write bytes); torch sum over the same 4 GiB; dsa_read_ceiling over "
                  "the same 4 GiB (the decode indexer's tiling with no arithmetic: 8 KB tiles, two in flight per "
                  "wave, streaming loads as the indexer issues them, or default-policy loads (cached_loads); "
                  "paged = 16 KB blocks in a scattered order); torch.matmul of two 8192x8192 bf16 matrices"}
    del sink
    del x, y, a, b
    torch.cuda.empty_cache()
    return res


def fp8_index_quality(B, torch, inp):
    """The e4m3fn indexer against the bf16 one on the same data (reported, not
    gated): q_I and k_I of a bf16 workload quantised per token with
    dsa_quantize_fp8, then scores and top-k of both compared."""
    T, HI, DI = inp.q_idx.shape
    pb16 = B.problem_from_inputs(inp)
    s16 = B.index_scores(pb16, inp.q_idx, None, inp.w, inp.k_cache, None)
    i16 = B.topk(pb16, s16)
    q8, qs = B.quantize_fp8(inp.q_idx.reshape(T, HI * DI), scale_repeat=HI)
    k8, ks = B.quantize_fp8(inp.k_cache.reshape(-1, DI))
    pb8 = B.make_problem(mode=inp.mode, q_pos=inp.q_pos, max_ctx=inp.max_ctx, num_seqs=inp.num_seqs,
                         block_table=inp.block_table, num_blocks=inp.num_blocks, max_seq_len=inp.max_seq_len,
                         index_heads=HI, index_dim=DI, topk=inp.topk, index_dtype=B.FP8_E4M3FN)
    s8 = B.index_scores(pb8, q8.view(T, HI, DI).view(torch.float8_e4m3fn), qs.view(T, HI), inp.w,
                        k8.view(inp.k_cache.shape).view(torch.float8_e4m3fn), ks.view(inp.k_cache.shape[:-1]))
    i8 = B.topk(pb8, s8)
    torch.cuda.synchronize()
    n = (inp.q_pos.long() + 1)
    valid = torch.arange(s16.shape[1], device="cuda")[None, :] < n[:, None]
    rel = ((s8 - s16).abs() / s16.abs().clamp_min(1e-30))[valid]
    recall = []
    for r in range(T):
        a, b = i16[r], i8[r]
        a, b = a[a >= 0], b[b >= 0]
        recall.append(torch.isin(b, a).float().mean().item() if a.numel() else 1.0)
    return {"workload": inp.wl.name, "score_rel_err_median": round(rel.median().item(), 5),
            "score_rel_err_p99": round(torch.quantile(rel[::max(1, rel.numel() // 1000000)].float(), 0.99).item(), 5),
            "topk_recall_mean": round(sum(recall) / len(recall), 4), "topk_recall_min": round(min(recall), 4),
            "how": "per-token amax/448 scales (dsa_quantize_fp8), e4m3fn indexer vs the bf16 indexer on the same "
                   "bf16 data; recall = share of the fp8 selection inside the bf16 selection"}


def time_op(torch, op, steps, warmup, settle_ms):
    """Mean ms of `op` over `steps` back-to-back calls after a settle and `warmup` calls."""
    settle(torch, op, settle_ms)
    for _ in range(warmup):
        op()
    e0, e1 = make_events(torch, 2)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(steps):
        op()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def dense_line(B, torch, inp, dsa_ms, steps, warmup, settle_ms):
    """Dense MLA over every candidate (dsa_dense_mla: no indexer, no selection) on the
    same inputs, against the DSA step time `dsa_ms`."""
    wl = inp.wl
    pb = B.problem_from_inputs(inp)
    ws = torch.empty(max(1, B.workspace_size(B.OP_DENSE_MLA, pb)), dtype=torch.uint8, device="cuda")
    T = inp.num_q
    out = torch.empty((T, wl.heads, wl.v_dim), dtype=inp.q.dtype, device="cuda")
    lse = torch.empty((T, wl.heads), dtype=torch.float32, device="cuda")
    op = lambda: B.dense_mla(pb, inp.sm_scale, inp.q, inp.kv_cache, out=out, lse=lse, ws=ws)
    ms = time_op(torch, op, steps, warmup, settle_ms)
    n_total = int((inp.q_pos.to("cpu").long() + 1).sum())
    e = ELEM[wl.mla_dtype]
    flops = n_total * wl.heads * 2 * (wl.qk_dim + wl.v_dim)
    nbytes = n_total * wl.qk_dim * e + T * wl.heads * (wl.qk_dim + wl.v_dim) * e
    del ws, out, lse
    return {"dense_mla_ms": round(ms, 4), "dsa_step_ms": round(dsa_ms, 4), "dense_over_dsa": round(ms / dsa_ms, 3),
            "dense_tokens_per_s": round(T / (ms * 1e-3), 1), "dense_rows": n_total,
            "dense_mfma_frac": round(flops / (ms * 1e-3) / 1e12 / MFMA_PEAK_TFLOPS[wl.mla_dtype], 4),
            "dense_hbm_frac": round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}


def warmup_objective_line(B, torch, inp, steps, settle_ms):
    """The indexer's warm-up objective (dsa_indexer_kl_loss with the backward) on
    the prefill inputs: step time, stage times and their matrix-core fractions."""
    wl = inp.wl
    pb = B.problem_from_inputs(inp)
    ws = torch.empty(B.workspace_size(B.OP_INDEXER_KL_LOSS, pb), dtype=torch.uint8, device="cuda")
    T = inp.num_q
    loss = torch.empty(T, dtype=torch.float32, device="cuda")
    dq = torch.empty((T, wl.index_heads, wl.index_dim), dtype=torch.float32, device="cuda")
    dw = torch.empty((T, wl.index_heads), dtype=torch.float32, device="cuda")
    dk = torch.zeros(tuple(inp.k_cache.shape), dtype=torch.float32, device="cuda")
    # The frozen dense attention of the warm-up runs anyway and returns each head's
    # log-sum-exp; the objective's target then needs one pass over the rows.
    _, lse = B.dense_mla(pb, inp.sm_scale, inp.q, inp.kv_cache)
    call = lambda ev=None, given=True: B.indexer_kl_loss(pb, inp.q_idx, inp.w, inp.k_cache, inp.q, inp.kv_cache,
                                                         inp.sm_scale, lse=lse if given else None, loss=loss, dq=dq,
                                                         dw=dw, dk=dk, ws=ws, stage_events=ev)
    ms = time_op(torch, call, steps, 1, settle_ms)
    ms_self = time_op(torch, lambda: call(given=False), steps, 1, 0)
    evs = [make_events(torch, 5) for _ in range(steps)]
    torch.cuda.synchronize()
    for i in range(steps):
        call(evs[i])
    torch.cuda.synchronize()
    st = [sum(evs[i][j].elapsed_time(evs[i][j + 1]) for i in range(steps)) / steps for j in range(4)]
    pairs = int((inp.q_pos.to("cpu").long() + 1).sum())
    peak = MFMA_PEAK_TFLOPS["bf16"]
    f_probs = pairs * wl.heads * 2 * wl.qk_dim                     # the logits of the weights pass
    f_scores = pairs * wl.index_heads * 2 * wl.index_dim
    f_bwd = 4 * pairs * wl.index_heads * 2 * wl.index_dim           # q.k again and the dq product; the same for dk
    kl_bytes = T * ((inp.max_ctx + 63) // 64 * 64) * 4 * 3
    frac = lambda f, t: round(f / (t * 1e-3) / 1e12 / peak, 4)
    del ws, loss, dq, dw, dk, lse
    return {"workload": wl.name,
            "step": "dsa_indexer_kl_loss (target from the dense attention's lse, scores, KL, backward)",
            "ms_per_step": round(ms, 3), "queries_per_s": round(T / (ms * 1e-3), 1),
            "self_contained_ms_per_step": round(ms_self, 3),
            "stages_ms": {"target_probs": round(st[0], 3), "scores": round(st[1], 3), "kl_rows": round(st[2], 3),
                          "backward": round(st[3], 3)},
            "mfma_frac": {"target_probs": frac(f_probs, st[0]), "scores": frac(f_scores, st[1]),
                          "backward": frac(f_bwd, st[3])},
            "kl_rows_hbm_frac": round(kl_bytes / (st[2] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "step_mfma_frac": frac(f_probs + f_scores + f_bwd, ms)}


def stage2_line(B, torch, inp, steps, settle_ms):
    """Stage 2 of training on the prefill inputs: the sparse forward (selection,
    output, lse), the indexer scores, the attention backward (dq, the cache rows'
    gradients, the indexer's target over the selection), the KL on the selection
    and the indexer backward.  Step time, stage times and matrix-core fractions."""
    wl = inp.wl
    pb = B.problem_from_inputs(inp)
    T, H, D, Dv, k = inp.num_q, wl.heads, wl.qk_dim, wl.v_dim, inp.topk
    fws = torch.empty(B.workspace_size(B.OP_FORWARD, pb), dtype=torch.uint8, device="cuda")
    bws = torch.empty(B.workspace_size(B.OP_SPARSE_MLA_BACKWARD, pb), dtype=torch.uint8, device="cuda")
    iws = torch.empty(max(1, B.workspace_size(B.OP_INDEXER_BACKWARD, pb)), dtype=torch.uint8, device="cuda")
    out = torch.empty((T, H, Dv), dtype=inp.q.dtype, device="cuda")
    lse = torch.empty((T, H), dtype=torch.float32, device="cuda")
    idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
    scores = torch.empty((T, (inp.max_ctx + 63) // 64 * 64), dtype=torch.float32, device="cuda")
    dq = torch.empty((T, H, D), dtype=torch.float32, device="cuda")
    dkv = torch.zeros(tuple(inp.kv_cache.shape[:-1]) + (D,), dtype=torch.float32, device="cuda")
    probs = torch.empty((T, k), dtype=torch.float32, device="cuda")
    loss = torch.empty(T, dtype=torch.float32, device="cuda")
    dqi = torch.empty((T, wl.index_heads, wl.index_dim), dtype=torch.float32, device="cuda")
    dwi = torch.empty((T, wl.index_heads), dtype=torch.float32, device="cuda")
    dki = torch.zeros(tuple(inp.k_cache.shape), dtype=torch.float32, device="cuda")
    g = torch.Generator(device="cuda").manual_seed(77)
    dout = (torch.randn((T, H, Dv), device="cuda", generator=g) * 0.05).to(torch.bfloat16)

    def call(ev=None):
        mark = (lambda i: ev[i].record()) if ev is not None else (lambda i: None)
        mark(0)
        B.forward(pb, inp.q_idx, inp.q_scale, inp.w, inp.k_cache, inp.k_scale, inp.q, inp.kv_cache, inp.sm_scale,
                  out=out, lse=lse, topk_idx=idx, ws=fws)
        mark(1)
        B.index_scores(pb, inp.q_idx, inp.q_scale, inp.w, inp.k_cache, inp.k_scale, scores=scores,
                       ld=scores.shape[1])
        mark(2)
        B.sparse_mla_backward(pb, inp.sm_scale, inp.q, inp.kv_cache, idx, out, lse, dout, dq=dq, dkv=dkv,
                              probs=probs, ws=bws)
        mark(3)
        B.sparse_indexer_kl(pb, scores, idx, probs, loss=loss)
        mark(4)
        B.indexer_backward_selected(pb, inp.q_idx, inp.w, inp.k_cache, scores, idx, dq=dqi, dw=dwi, dk=dki,
                                    ws=iws)
        mark(5)

    ms = time_op(torch, call, steps, 1, settle_ms)
    evs = [make_events(torch, 6) for _ in range(steps)]
    torch.cuda.synchronize()
    for i in range(steps):
        call(evs[i])
    torch.cuda.synchronize()
    st = [sum(evs[i][j].elapsed_time(evs[i][j + 1]) for i in range(steps)) / steps for j in range(5)]
    n = inp.q_pos.to("cpu").long() + 1
    pairs = int(n.sum())
    sel = int(n.clamp(max=k).sum())
    f_idx = pairs * wl.index_heads * 2 * wl.index_dim
    f_fwd = f_idx + sel * H * 2 * (D + Dv)
    # per selected (query, row): the logits again, dP, dq, and the row's key and value gradients
    f_bwd = sel * H * 2 * (D + Dv + D + Dv + D)
    # dq, dw over the selected pairs (two products each), dk over every causal pair (two products)
    f_ibwd = 2 * f_idx + 2 * sel * wl.index_heads * 2 * wl.index_dim
    peak = MFMA_PEAK_TFLOPS["bf16"]
    frac = lambda f, t: round(f / (t * 1e-3) / 1e12 / peak, 4)
    contrib_bytes = 2 * sel * D * 2
    del fws, bws, iws, out, lse, idx, scores, dq, dkv, probs, loss, dqi, dwi, dki, dout
    torch.cuda.empty_cache()
    return {"workload": wl.name,
            "step": "dsa_forward + dsa_index_scores + dsa_sparse_mla_backward + dsa_sparse_indexer_kl + "
                    "dsa_indexer_backward_selected",
            "ms_per_step": round(ms, 3), "tokens_per_s": round(T / (ms * 1e-3), 1),
            "stages_ms": {"forward": round(st[0], 3), "index_scores": round(st[1], 3),
                          "attention_backward": round(st[2], 3), "sparse_kl": round(st[3], 3),
                          "indexer_backward": round(st[4], 3)},
            "mfma_frac": {"forward": frac(f_fwd, st[0]), "attention_backward": frac(f_bwd, st[2]),
                          "indexer_backward": frac(f_ibwd, st[4])},
            "attention_backward_row_gradient_bytes": contrib_bytes,
            "note": "the attention backward's cache-row gradients make one bf16 round trip through HBM "
                    "(written per selected row, summed in fp32 per token in query order)"}


def cpu_baseline(inp, seconds):
    """The float64 oracle, as it stands, on the queries of the timed batch, for a bounded time."""
    import numpy as np
    import oracle
    from workloads import raw_numpy, dtype_tag
    oi = oracle.OracleInputs(
        mode=inp.mode, q_pos=raw_numpy(inp.q_pos).astype(np.int64),
        block_table=None if inp.block_table is None else raw_numpy(inp.block_table).astype(np.int64),
        block_size=inp.block_size, index_dtype=dtype_tag(inp.q_idx), q_idx=raw_numpy(inp.q_idx),
        q_scale=raw_numpy(inp.q_scale), w=raw_numpy(inp.w), k_cache=raw_numpy(inp.k_cache),
        k_scale=raw_numpy(inp.k_scale), mla_dtype=dtype_tag(inp.q), q=raw_numpy(inp.q),
        kv_cache=raw_numpy(inp.kv_cache), topk=inp.topk, sm_scale=inp.sm_scale, v_dim=inp.wl.v_dim)
    threads = None
    try:
        from threadpoolctl import threadpool_info
        threads = max((p.get("num_threads", 1) for p in threadpool_info()), default=1)
    except Exception:
        pass
    # Cycle over the batch's queries until `seconds` of CPU work have run (the
    # oracle keeps no state between queries, so a repeated query costs the same).
    done = 0
    t0 = time.perf_counter()
    while True:
        oracle.forward(oi, rows=[done % inp.num_q])
        done += 1
        if time.perf_counter() - t0 >= seconds:
            break
    el = time.perf_counter() - t0
    passes = done / inp.num_q
    return {"value": done / el, "unit": "tokens/s", "cores": threads or os.cpu_count(), "kind": "oracle",
            "host_cpu_count": os.cpu_count(),
            "sample": f"{done} decode queries ({passes:.1f} passes over the {inp.num_q} queries of the timed "
                      f"batch; full indexer over each context, top-k, attention), float64 NumPy with "
                      f"{threads or os.cpu_count()} BLAS threads on a host of {os.cpu_count()} CPUs, {el:.1f} s wall"}


def prefill_line(B, torch, generate, wl, settle_ms, rotate, dense=False, warmup_objective=False, steps=3,
                 stage2=False):
    """One prefill workload: the fused step (input sets rotated), each op alone over
    every query row, the stages as the fused call runs them, and their matrix-core
    fractions (indexer against its own dtype's peak, attention against bf16)."""
    log(f"prefill: {wl.name}")
    pins = make_sets(generate, wl, rotate)
    pin = pins[0]
    pms, _ = time_forward(B, torch, pins, steps, 1, settle_ms)
    pf_idx, pf_mla = algorithmic_flops(pin)
    idx_peak = MFMA_PEAK_TFLOPS[wl.index_dtype]
    mla_peak = MFMA_PEAK_TFLOPS[wl.mla_dtype]
    # each stage alone over every query row, one call each (the forward processes
    # the rows in query chunks; its stage events cover the first chunk only)
    pb = B.problem_from_inputs(pin)
    sc = torch.empty((pin.num_q, pin.max_ctx), dtype=torch.float32, device="cuda")
    idx = torch.empty((pin.num_q, pin.topk), dtype=torch.int32, device="cuda")
    tws = torch.empty(B.workspace_size(B.OP_TOPK, pb), dtype=torch.uint8, device="cuda")
    mws = torch.empty(max(1, B.workspace_size(B.OP_SPARSE_MLA, pb)), dtype=torch.uint8, device="cuda")
    ops = [lambda: B.index_scores(pb, pin.q_idx, pin.q_scale, pin.w, pin.k_cache, pin.k_scale, scores=sc),
           lambda: B.topk(pb, sc, idx=idx, ws=tws),
           lambda: B.sparse_mla(pb, pin.sm_scale, pin.q, pin.kv_cache, idx, ws=mws)]
    stage_ms = []
    for op in ops:
        settle(torch, op, settle_ms / 2)
        e0, e1 = make_events(torch, 2)
        e0.record()
        for _ in range(3):
            op()
        e1.record()
        torch.cuda.synchronize()
        stage_ms.append(e0.elapsed_time(e1) / 3)
    fused = fused_prefill_stages(B, torch, pin, settle_ms / 2)
    planted = None
    if pin.planted is not None:
        # share of planted keys among the selected positions of the rows that
        # select (n > k), against their share among those rows' candidates
        mark = torch.zeros(pin.max_ctx, dtype=torch.bool, device="cuda")
        mark[pin.planted] = True
        rows_sel = (pin.q_pos.long() + 1) > pin.topk
        sel = idx[rows_sel]
        cum = torch.cumsum(mark.long(), 0)
        planted = {"share_in_topk": round(mark[sel.long()].float().mean().item(), 4),
                   "share_in_candidates": round((cum[pin.q_pos.long()[rows_sel]].float() /
                                                 (pin.q_pos.long()[rows_sel] + 1).float()).mean().item(), 4)}
    tf = lambda f, ms, peak: round(f / (ms * 1e-3) / 1e12 / peak, 4)
    line = {
        "workload": wl.name, "index_dtype": wl.index_dtype, "tokens_per_s": round(pin.num_q / (pms * 1e-3), 1),
        "ms_per_step": round(pms, 3), "input_sets_rotated": len(pins),
        "stage_ops_ms_all_rows": {"index_scores": round(stage_ms[0], 3), "topk": round(stage_ms[1], 3),
                                  "sparse_mla": round(stage_ms[2], 3)},
        "fused_stages_ms": {"indexer": round(fused[0], 3), "topk": round(fused[1], 3), "attention": round(fused[2], 3)},
        "indexer_peak_tflops": idx_peak,
        "indexer_mfma_frac_fused": tf(pf_idx, fused[0], idx_peak),
        "attention_mfma_frac_fused": tf(pf_mla, fused[2], mla_peak),
        "indexer_mfma_frac": tf(pf_idx, stage_ms[0], idx_peak),
        "attention_mfma_frac": tf(pf_mla, stage_ms[2], mla_peak),
        "step_mfma_time_frac": round((pf_idx / (idx_peak * 1e12) + pf_mla / (mla_peak * 1e12)) / (pms * 1e-3), 4),
        "planted_keys": planted}
    log(f"prefill {wl.name}: {pms:.2f} ms/step, indexer {stage_ms[0]:.2f} ms alone, {fused[0]:.2f} ms fused")
    del sc, idx, tws, mws, pins
    torch.cuda.empty_cache()
    extra = {}
    if dense:
        extra["dense"] = dense_line(B, torch, pin, pms, 2, 1, settle_ms)
    if warmup_objective:
        log("indexer warm-up objective on the prefill inputs")
        extra["warmup_objective"] = warmup_objective_line(B, torch, pin, 2, settle_ms)
        log(f"warm-up objective: {extra['warmup_objective']['ms_per_step']:.2f} ms")
    if stage2:
        log("stage-2 sparse training step on the prefill inputs")
        extra["sparse_training"] = stage2_line(B, torch, pin, 2, settle_ms)
        log(f"stage-2 step: {extra['sparse_training']['ms_per_step']:.2f} ms")
    return line, extra


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default=None)
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--settle-ms", type=float, default=400.0,
                    help="untimed run-in before each timed region, so the shader clock has settled")
    ap.add_argument("--rotate", type=int, default=0,
                    help="input sets each timed region cycles through (0: enough that no step finds its inputs "
                         "left in the 256 MB MALL by an earlier step)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true", help="skip the secondary prefill measurements")
    ap.add_argument("--no-prefill-64k", action="store_true", help="skip the 64K prefill with the e4m3fn indexer")
    ap.add_argument("--no-fp8-decode", action="store_true", help="skip the secondary fp8-indexer decode measurement")
    ap.add_argument("--fp8-workload", default="decode_128k_paged_fp8")
    ap.add_argument("--no-exact-decode", action="store_true",
                    help="skip the secondary decode line with every context exactly 128K tokens")
    ap.add_argument("--exact-workload", default="decode_128k_exact_paged_bf16")
    ap.add_argument("--no-8k-decode", action="store_true", help="skip the 16 x 8K contiguous decode line")
    ap.add_argument("--no-dense", action="store_true",
                    help="skip the dense-MLA comparison (attention over every candidate) on the same inputs")
    ap.add_argument("--no-warmup-objective", action="store_true",
                    help="skip the indexer warm-up objective (loss and backward) on the prefill inputs")
    ap.add_argument("--no-stage2", action="store_true",
                    help="skip the Stage-2 sparse training step (forward, attention and indexer backward)")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the measured ceilings and the fp8 indexing-quality report")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="also run one plain device copy of this many MiB (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the path is data-parallel across sequences; sharding is described, not built)", file=sys.stderr)
        sys.exit(2)

    env = env_info()
    import torch
    from sparse_long_context_relu_amd import binding as B
    from workloads import WORKLOADS, BENCH_DEFAULT, generate
    env["torch"] = torch.__version__
    env["hip_runtime"] = getattr(torch.version, "hip", None)

    if args.copy_mib:
        # a plain copy of known size: its FETCH_SIZE / WRITE_SIZE calibrate the traffic counters
        src = torch.ones(args.copy_mib << 18, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"calibration copy: {args.copy_mib} MiB read + {args.copy_mib} MiB written")
        del src, dst
    env["gpu"] = torch.cuda.get_device_name(0)
    n_sets = lambda wl_inp: args.rotate if args.rotate > 0 else rotation_sets(algorithmic_bytes(wl_inp)[1])
    name = args.workload or BENCH_DEFAULT
    wl = WORKLOADS[name]
    log(f"generating {name} on cuda:0")
    inp = generate(wl, "cuda")
    sets = make_sets(generate, wl, n_sets(inp), first=inp)
    torch.cuda.synchronize()
    log(f"timing {args.steps} steps after {args.warmup} warm-up steps, cycling {len(sets)} input sets")
    ms, stages = time_forward(B, torch, sets, args.steps, args.warmup, args.settle_ms)
    del sets
    tokens = inp.num_q
    value = tokens / (ms * 1e-3)
    idx_bytes, step_bytes = algorithmic_bytes(inp)
    idx_flops, mla_flops = algorithmic_flops(inp)
    log(f"{ms:.3f} ms/step; stages (indexer, top-k, attention) ms = {[round(s, 4) for s in stages]}")

    if wl.mode == "decode":
        achieved = idx_bytes / (stages[0] * 1e-3) / 1e9
        roof = {"bound": "hbm", "kernel": "indexer_decode_kernel", "achieved": round(achieved, 1),
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": measured_traffic("indexer_decode_kernel", name), "bytes_per_launch": idx_bytes,
                "launch_ms": round(stages[0], 5)}
    else:
        # the step's stage events cover its first query chunk; the indexer's time
        # over every chunk comes from one call per chunk
        stages = fused_prefill_stages(B, torch, inp, args.settle_ms / 2)
        achieved = idx_flops / (stages[0] * 1e-3) / 1e12
        peak = MFMA_PEAK_TFLOPS[wl.index_dtype]
        roof = {"bound": "mfma", "kernel": "indexer_prefill_kernel", "achieved": round(achieved, 2),
                "peak": peak, "unit": "TFLOP/s", "frac": round(achieved / peak, 4), "traffic": None,
                "note": "indexer time summed over the query chunks, one dsa_forward per chunk"}

    result = {
        "metric": METRIC, "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "settle_ms": args.settle_ms, "ms_per_step": round(ms, 4), "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None, "dtype": wl.mla_dtype if wl.index_dtype != "fp8" else "bf16+fp8",
        "data": "synthetic (seeded; no dataset or weights)",
        "config": {"workload": name, "mode": wl.mode, "batch": wl.num_seqs,
                   "context": list(wl.length_range) if wl.length_range else wl.length,
                   "context_total": int((inp.q_pos.long() + 1).sum()), "paged": wl.paged, "topk": wl.topk,
                   "index_heads": wl.index_heads, "index_dim": wl.index_dim, "heads": wl.heads,
                   "qk_dim": wl.qk_dim, "v_dim": wl.v_dim, "index_dtype": wl.index_dtype,
                   "parallelism": "single GPU"},
        "roofline": roof,
        "stages_ms": {"indexer": round(stages[0], 4), "topk": round(stages[1], 4), "attention": round(stages[2], 4)},
        "input_sets_rotated": n_sets(inp),
        "step_algorithmic_bytes": step_bytes,
        "step_hbm_frac": round(step_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "env": env,
    }
    if wl.mode == "decode":
        result["stage_rooflines"] = decode_stage_rooflines(inp, stages)

    if wl.mode == "decode" and wl.index_dtype == "bf16" and not args.no_extras:
        log("fp8 indexing quality against bf16 on the same inputs")
        result["fp8_index_quality"] = fp8_index_quality(B, torch, inp)
        torch.cuda.empty_cache()
    dense = {}
    if not args.no_dense:
        log("dense MLA on the same inputs")
        dense[name] = dense_line(B, torch, inp, ms, max(3, args.steps // 4), 1, args.settle_ms)
        log(f"dense: {dense[name]['dense_mla_ms']:.3f} ms ({dense[name]['dense_over_dsa']:.2f}x the DSA step)")

    def decode_line(name, fp8_prep):
        """Another decode workload through the same step, cycling its input sets (for
        e4m3fn indexing: the new tokens' index queries and keys arrive in bf16 and are
        quantised with dsa_quantize_fp8 and appended with dsa_append_index_keys inside
        the step)."""
        log(f"secondary: {name}")
        din = generate(WORKLOADS[name], "cuda")
        dsets = make_sets(generate, WORKLOADS[name], n_sets(din), first=din)
        T, HI, DI = din.num_q, din.wl.index_heads, din.wl.index_dim
        preps, extra = None, 0
        if fp8_prep:
            g = torch.Generator(device="cuda").manual_seed(1234)
            q_new = torch.randn((T, HI * DI), device="cuda", generator=g).to(torch.bfloat16)
            k_new = torch.randn((T, DI), device="cuda", generator=g).to(torch.bfloat16)

            def prep_for(x):
                dpb = B.problem_from_inputs(x)
                q8 = x.q_idx.view(T, HI * DI)

                def prep():
                    B.quantize_fp8(q_new, scale_repeat=HI, dst=q8, scale=x.q_scale)
                    B.append_index_keys(dpb, k_new, x.k_cache, x.k_scale)
                return prep

            preps = [prep_for(x) for x in dsets]
            extra = T * (HI * DI * 3 + HI * 4) + T * (DI * 3 + 4)      # bf16 in, e4m3 + scales out
        dms, dst = time_forward(B, torch, dsets, args.steps, args.warmup, args.settle_ms, preps=preps)
        d_idx, d_step = algorithmic_bytes(din)
        line = {"workload": name, "step": "quantise q_I + append k_I + dsa_forward" if fp8_prep else "dsa_forward",
                "batch": T, "context_total": int((din.q_pos.long() + 1).sum()),
                "tokens_per_s": round(T / (dms * 1e-3), 1), "ms_per_step": round(dms, 4),
                "input_sets_rotated": len(dsets),
                "stages_ms": {"indexer": round(dst[0], 4), "topk": round(dst[1], 4), "attention": round(dst[2], 4)},
                "indexer_bytes_per_launch": d_idx,
                "indexer_hbm_frac": round(d_idx / (dst[0] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                "stage_rooflines": decode_stage_rooflines(din, dst),
                "step_algorithmic_bytes": d_step + extra,
                "step_hbm_frac": round((d_step + extra) / (dms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
        log(f"{name}: {dms:.3f} ms/step, indexer {dst[0]:.4f} ms")
        del dsets
        if not args.no_dense and not fp8_prep:
            dense[name] = dense_line(B, torch, din, dms, max(3, args.steps // 4), 1, args.settle_ms)
        del din
        torch.cuda.empty_cache()
        return line

    if wl.mode == "decode":
        inp = None
        torch.cuda.empty_cache()
        if not args.no_exact_decode:
            # every sequence exactly 128K tokens (the 128K-context headline shape)
            result["exact_128k_decode"] = decode_line(args.exact_workload, False)
        if not args.no_fp8_decode:
            result["fp8_decode"] = decode_line(args.fp8_workload, True)
        if not args.no_8k_decode:
            # 16 sequences of 8K tokens, contiguous caches (small enough for the MALL: rotated)
            result["decode_8k"] = decode_line("decode_8k_bf16", False)

    if not args.no_prefill:
        inp = None
        torch.cuda.empty_cache()
        pwl = WORKLOADS["prefill_16k_bf16"]
        result["prefill"], extra = prefill_line(B, torch, generate, pwl, args.settle_ms, max(2, args.rotate),
                                                dense=not args.no_dense,
                                                warmup_objective=not args.no_warmup_objective,
                                                stage2=not args.no_stage2)
        if "dense" in extra:
            dense[pwl.name] = extra["dense"]
        if "warmup_objective" in extra:
            result["warmup_objective"] = extra["warmup_objective"]
        if "sparse_training" in extra:
            result["sparse_training"] = extra["sparse_training"]
        torch.cuda.empty_cache()
        if not args.no_prefill_64k:
            result["prefill_64k_fp8"], _ = prefill_line(B, torch, generate, WORKLOADS["prefill_64k_fp8"],
                                                        args.settle_ms, max(2, args.rotate))
            torch.cuda.empty_cache()
    if dense:
        # the comparison the pages draw: DSA against dense MLA over the same contexts
        result["dense_comparison"] = dense
    if not args.no_extras:
        inp = None
        torch.cuda.empty_cache()
        log("measured ceilings")
        result["measured_ceilings"] = mc = measured_ceilings(B, torch)
        if result["roofline"].get("bound") == "hbm" and wl.paged:
            # the dominant kernel against the read rate its own access shape reaches with no arithmetic
            result["roofline"]["frac_of_measured_shape_read"] = round(
                result["roofline"]["achieved"] / mc["indexer_shape_paged_read_gbs"], 4)
    if not args.no_cpu_baseline:
        if inp is None:
            inp = generate(wl, "cuda")
        log(f"cpu baseline: oracle for ~{args.cpu_seconds:.0f} s")
        result["cpu_baseline"] = cpu_baseline(inp, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
