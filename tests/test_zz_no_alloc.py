"""dsa_forward_noalloc (the library's static scratch in place of a workspace) against
dsa_forward on the same inputs, through the C ABI: the same kernels and layouts, so
the same bytes.  Two calls in a row on one GPU share the scratch; the second, smaller
problem must not see anything the first one left there."""
import pytest
import torch

from tests.test_gpu_ops import B, DEV, _say, big_dims
from workloads import generate

pytestmark = pytest.mark.gpu


def _both(inp):
    pb = B().problem_from_inputs(inp)
    ref = B().forward_inputs(inp)
    T, H, Dv, k = inp.num_q, inp.wl.heads, inp.wl.v_dim, inp.topk
    out = torch.full((T, H, Dv), 7.0, dtype=inp.q.dtype, device=DEV)
    lse = torch.full((T, H), 7.0, dtype=torch.float32, device=DEV)
    idx = torch.full((T, k), 7, dtype=torch.int32, device=DEV)
    B().forward_noalloc(pb, inp.q_idx, inp.q_scale, inp.w, inp.k_cache, inp.k_scale, inp.q, inp.kv_cache,
                        inp.sm_scale, out, lse=lse, topk_idx=idx)
    torch.cuda.synchronize()
    return ref, (out, lse, idx)


CALLS = [
    # a paged decode batch, then a smaller contiguous one on the same scratch
    ("decode_paged", dict(mode="decode", num_seqs=4, length=9000, k=2048, paged=True), [9000, 4097, 2000, 1]),
    ("decode_small", dict(mode="decode", num_seqs=2, length=3000, k=2048), [3000, 2100]),
    # a prefill (one-workgroup-per-row top-k), then a smaller one (sliced top-k, split attention rows)
    ("prefill", dict(mode="prefill", length=2600, k=2048, prefill_q_start=2200), None),
    ("prefill_small_fp8", dict(mode="prefill", length=2300, k=2048, prefill_q_start=2150, index_dtype="fp8"), None),
]


def test_noalloc_equals_forward_on_consecutive_calls():
    for name, kw, lengths in CALLS:
        _say("forward_noalloc", name)
        inp = generate(big_dims(**kw), DEV, lengths=lengths)
        (o1, l1, i1), (o2, l2, i2) = _both(inp)
        assert torch.equal(i1, i2), f"{name}: selection"
        assert torch.equal(o1, o2), f"{name}: out"
        assert torch.equal(l1, l2), f"{name}: lse"
