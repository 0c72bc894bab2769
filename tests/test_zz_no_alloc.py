"""fx_sparse_decode_noalloc (decode partials in the library's static per-GPU array, no
workspace, no allocation) against fx_sparse_decode (partials in the caller's workspace),
through the C ABI: identical bits, on two calls in a row, the second with a smaller input
than the first (a plan with fewer units, another dtype and head dim)."""
import numpy as np
import pytest
import torch

import block_sparse_decode_summary_amd as fx
from workloads import generate, small_workload

from gpu_harness import INT32_MAX, make_plan, say, softmax_scale

pytestmark = pytest.mark.gpu
DEV = "cuda"
SCRATCH_LIMIT = 8 << 20


def _decode_both(name: str):
    w = small_workload(name)
    say(f"[noalloc] {w.name}: B={w.batch} Hkv={w.num_kv_heads} d={w.head_dim} {w.dtype}")
    inp = generate(w, DEV)
    plan = make_plan(w)
    assert 0 < fx.fx_noalloc_scratch_bytes(plan) <= SCRATCH_LIMIT
    bufs = fx.allocate_step_buffers(plan, DEV)
    fx.fx_build_summaries(plan, inp.K, inp.seq_lens, 0, INT32_MAX, bufs.summaries)
    fx.fx_select(plan, inp.q, bufs.summaries, inp.logits,
                 bufs.evicted_mask if w.has_nosa else None, inp.seq_lens, bufs.sel_idx,
                 bufs.sel_cnt, bufs.workspace)
    scale = softmax_scale(w)
    out_ns = torch.full_like(bufs.out, float("nan"))
    lse_ns = torch.full_like(bufs.lse, float("nan"))
    fx.fx_sparse_decode_noalloc(plan, inp.q, inp.K, inp.V, inp.seq_lens, bufs.sel_idx,
                                bufs.sel_cnt, scale, out_ns, lse_ns)
    fx.fx_sparse_decode(plan, inp.q, inp.K, inp.V, inp.seq_lens, bufs.sel_idx, bufs.sel_cnt,
                        scale, bufs.out, bufs.lse, bufs.workspace)
    torch.cuda.synchronize()
    assert fx.fx_read_error(plan) == 0
    a = bufs.out.view(torch.int16 if w.dtype == "bf16" else torch.int32).cpu().numpy()
    b = out_ns.view(torch.int16 if w.dtype == "bf16" else torch.int32).cpu().numpy()
    assert np.array_equal(a, b), f"{w.name}: out differs"
    assert np.array_equal(bufs.lse.view(torch.int32).cpu().numpy(),
                          lse_ns.view(torch.int32).cpu().numpy()), f"{w.name}: lse differs"
    say(f"[noalloc] {w.name}: identical to fx_sparse_decode "
        f"({fx.fx_noalloc_scratch_bytes(plan)} scratch bytes)")
    return plan


def test_noalloc_decode_equals_workspace_decode_twice():
    # The first call: 48 units of ragged lengths, segments cut units (the merge runs).
    big = _decode_both("mixed_serving")
    # The second, smaller: 2 units, float32, d 64; the array still holds the first call's
    # partials.
    small = _decode_both("tiny")
    assert fx.fx_noalloc_scratch_bytes(small) < fx.fx_noalloc_scratch_bytes(big)


def test_noalloc_decode_validates_like_fx_sparse_decode():
    w = small_workload("tiny")
    plan = make_plan(w)
    bufs = fx.allocate_step_buffers(plan, DEV)
    inp = generate(w, DEV)
    lib = fx.load_library()
    st = lib.fx_sparse_decode_noalloc(plan.handle, inp.q.data_ptr(), inp.K.data_ptr(),
                                      inp.V.data_ptr(), inp.seq_lens.data_ptr(),
                                      bufs.sel_idx.data_ptr(), bufs.sel_cnt.data_ptr(), 0.0,
                                      bufs.out.data_ptr(), None, None)
    assert st == fx.FX_E_INVALID          # softmax_scale must be positive
    st = lib.fx_sparse_decode_noalloc(plan.handle, inp.q.data_ptr() + 4, inp.K.data_ptr(),
                                      inp.V.data_ptr(), inp.seq_lens.data_ptr(),
                                      bufs.sel_idx.data_ptr(), bufs.sel_cnt.data_ptr(), 0.125,
                                      bufs.out.data_ptr(), None, None)
    assert st == fx.FX_E_INVALID          # q not 16-byte aligned
