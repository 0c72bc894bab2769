"""fx_select_delta (selection and its differences in one call) against fx_select followed
by fx_selection_delta, and against the oracle's set differences.

Both paths run side by side with their own state (eviction masks, previous selections);
selections, counts, masks and the added / removed lists must agree bit for bit.
"""
import numpy as np
import pytest
import torch

import block_sparse_decode_summary_amd as fx
from oracle.delta import selection_delta
from workloads import (HeadPolicy, MODE_NOSA, MODE_RETRIEVAL, MODE_STREAMING, WORKLOAD_NAMES,
                       Workload, generate, query_at_step, small_workload)

from gpu_harness import INT32_MAX, make_plan, oracle_unit, say

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _both(w: Workload, steps: int, oracle_units=()):
    say(f"[select_delta] {w.name}: units={w.num_units} t_cap={w.t_cap} steps={steps}")
    inp = generate(w, DEV)
    plan = make_plan(w)
    A = fx.allocate_step_buffers(plan, DEV)     # separate calls
    B = fx.allocate_step_buffers(plan, DEV)     # fused call
    fx.fx_build_summaries(plan, inp.K, inp.seq_lens, 0, INT32_MAX, A.summaries)
    evicted = {u: None for u in oracle_units}
    prev_ref = {u: np.zeros(0, np.int64) for u in oracle_units}
    for t in range(steps):
        q = query_at_step(w, t, DEV) if t > 0 else inp.q
        A.prev_idx.copy_(A.sel_idx)
        A.prev_cnt.copy_(A.sel_cnt)
        fx.fx_select(plan, q, A.summaries, inp.logits, A.evicted_mask if w.has_nosa else None,
                     inp.seq_lens, A.sel_idx, A.sel_cnt, A.workspace)
        fx.fx_selection_delta(plan, A.prev_idx, A.prev_cnt, A.sel_idx, A.sel_cnt, A.added,
                              A.added_cnt, A.removed, A.removed_cnt)
        B.prev_idx.copy_(B.sel_idx)
        B.prev_cnt.copy_(B.sel_cnt)
        fx.fx_select_delta(plan, q, A.summaries, inp.logits,
                           B.evicted_mask if w.has_nosa else None, inp.seq_lens, B.prev_idx,
                           B.prev_cnt, B.sel_idx, B.sel_cnt, B.added, B.added_cnt, B.removed,
                           B.removed_cnt, B.workspace)
        torch.cuda.synchronize()
        for name in ("sel_idx", "sel_cnt", "added", "added_cnt", "removed", "removed_cnt",
                     "evicted_mask"):
            assert torch.equal(getattr(A, name), getattr(B, name)), f"{w.name} step {t}: {name}"
        if oracle_units:
            added, added_cnt = B.added.cpu().numpy(), B.added_cnt.cpu().numpy()
            removed, removed_cnt = B.removed.cpu().numpy(), B.removed_cnt.cpu().numpy()
            for u in oracle_units:
                ref = oracle_unit(inp, u, q, evicted[u])
                evicted[u] = ref.evicted
                a_ref, r_ref = selection_delta(prev_ref[u], ref.sel)
                assert list(added[u, :added_cnt[u]]) == list(a_ref), f"unit {u} step {t}: added"
                assert list(removed[u, :removed_cnt[u]]) == list(r_ref), f"unit {u} step {t}: removed"
                prev_ref[u] = ref.sel
    assert fx.fx_read_error(plan) == 0
    say(f"[select_delta] {w.name}: ok")


@pytest.mark.parametrize("name", WORKLOAD_NAMES)
def test_select_delta_equals_separate_calls(name):
    w = small_workload(name)
    _both(w, steps=min(w.steps, 6), oracle_units=(0, w.num_units - 1))


def test_select_delta_workspace_path():
    """Units with more than 8192 block slots: the selection kernel of the workspace path,
    then the delta kernel."""
    t_cap = 8192 * 16 + 3000
    pol = HeadPolicy(MODE_RETRIEVAL, block=16, sub_block=16, top_k=40, force_sink=1, force_last=1)
    w = Workload(name="select_delta_mem", batch=2, num_q_heads=4, num_kv_heads=2, head_dim=64,
                 dtype="bf16", t_cap=t_cap, seq_lens=(t_cap, 70001), policies=(pol,) * 4, seed=90,
                 sink_scaled_tokens=4, needles_per_head=3, steps=3, drift=(0.9, 0.44))
    _both(w, steps=3)


def test_select_delta_flags_a_bad_previous_selection():
    w = small_workload("qwen7b_layer")
    say("[select_delta] bad previous selection")
    inp = generate(w, DEV)
    plan = make_plan(w)
    B = fx.allocate_step_buffers(plan, DEV)
    fx.fx_build_summaries(plan, inp.K, inp.seq_lens, 0, INT32_MAX, B.summaries)
    fx.fx_select(plan, inp.q, B.summaries, None, None, inp.seq_lens, B.sel_idx, B.sel_cnt,
                 B.workspace)
    B.prev_idx.copy_(B.sel_idx)
    B.prev_cnt.copy_(B.sel_cnt)
    last = int(B.sel_cnt[0].item()) - 1
    B.prev_idx[0, last] = 1 << 30              # not a block of the unit
    fx.fx_select_delta(plan, inp.q, B.summaries, None, None, inp.seq_lens, B.prev_idx,
                       B.prev_cnt, B.sel_idx, B.sel_cnt, B.added, B.added_cnt, B.removed,
                       B.removed_cnt, B.workspace)
    torch.cuda.synchronize()
    assert fx.fx_read_error(plan) == fx.FX_ERR_SEL_INDEX
    cnt = B.added_cnt.cpu().numpy()
    # Same query: nothing changed except unit 0, whose last block now counts as added.
    assert cnt[0] == 1 and B.added[0, 0].item() == B.sel_idx[0, last].item()
    assert np.all(cnt[1:] == 0) and np.all(B.removed_cnt.cpu().numpy() == 0)
    with pytest.raises(fx.FxError):            # previous and current lists must differ
        fx.fx_select_delta(plan, inp.q, B.summaries, None, None, inp.seq_lens, B.sel_idx,
                           B.sel_cnt, B.sel_idx, B.sel_cnt, B.added, B.added_cnt, B.removed,
                           B.removed_cnt, B.workspace)


@pytest.mark.parametrize("n_small", [256, 512])
def test_one_kernel_and_two_kernel_selection_agree(n_small):
    """Units of at most 512 block slots (key-side summaries) take the selection kernel that
    forms the scores itself, with 256 threads up to 256 slots and 512 threads above; 513
    slots take the scoring kernel followed by the selection kernel.  Plans of n_small and
    n_small + 1 block slots (256 / 257: the two fused widths; 512 / 513: fused and two
    kernels) on the same cache, queries and eviction logits give the same scores,
    selections, eviction masks and differences, bit for bit."""
    g = 16
    pols = (HeadPolicy(MODE_RETRIEVAL, block=g, sub_block=g, top_k=12, force_sink=1, force_last=1),
            HeadPolicy(MODE_NOSA, block=g, sub_block=g, top_k=8, k_evict=24),
            HeadPolicy(MODE_STREAMING, block=g, sub_block=g, sink_tokens=16, local_tokens=64),
            HeadPolicy(MODE_RETRIEVAL, block=g, sub_block=g, budget=0.05, force_sink=1,
                       force_last=1))
    wB = Workload(name="one_vs_two_kernels", batch=3, num_q_heads=8, num_kv_heads=4,
                  head_dim=128, dtype="bf16", t_cap=n_small * g + g,
                  seq_lens=(n_small * g, 2000, 3001), policies=pols * 3, seed=91,
                  sink_scaled_tokens=4, needles_per_head=2, steps=4, drift=(0.9, 0.44))
    wA = wB.replace(t_cap=n_small * g)
    say(f"[select one/two kernels] units={wB.num_units} n_cap {n_small} and {n_small + 1}")
    inp = generate(wB, DEV)
    KA = inp.K[:, :, :wA.t_cap].contiguous()
    offA, offB = wA.block_offsets(), wB.block_offsets()
    logitsA = torch.cat([inp.logits[int(offB[u]):int(offB[u]) + wA.n_cap(u)]
                         for u in range(wA.num_units)])
    plans = [make_plan(wA), make_plan(wB)]
    bufs = [fx.allocate_step_buffers(p, DEV) for p in plans]
    fx.fx_build_summaries(plans[0], KA, inp.seq_lens, 0, INT32_MAX, bufs[0].summaries)
    fx.fx_build_summaries(plans[1], inp.K, inp.seq_lens, 0, INT32_MAX, bufs[1].summaries)
    masks = [w.mask_word_offsets() for w in (wA, wB)]
    for t in range(wB.steps):
        q = query_at_step(wB, t, DEV) if t > 0 else inp.q
        for p, X, lg in zip(plans, bufs, (logitsA, inp.logits)):
            X.prev_idx.copy_(X.sel_idx)
            X.prev_cnt.copy_(X.sel_cnt)
            fx.fx_select_delta(p, q, X.summaries, lg, X.evicted_mask, inp.seq_lens, X.prev_idx,
                               X.prev_cnt, X.sel_idx, X.sel_cnt, X.added, X.added_cnt,
                               X.removed, X.removed_cnt, X.workspace)
        torch.cuda.synchronize()
        A, B = bufs
        for u in range(wB.num_units):
            T = wB.seq_lens[u // wB.num_kv_heads]
            n_full = T // g
            for name in ("sel", "added", "removed"):
                idx = getattr(A, "sel_idx" if name == "sel" else name)
                cnt = getattr(A, "sel_cnt" if name == "sel" else name + "_cnt")
                idxB = getattr(B, "sel_idx" if name == "sel" else name)
                cntB = getattr(B, "sel_cnt" if name == "sel" else name + "_cnt")
                c = int(cnt[u])
                assert c == int(cntB[u]), f"step {t} unit {u}: {name} count"
                assert torch.equal(idx[u, :c], idxB[u, :c]), f"step {t} unit {u}: {name}"
            if pols[u % 4].mode != MODE_STREAMING:
                sA = A.workspace[int(offA[u]) * 4:(int(offA[u]) + n_full) * 4].view(torch.int32)
                sB = B.workspace[int(offB[u]) * 4:(int(offB[u]) + n_full) * 4].view(torch.int32)
                assert torch.equal(sA, sB), f"step {t} unit {u}: scores"
            mA = A.evicted_mask[int(masks[0][u]):int(masks[0][u + 1])]
            mB = B.evicted_mask[int(masks[1][u]):int(masks[1][u]) + len(mA)]
            assert torch.equal(mA, mB), f"step {t} unit {u}: eviction mask"
    for p in plans:
        assert fx.fx_read_error(p) == 0
    say("[select one/two kernels] ok")
