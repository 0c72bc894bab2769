"""Every unit of every full-size workload against the oracle (needs an MI355X).

The five workloads at their full sizes, in the launch configuration bench.py times
(default plan, fx_build_summaries over the cache, then fx_select_delta and
fx_sparse_decode as in a bench step).  For every unit: summaries, float32 scores,
selections, -1 padding and the differences bit-exact; out and lse within the decode
tolerances; for NOSA units the eviction mask bit-exact and the locality bound
|cur & prev| / |cur| >= k_e / k every step.  nosa_drift runs all 64 drift steps this way.
Two plans of 128 units with 2049-4096 and 4097-8192 block slots run the register
selections with 512 threads and 8 blocks per thread, and with 256 threads and 32 blocks
per thread.

The oracle runs on the host in a thread pool (NumPy releases the interpreter lock in
its array work; one BLAS thread per call).  The largest ratio of error to allowed error
over each workload's outputs is printed.
"""
import concurrent.futures as cf
import math
import os

import numpy as np
import pytest
import torch
from threadpoolctl import threadpool_limits

import block_sparse_decode_summary_amd as fx
from oracle.delta import locality, selection_delta
from oracle.pooling import block_summaries, sub_block_means
from oracle.step import unit_step
from workloads import (HeadPolicy, MODE_NOSA, MODE_RETRIEVAL, MODE_STREAMING, WORKLOAD_NAMES,
                       Workload, generate, get_workload, query_at_step)
from workloads.generate import unit_logits

from gpu_harness import (INT32_MAX, LSE_TOL, TOL, GpuView, assert_close, make_plan, say,
                         softmax_scale)

pytestmark = pytest.mark.gpu
DEV = "cuda"
THREADS = min(16, len(os.sched_getaffinity(0)))


def _widen(t: torch.Tensor) -> np.ndarray:
    """float64 copy of a bf16 / f32 host tensor (exact)."""
    if t.dtype == torch.bfloat16:
        u = t.view(torch.int16).numpy().view(np.uint16)
        return (u.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return t.numpy().astype(np.float64)


class UnitData:
    """One unit's host inputs.  Made in the main thread (raw copies of the valid K and V
    rows); widened to float64, and its summaries built by the oracle, in a worker."""

    def __init__(self, w: Workload, inp, u: int):
        self.u = u
        self.b, self.h = divmod(u, w.num_kv_heads)
        self.T = w.seq_lens[self.b]
        self.raw = (inp.K[self.b, self.h, :self.T].to("cpu"), inp.V[self.b, self.h, :self.T].to("cpu"))
        self.logits = unit_logits(inp, u)
        self.K = self.V = self.summ = None

    def ready(self, w: Workload) -> None:
        if self.K is None:
            self.K, self.V = _widen(self.raw[0]), _widen(self.raw[1])
            self.raw = None
            pol = w.policies[self.u]
            fn = block_summaries if w.pooling == 0 else sub_block_means
            self.summ = fn(self.K, pol.block, pol.sub_block, w.dtype)


def _compare(w: Workload, gv: GpuView, u: int, ref, q_rows, tag: str) -> float:
    g = gv.unit(u)
    assert np.array_equal(g.summaries, ref.summaries), f"{tag}: summaries differ"
    if ref.scores is not None:
        assert np.array_equal(g.scores.view(np.uint32), ref.scores.view(np.uint32)), \
            f"{tag}: scores differ"
    assert np.array_equal(g.sel, ref.sel), f"{tag}: selection {g.sel} vs {ref.sel}"
    assert gv.padding_ok(u), f"{tag}: sel_idx padding"
    rtol, atol = TOL[w.dtype]
    r = assert_close(f"{tag} out", g.out, ref.out_exact, rtol, atol)
    assert_close(f"{tag} lse", g.lse, ref.lse, *LSE_TOL)
    return r


def _step_all(w: Workload, inp, q: torch.Tensor, gv: GpuView, cache, evicted, prev, deltas,
              t: int, check_out: bool = True) -> float:
    """Oracle step of every unit (thread pool), compared with the GPU's step t.  cache:
    a dict that keeps each unit's host data across steps, or None (made and dropped)."""
    G = w.group
    qh = _widen(q.to("cpu"))
    added, added_cnt, removed, removed_cnt = deltas
    scale = softmax_scale(w)

    def one(d: UnitData):
        u = d.u
        d.ready(w)
        pol = w.policies[u]
        q_rows = qh[d.b, d.h * G:(d.h + 1) * G]
        ref = unit_step(pol, d.T, w.dtype, q_rows, d.K, d.V, scale, logits=d.logits,
                        evicted=evicted[u], summaries=d.summ, pooling=w.pooling)
        tag = f"{w.name} unit {u} step {t}"
        if check_out:
            ratio = _compare(w, gv, u, ref, q_rows, tag)
        else:
            ratio = 0.0
            g = gv.unit(u)
            assert np.array_equal(g.sel, ref.sel), f"{tag}: selection {g.sel} vs {ref.sel}"
            if ref.scores is not None:
                assert np.array_equal(g.scores.view(np.uint32), ref.scores.view(np.uint32)), \
                    f"{tag}: scores differ"
        if pol.mode == MODE_NOSA:
            n_full = d.T // pol.block
            got = gv.evicted(u)
            assert np.array_equal(got[:n_full], ref.evicted[:n_full]), f"{tag}: eviction mask"
            assert not got[n_full:].any(), f"{tag}: mask bits past the full blocks"
            if t > 0:
                k = pol.k_evict + pol.top_k
                assert locality(prev[u], ref.sel) >= pol.k_evict / k, f"{tag}: locality"
        a_ref, r_ref = selection_delta(prev[u], ref.sel)
        assert list(added[u, :added_cnt[u]]) == list(a_ref), f"{tag}: added"
        assert list(removed[u, :removed_cnt[u]]) == list(r_ref), f"{tag}: removed"
        assert np.all(added[u, added_cnt[u]:] == -1) and np.all(removed[u, removed_cnt[u]:] == -1)
        return u, ref, ratio

    worst = 0.0
    pending = []

    def drain(n_keep: int) -> None:
        nonlocal worst
        while len(pending) > n_keep:
            u, ref, ratio = pending.pop(0).result()
            evicted[u] = ref.evicted
            prev[u] = ref.sel
            worst = max(worst, ratio)

    with threadpool_limits(limits=1), cf.ThreadPoolExecutor(THREADS) as ex:
        for u in range(w.num_units):
            if cache is not None and u in cache:
                d = cache[u]
            else:
                d = UnitData(w, inp, u)
                if cache is not None:
                    cache[u] = d
            pending.append(ex.submit(one, d))
            drain(2 * THREADS)      # bounds the host copies held at once
        drain(0)
    return worst


def _run_full(w: Workload, steps: int, out_steps=None):
    say(f"[full] {w.name}: B={w.batch} Hq={w.num_q_heads} Hkv={w.num_kv_heads} d={w.head_dim} "
        f"{w.dtype} t_cap={w.t_cap} units={w.num_units} steps={steps}")
    inp = generate(w, DEV)
    plan = make_plan(w)
    A = fx.allocate_step_buffers(plan, DEV)
    B = fx.allocate_step_buffers(plan, DEV)
    fx.fx_build_summaries(plan, inp.K, inp.seq_lens, 0, INT32_MAX, A.summaries)
    cache = {} if steps > 1 else None
    evicted = [None] * w.num_units
    prev = [np.zeros(0, np.int64)] * w.num_units
    cur, old = A, B
    worst = 0.0
    mask = A.evicted_mask if w.has_nosa else None
    for t in range(steps):
        q = query_at_step(w, t, DEV) if t > 0 else inp.q
        fx.fx_select_delta(plan, q, A.summaries, inp.logits, mask, inp.seq_lens, old.sel_idx,
                           old.sel_cnt, cur.sel_idx, cur.sel_cnt, A.added, A.added_cnt,
                           A.removed, A.removed_cnt, A.workspace)
        fx.fx_sparse_decode(plan, q, inp.K, inp.V, inp.seq_lens, cur.sel_idx, cur.sel_cnt,
                            softmax_scale(w), A.out, A.lse, A.workspace)
        torch.cuda.synchronize()
        # GpuView reads summaries, scores (workspace), out, lse and the mask from A and the
        # selection from `cur`.
        A.sel_idx, A.sel_cnt, keep = cur.sel_idx, cur.sel_cnt, (A.sel_idx, A.sel_cnt)
        gv = GpuView(plan, A, w)
        A.sel_idx, A.sel_cnt = keep
        deltas = (A.added.cpu().numpy(), A.added_cnt.cpu().numpy(), A.removed.cpu().numpy(),
                  A.removed_cnt.cpu().numpy())
        check_out = out_steps is None or t in out_steps
        worst = max(worst, _step_all(w, inp, q, gv, cache, evicted, prev, deltas, t, check_out))
        say(f"[full] {w.name}: step {t} every unit matches (max err/limit so far {worst:.3f})")
        cur, old = old, cur
    assert fx.fx_read_error(plan) == 0
    say(f"[full] {w.name}: max |err| / allowed over all outputs = {worst:.4f}")
    del inp, A, B, cache
    torch.cuda.empty_cache()
    return worst


@pytest.mark.parametrize("name", [n for n in WORKLOAD_NAMES if n != "nosa_drift"])
def test_full_size_every_unit(name):
    _run_full(get_workload(name), steps=1)


def test_nosa_drift_full_trajectory():
    """All 64 drift steps of the NOSA workload at full size, every unit every step."""
    w = get_workload("nosa_drift")
    _run_full(w, steps=w.steps)


def _wide_plan_workload(n_cap: int) -> Workload:
    """128 units (64 sequences x 2 kv heads), block 16, d 64: t_cap = 16 * n_cap gives
    n_cap block slots, so the 256-thread selection keeps 16 (n_cap <= 4096) or 32
    (<= 8192) blocks per thread.  Most sequences are short; two reach the capacity."""
    t_cap = 16 * n_cap
    rng = np.random.default_rng(n_cap)
    lens = [int(x) for x in rng.integers(100, 3000, size=64)]
    lens[5], lens[40] = t_cap, t_cap - 9
    pols = (HeadPolicy(MODE_RETRIEVAL, block=16, sub_block=4, budget=float(np.float32(0.03)),
                       force_sink=1, force_last=1),
            HeadPolicy(MODE_NOSA, block=16, sub_block=8, top_k=12, k_evict=20))
    return Workload(name=f"wide_{n_cap}", batch=64, num_q_heads=4, num_kv_heads=2, head_dim=64,
                    dtype="bf16", t_cap=t_cap, seq_lens=tuple(lens), policies=pols * 64,
                    seed=1000 + n_cap, sink_scaled_tokens=4, needles_per_head=2,
                    drift=(0.9, 0.44), steps=2)


@pytest.mark.parametrize("n_cap", [3000, 6000])
def test_register_selection_of_wide_units(n_cap):
    w = _wide_plan_workload(n_cap)
    plan = make_plan(w)
    assert plan.units >= 128
    _run_full(w, steps=2)
