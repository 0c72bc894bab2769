"""Exp-delayed eviction scores in attention (fx_sparse_decode_ed) vs the CPU oracle.

[NOSA-DE] Methodik §1, "ED-DMA", read as: block j's raw eviction logit is added to the
attention logit of each of its tokens in NOSA units.  NOSA units are compared with the
oracle (unit_step with ed=True) at the decode tolerances; units of the other modes must
come out bit-identical to fx_sparse_decode, since the entry point leaves them alone.
"""
import numpy as np
import pytest
import torch

import block_sparse_decode_summary_amd as fx
from workloads import (HeadPolicy, MODE_NOSA, MODE_RETRIEVAL, MODE_STREAMING, Workload, generate,
                       get_workload, query_at_step, small_workload)

from gpu_harness import (INT32_MAX, GpuView, compare_unit, make_plan, oracle_unit, say,
                         softmax_scale)

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _custom(name, batch, Hq, Hkv, d, dtype, t_cap, lens, pols, seed=60, steps=1):
    return Workload(name=name, batch=batch, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=d,
                    dtype=dtype, t_cap=t_cap, seq_lens=tuple(lens), policies=tuple(pols), seed=seed,
                    sink_scaled_tokens=4, needles_per_head=2, steps=steps,
                    drift=(0.9, 0.44) if steps > 1 else None)


def _step(plan, bufs, inp, q, logits, build):
    """Select, then the plain decode (returned as host copies) and the ED decode (left in
    bufs.out / bufs.lse)."""
    w = inp.workload
    if build:
        fx.fx_build_summaries(plan, inp.K, inp.seq_lens, 0, INT32_MAX, bufs.summaries)
    fx.fx_select(plan, q, bufs.summaries, inp.logits, bufs.evicted_mask if w.has_nosa else None,
                 inp.seq_lens, bufs.sel_idx, bufs.sel_cnt, bufs.workspace)
    scale = softmax_scale(w)
    fx.fx_sparse_decode(plan, q, inp.K, inp.V, inp.seq_lens, bufs.sel_idx, bufs.sel_cnt, scale,
                        bufs.out, bufs.lse, bufs.workspace)
    plain_out = bufs.out.clone()
    plain_lse = bufs.lse.clone()
    fx.fx_sparse_decode_ed(plan, q, inp.K, inp.V, inp.seq_lens, bufs.sel_idx, bufs.sel_cnt, logits,
                           scale, bufs.out, bufs.lse, bufs.workspace)
    torch.cuda.synchronize()
    return plain_out, plain_lse


def _check_units(w, inp, q, gv, plain_out, plain_lse, units, evicted):
    G = w.group
    po = plain_out.cpu().to(torch.float64).numpy()
    pl = plain_lse.cpu().to(torch.float64).numpy()
    n_nosa = 0
    for u in units:
        b, h = divmod(u, w.num_kv_heads)
        if w.policies[u].mode == MODE_NOSA:
            ref = oracle_unit(inp, u, q, evicted.get(u), ed=True)
            compare_unit(w, u, gv, ref)
            evicted[u] = ref.evicted
            n_nosa += 1
        else:
            rows = slice(h * G, (h + 1) * G)
            assert np.array_equal(gv.out[b, rows], po[b, rows]), f"unit {u}: out differs from plain"
            assert np.array_equal(gv.lse[b, rows], pl[b, rows]), f"unit {u}: lse differs from plain"
    return n_nosa


def _run(w: Workload, steps: int = 1, units=None):
    say(f"[ed] {w.name}: B={w.batch} Hq={w.num_q_heads} Hkv={w.num_kv_heads} d={w.head_dim} "
        f"{w.dtype} t_cap={w.t_cap} steps={steps}")
    inp = generate(w, DEV)
    plan = make_plan(w)
    bufs = fx.allocate_step_buffers(plan, DEV)
    units = list(range(w.num_units)) if units is None else units
    steps = min(steps, w.steps)       # later steps need a drifting query
    evicted = {}
    n_nosa = 0
    for t in range(steps):
        q = query_at_step(w, t, DEV) if t > 0 else inp.q
        plain_out, plain_lse = _step(plan, bufs, inp, q, inp.logits, build=(t == 0))
        gv = GpuView(plan, bufs, w)
        n_nosa += _check_units(w, inp, q, gv, plain_out, plain_lse, units, evicted)
    assert fx.fx_read_error(plan) == 0
    say(f"[ed] {w.name}: ok ({n_nosa} NOSA unit-steps)")
    return n_nosa


@pytest.mark.parametrize("name", ["nosa_drift", "mixed_serving"])
def test_ed_small_workloads(name):
    """nosa_drift: every kv head NOSA; mixed_serving: none (the call must equal the plain one)."""
    w = small_workload(name)
    n = _run(w, steps=min(w.steps, 4))
    assert (n > 0) == w.has_nosa


@pytest.mark.parametrize("name", ["nosa_drift", "mixed_serving"])
def test_ed_full_size_sampled(name):
    """Full workload sizes in the benchmark's launch configuration; sampled units."""
    w = get_workload(name)
    rng = np.random.default_rng(300)
    nosa = [u for u in range(w.num_units) if w.policies[u].mode == MODE_NOSA]
    other = [u for u in range(w.num_units) if w.policies[u].mode != MODE_NOSA]
    pick = lambda us, k: list(rng.choice(us, size=min(k, len(us)), replace=False)) if us else []
    units = sorted(set(pick(nosa, 5) + pick(other, 3) + [w.num_units - 1]))
    assert (_run(w, steps=2, units=units) > 0) == w.has_nosa
    torch.cuda.empty_cache()


@pytest.mark.parametrize("G,d,dtype", [(1, 128, "bf16"), (3, 64, "bf16"), (8, 128, "bf16"),
                                       (5, 128, "f32")])
def test_ed_group_sizes_ragged_lengths(G, d, dtype):
    """Group sizes whose ED kernel holds fewer workgroups per CU than the plain one, ragged
    and degenerate lengths, mixed modes."""
    lens = [0, 1, 17, 1000, 2999]
    pols = []
    for _ in lens:
        pols += [HeadPolicy(MODE_NOSA, block=16, sub_block=8, top_k=2, k_evict=3, force_sink=1,
                            force_last=1),
                 HeadPolicy(MODE_RETRIEVAL, block=32, sub_block=16, top_k=4, force_sink=1,
                            force_last=1),
                 HeadPolicy(MODE_NOSA, block=64, sub_block=16, top_k=3, k_evict=0),
                 HeadPolicy(MODE_STREAMING, block=16, sub_block=16, sink_tokens=5, local_tokens=40)]
    w = _custom(f"ed_g{G}_d{d}_{dtype}", len(lens), 4 * G, 4, d, dtype, 3000, lens, pols, steps=2)
    assert _run(w, steps=2) > 0


def test_ed_nonfinite_logit_counts_as_zero():
    w = small_workload("nosa_drift")
    say(f"[ed] nonfinite: {w.name}")
    inp = generate(w, DEV)
    plan = make_plan(w)
    bufs = fx.allocate_step_buffers(plan, DEV)
    _step(plan, bufs, inp, inp.q, inp.logits, build=True)
    sel_idx = bufs.sel_idx.cpu().numpy()
    sel_cnt = bufs.sel_cnt.cpu().numpy()
    offs = w.block_offsets()
    # One selected block in each of the first three NOSA units: NaN, +inf, -inf.
    nosa = [u for u in range(w.num_units) if w.policies[u].mode == MODE_NOSA and sel_cnt[u] > 1][:3]
    assert len(nosa) == 3
    bad = inp.logits.clone()
    zero = inp.logits.clone()
    for u, v in zip(nosa, (float("nan"), float("inf"), float("-inf"))):
        slot = int(offs[u]) + int(sel_idx[u, 1])
        bad[slot] = v
        zero[slot] = 0.0
    assert fx.fx_read_error(plan) == 0
    scale = softmax_scale(w)
    outs = []
    for lg in (zero, bad):
        fx.fx_sparse_decode_ed(plan, inp.q, inp.K, inp.V, inp.seq_lens, bufs.sel_idx,
                               bufs.sel_cnt, lg, scale, bufs.out, bufs.lse, bufs.workspace)
        torch.cuda.synchronize()
        outs.append((bufs.out.cpu().clone(), bufs.lse.cpu().clone()))
        err = fx.fx_read_error(plan)
        assert err == (fx.FX_ERR_NONFINITE if lg is bad else 0), err
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])


def test_ed_without_nosa_units_is_plain_and_null_logits_rules():
    lens = [500, 1200]
    pols = [HeadPolicy(MODE_RETRIEVAL, block=16, sub_block=4, top_k=5, force_sink=1, force_last=1),
            HeadPolicy(MODE_STREAMING, block=16, sub_block=16, sink_tokens=4, local_tokens=64)] * 2
    w = _custom("ed_no_nosa", 2, 4, 2, 128, "bf16", 1500, lens, pols)
    say(f"[ed] {w.name}")
    inp = generate(w, DEV)
    plan = make_plan(w)
    bufs = fx.allocate_step_buffers(plan, DEV)
    plain_out, plain_lse = _step(plan, bufs, inp, inp.q, None, build=True)
    assert torch.equal(bufs.out, plain_out) and torch.equal(bufs.lse, plain_lse)
    # A plan with NOSA units refuses NULL logits before enqueuing anything.
    w2 = small_workload("nosa_drift")
    inp2 = generate(w2, DEV)
    plan2 = make_plan(w2)
    bufs2 = fx.allocate_step_buffers(plan2, DEV)
    with pytest.raises(RuntimeError):
        fx.fx_sparse_decode_ed(plan2, inp2.q, inp2.K, inp2.V, inp2.seq_lens, bufs2.sel_idx,
                               bufs2.sel_cnt, None, softmax_scale(w2), bufs2.out, bufs2.lse,
                               bufs2.workspace)
    assert fx.fx_read_error(plan) == 0 and fx.fx_read_error(plan2) == 0
