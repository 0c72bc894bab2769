"""HIP library vs CPU oracle, element by element (needs an MI355X).

Bar: summaries, scores, selected indices, eviction masks and deltas bit-exact;
out within |d| <= atol + rtol |ref| (bf16: rtol 2e-2, atol 1e-2; fp32: 1e-4, 1e-4)
against the oracle's float64 value; lse within rtol 1e-5, atol 1e-4.
"""
import dataclasses
import math

import numpy as np
import pytest
import torch

import block_sparse_decode_summary_amd as fx
from oracle.delta import locality, selection_delta
from oracle.step import unit_step
from workloads import (HeadPolicy, MODE_NOSA, MODE_RETRIEVAL, MODE_STREAMING, WORKLOAD_NAMES,
                       Workload, append_tokens, generate, get_workload, query_at_step,
                       small_workload, unit_arrays)

from gpu_harness import (INT32_MAX, GpuView, compare_unit, make_plan, oracle_unit,
                         run_select_decode, say, softmax_scale, assert_close, TOL)

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _run_and_compare_all(w: Workload, split_tokens: int = 0, steps: int = 1):
    say(f"[parity] {w.name}: B={w.batch} Hq={w.num_q_heads} Hkv={w.num_kv_heads} d={w.head_dim} "
        f"{w.dtype} t_cap={w.t_cap} split={split_tokens} steps={steps}")
    inp = generate(w, DEV)
    plan = make_plan(w, split_tokens)
    bufs = fx.allocate_step_buffers(plan, DEV)
    evicted = {u: None for u in range(w.num_units)}
    prev = {u: np.zeros(0, np.int64) for u in range(w.num_units)}
    for t in range(steps):
        q = query_at_step(w, t, DEV) if t > 0 else inp.q
        bufs.prev_idx.copy_(bufs.sel_idx)
        bufs.prev_cnt.copy_(bufs.sel_cnt)
        run_select_decode(plan, bufs, inp, q, build=(t == 0))
        fx.fx_selection_delta(plan, bufs.prev_idx, bufs.prev_cnt, bufs.sel_idx, bufs.sel_cnt,
                              bufs.added, bufs.added_cnt, bufs.removed, bufs.removed_cnt)
        gv = GpuView(plan, bufs, w)
        added = bufs.added.cpu().numpy()
        added_cnt = bufs.added_cnt.cpu().numpy()
        removed = bufs.removed.cpu().numpy()
        removed_cnt = bufs.removed_cnt.cpu().numpy()
        for u in range(w.num_units):
            ref = oracle_unit(inp, u, q, evicted[u])
            compare_unit(w, u, gv, ref)
            if w.policies[u].mode == MODE_NOSA:
                n_full = w.seq_lens[u // w.num_kv_heads] // w.policies[u].block
                got_ev = gv.evicted(u)
                assert np.array_equal(got_ev[:n_full], ref.evicted[:n_full]), f"unit {u} mask step {t}"
                assert not got_ev[n_full:].any()
                evicted[u] = ref.evicted
                if t > 0:
                    p = w.policies[u]
                    assert locality(prev[u], ref.sel) >= p.k_evict / (p.k_evict + p.top_k)
            a_ref, r_ref = selection_delta(prev[u], ref.sel)
            assert list(added[u, :added_cnt[u]]) == list(a_ref), f"unit {u} added, step {t}"
            assert list(removed[u, :removed_cnt[u]]) == list(r_ref), f"unit {u} removed, step {t}"
            assert np.all(added[u, added_cnt[u]:] == -1) and np.all(removed[u, removed_cnt[u]:] == -1)
            prev[u] = ref.sel
    assert fx.fx_read_error(plan) == 0
    say(f"[parity] {w.name}: ok")


@pytest.mark.parametrize("name", WORKLOAD_NAMES)
def test_parity_small_workloads(name):
    w = small_workload(name)
    _run_and_compare_all(w, steps=w.steps)


@pytest.mark.parametrize("name", WORKLOAD_NAMES)
def test_parity_full_size_sampled(name):
    """Full workload sizes in the launch configuration the benchmark uses; sampled units."""
    w = get_workload(name)
    say(f"[full] {name}: generating B={w.batch} t_cap={w.t_cap}")
    inp = generate(w, DEV)
    plan = make_plan(w)
    bufs = fx.allocate_step_buffers(plan, DEV)
    steps = 2 if w.has_nosa else 1
    rng = np.random.default_rng(100 + WORKLOAD_NAMES.index(name))
    units = sorted(set([0, w.num_units - 1] + list(rng.choice(w.num_units, size=min(6, w.num_units),
                                                              replace=False))))
    evicted = {u: None for u in units}
    for t in range(steps):
        q = query_at_step(w, t, DEV) if t > 0 else inp.q
        say(f"[full] {name}: step {t} (split {plan.split_tokens}), units {units}")
        run_select_decode(plan, bufs, inp, q, build=(t == 0))
        gv = GpuView(plan, bufs, w)
        for u in units:
            ref = oracle_unit(inp, u, q, evicted[u])
            compare_unit(w, u, gv, ref)
            if w.policies[u].mode == MODE_NOSA:
                evicted[u] = ref.evicted
    # Properties at every unit: counts within the plan bound, ascending selections,
    # finite outputs.
    cnt = gv.sel_cnt
    assert np.all(cnt >= 0) and np.all(cnt <= plan.max_selected)
    for u in range(w.num_units):
        s = gv.sel_idx[u, :cnt[u]]
        assert np.all(np.diff(s) > 0)
    assert np.all(np.isfinite(gv.out))
    assert fx.fx_read_error(plan) == 0
    del inp, bufs
    torch.cuda.empty_cache()


def _custom(name, batch, Hq, Hkv, d, dtype, t_cap, lens, pols, seed=50):
    return Workload(name=name, batch=batch, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=d,
                    dtype=dtype, t_cap=t_cap, seq_lens=tuple(lens), policies=tuple(pols), seed=seed,
                    sink_scaled_tokens=4, needles_per_head=2)


def test_dense_when_everything_is_selected():
    """Block size 1 with k = n, and a budget covering all blocks, are dense attention."""
    T = 300
    for g, k in ((1, T), (16, 1000)):
        pol = HeadPolicy(MODE_RETRIEVAL, block=g, sub_block=1, top_k=k)
        w = _custom(f"dense_g{g}", 1, 4, 2, 64, "bf16", T, [T], [pol, pol])
        _run_and_compare_all(w)
        inp = generate(w, DEV)
        plan = make_plan(w)
        bufs = fx.allocate_step_buffers(plan, DEV)
        run_select_decode(plan, bufs, inp, inp.q)
        torch.cuda.synchronize()
        qf = inp.q.double().cpu()
        Kf = inp.K.double().cpu()
        Vf = inp.V.double().cpu()
        for h in range(2):
            qr = qf[0, 2 * h:2 * h + 2]
            s = (qr @ Kf[0, h, :T].T) / math.sqrt(64)
            dense = torch.softmax(s, dim=-1) @ Vf[0, h, :T]
            assert_close("dense", bufs.out[0, 2 * h:2 * h + 2].double().cpu().numpy(), dense.numpy(),
                         *TOL["bf16"])


def test_ragged_degenerate_lengths_and_mixed_modes():
    lens = [0, 1, 15, 16, 17, 1000]
    pols = []
    for _ in lens:
        pols += [HeadPolicy(MODE_RETRIEVAL, block=16, sub_block=4, top_k=3, force_sink=1, force_last=1),
                 HeadPolicy(MODE_STREAMING, block=16, sub_block=16, sink_tokens=5, local_tokens=20),
                 HeadPolicy(MODE_NOSA, block=16, sub_block=8, top_k=2, k_evict=2)]
    w = _custom("ragged_mixed", len(lens), 6, 3, 128, "bf16", 1024, lens, pols)
    _run_and_compare_all(w, steps=1)
    for split in (64, 2048):
        _run_and_compare_all(w.replace(name=f"ragged_mixed_s{split}"), split_tokens=split)
    # 257 block slots per unit: the 512-thread selection that forms its own scores; 513:
    # scores from the separate scoring kernel.
    for n_cap in (257, 513):
        _run_and_compare_all(w.replace(name=f"ragged_mixed_{n_cap}", t_cap=n_cap * 16), steps=1)


def test_segments_of_masked_slots_only():
    """The decode partitions token slots (selected blocks times the block size), so the tail
    of a partial last block counts as slots that read nothing.  With blocks of 128 tokens,
    lengths of the form 128 k + 1 and 64-slot segments, some segments hold only masked
    slots: every unit against the oracle, with few units (each unit cut into its own pieces)
    and with more units (stream-K across units), at 64-slot segments and the default."""
    lens_cycle = [1, 127, 128, 129, 255, 257, 385, 1025]
    pol_s = HeadPolicy(MODE_STREAMING, block=128, sub_block=128, sink_tokens=1, local_tokens=100000)
    pol_r = HeadPolicy(MODE_RETRIEVAL, block=128, sub_block=32, top_k=4, force_sink=1, force_last=1)
    for B in (4, 20):
        lens = [lens_cycle[i % len(lens_cycle)] for i in range(B)]
        w = _custom(f"masked_slots_b{B}", B, 4, 2, 64, "bf16", 1152, lens, [pol_s, pol_r] * B)
        _run_and_compare_all(w.replace(name=f"masked_slots_b{B}_s64"), split_tokens=64)
        _run_and_compare_all(w)


def test_more_units_than_one_scan_chunk():
    """2080 units (three chunks of the decode's unit scan, which keeps 1024 units in
    registers), ragged short lengths with empty units, all three modes: every unit against
    the oracle, with the default segment length and with 64-token segments."""
    rng = np.random.default_rng(2080)
    B, Hkv = 520, 4
    lens = [int(x) for x in rng.integers(0, 200, size=B)]
    lens[7] = lens[300] = 0
    pols = []
    for _ in range(B):
        pols += [HeadPolicy(MODE_RETRIEVAL, block=16, sub_block=8, top_k=3, force_sink=1, force_last=1),
                 HeadPolicy(MODE_STREAMING, block=16, sub_block=16, sink_tokens=5, local_tokens=40),
                 HeadPolicy(MODE_NOSA, block=16, sub_block=8, top_k=2, k_evict=3),
                 HeadPolicy(MODE_RETRIEVAL, block=16, sub_block=4, budget=float(np.float32(0.3)),
                            force_sink=1, force_last=1)]
    w = _custom("many_units", B, 2 * Hkv, Hkv, 64, "bf16", 256, lens, pols)
    assert w.num_units > 2 * 1024
    _run_and_compare_all(w)
    _run_and_compare_all(w.replace(name="many_units_s64"), split_tokens=64)


@pytest.mark.parametrize("G,d,dtype", [(1, 128, "bf16"), (3, 128, "bf16"), (8, 128, "bf16"),
                                       (2, 64, "bf16"), (5, 128, "f32"), (8, 64, "f32")])
def test_group_sizes_and_head_dims(G, d, dtype):
    Hkv = 2
    pol = HeadPolicy(MODE_RETRIEVAL, block=32, sub_block=16, budget=float(np.float32(0.1)),
                     force_sink=1, force_last=1)
    w = _custom(f"g{G}_d{d}_{dtype}", 2, G * Hkv, Hkv, d, dtype, 3000, [3000, 2211],
                [pol] * (2 * Hkv))
    _run_and_compare_all(w)


def test_wide_selection_workgroups():
    """Few units with thousands of block slots take the 1024-thread selection workgroups:
    every mode, budgets and NOSA state over two drift steps, against the oracle."""
    pols = []
    for _ in range(2):
        pols += [HeadPolicy(MODE_RETRIEVAL, block=8, sub_block=4, budget=float(np.float32(0.07)),
                            force_sink=1, force_last=1),
                 HeadPolicy(MODE_NOSA, block=8, sub_block=8, top_k=37, k_evict=90),
                 HeadPolicy(MODE_STREAMING, block=8, sub_block=8, sink_tokens=16, local_tokens=300)]
    w = _custom("wide_select", 2, 6, 3, 64, "bf16", 40000, [40000, 23457], pols)
    _run_and_compare_all(w.replace(drift=(0.9, 0.44), steps=2), steps=2)


def test_split_invariance_and_determinism():
    w = small_workload("qwen7b_layer")
    inp = generate(w, DEV)
    outs = []
    sels = []
    for split in (64, 256, 2048):
        plan = make_plan(w, split)
        bufs = fx.allocate_step_buffers(plan, DEV)
        run_select_decode(plan, bufs, inp, inp.q)
        o1 = bufs.out.clone()
        run_select_decode(plan, bufs, inp, inp.q)
        assert torch.equal(o1, bufs.out), f"split {split}: two runs differ"
        outs.append(o1.double().cpu().numpy())
        sels.append(bufs.sel_idx.cpu().numpy().copy())
    for s in sels[1:]:
        assert np.array_equal(s, sels[0])
    for o in outs[1:]:
        assert_close("split", o, outs[0], 2e-2, 1e-2)


def test_score_ties_prefer_lower_index():
    g, T = 16, 16 * 40
    pol = HeadPolicy(MODE_RETRIEVAL, block=g, sub_block=16, top_k=3, force_sink=0, force_last=0)
    w = _custom("ties", 1, 2, 1, 128, "bf16", T, [T], [pol])
    inp = generate(w, DEV)
    # Five identical copies of one block aligned with the query (scores far above the
    # needles') at blocks 7, 9, 20, 30, 33; top-3 must take the three lowest indices.
    src = inp.K[0, 0, 7 * g:8 * g].clone()
    src += 10.0 * inp.q[0, 0:2].float().mean(0).to(src.dtype)
    for j in (7, 9, 20, 30, 33):
        inp.K[0, 0, j * g:(j + 1) * g] = src
    plan = make_plan(w)
    bufs = fx.allocate_step_buffers(plan, DEV)
    run_select_decode(plan, bufs, inp, inp.q)
    gv = GpuView(plan, bufs, w)
    ref = oracle_unit(inp, 0, inp.q)
    compare_unit(w, 0, gv, ref)
    assert list(gv.unit(0).sel) == [7, 9, 20]


@pytest.mark.parametrize("dtype,t_cap", [("bf16", 12000), ("f32", 12000), ("bf16", 4000)])
def test_scores_with_wide_range_query_groups(dtype, t_cap):
    """The query rows of kv head 0 are scaled by 1, 2^-16, 2^16 and 2^-32 within each
    group: their float64 sums qs need more than 45 significant bits, so the chain's
    products qs[c] * S[c] are rounded (plain rows nearly always give exact ones), and the scores
    must still be the oracle's chain bit for bit; kv head 1 keeps plain rows.  t_cap
    12000 (750 block slots) scores in the tiled scoring kernel, 4000 (250) in the
    selection kernel that forms its own scores.  Scores, selections and outputs."""
    Hkv, G, d = 2, 4, 128
    pols = [HeadPolicy(MODE_RETRIEVAL, block=16, sub_block=4, budget=float(np.float32(0.05)),
                       force_sink=1, force_last=1),
            HeadPolicy(MODE_NOSA, block=16, sub_block=8, top_k=24, k_evict=48)]
    lens = [t_cap, t_cap * 7 // 9]
    w = _custom(f"wide_q_{dtype}_{t_cap}", 2, G * Hkv, Hkv, d, dtype, t_cap, lens, pols * 2)
    say(f"[parity] {w.name}")
    inp = generate(w, DEV)
    q = inp.q.clone()
    for g, e in enumerate((0, -16, 16, -32)):
        q[:, g, :] *= 2.0 ** e        # kv head 0 holds query heads 0..G-1
    plan = make_plan(w)
    bufs = fx.allocate_step_buffers(plan, DEV)
    run_select_decode(plan, bufs, inp, q)
    gv = GpuView(plan, bufs, w)
    for u in range(w.num_units):
        compare_unit(w, u, gv, oracle_unit(inp, u, q))
    assert fx.fx_read_error(plan) == 0


@pytest.mark.parametrize("t_cap", [8192 * 16, 8192 * 16 + 3000])
def test_many_blocks_per_unit(t_cap):
    """n_cap = 8192 is the largest unit whose selection keys stay in registers; one more
    block slot sends the plan through the workspace path of the selection kernel."""
    pols = [HeadPolicy(MODE_RETRIEVAL, block=16, sub_block=4, top_k=40, force_sink=1, force_last=1),
            HeadPolicy(MODE_NOSA, block=16, sub_block=8, top_k=24, k_evict=48),
            HeadPolicy(MODE_STREAMING, block=16, sub_block=16, sink_tokens=64, local_tokens=512)]
    w = _custom(f"blocks_{t_cap}", 2, 6, 3, 64, "bf16", t_cap, [t_cap, t_cap - 7], pols * 2)
    _run_and_compare_all(w.replace(drift=(0.9, 0.44)), steps=2)


def test_equal_values_take_lowest_indices():
    """Zero keys make every score +0 and zero logits tie every block, so the k best are the
    k lowest eligible indices, with far more equal candidates than one wave ranks."""
    g, T = 16, 16 * 3000 + 5
    pols = [HeadPolicy(MODE_RETRIEVAL, block=g, sub_block=16, top_k=100, force_sink=1, force_last=1),
            HeadPolicy(MODE_NOSA, block=g, sub_block=16, top_k=70, k_evict=90)]
    w = _custom("all_ties", 1, 4, 2, 128, "bf16", T, [T], pols)
    inp = generate(w, DEV)
    inp.K.zero_()
    inp.logits.zero_()
    plan = make_plan(w)
    bufs = fx.allocate_step_buffers(plan, DEV)
    run_select_decode(plan, bufs, inp, inp.q)
    gv = GpuView(plan, bufs, w)
    n_full, n_tot = T // g, -(-T // g)
    for u in range(2):
        ref = oracle_unit(inp, u, inp.q)
        compare_unit(w, u, gv, ref)
    # retrieval: F = {0, last}; NOSA: F = {last (partial)}, Γe = 0..89, Γq = 90..159.
    assert list(gv.unit(0).sel) == list(range(0, 101)) + [n_tot - 1]
    assert list(gv.unit(1).sel) == list(range(0, 160)) + [n_tot - 1]
    ev = gv.evicted(1)
    assert not ev[:90].any() and ev[90:n_full].all() and not ev[n_full:].any()
    assert fx.fx_read_error(plan) == 0


def test_growing_context_decode_loop():
    """The decode loop: every step appends one token to every sequence, the newest full
    block's summary is (re)built, new full blocks become score and eviction candidates,
    and the eviction mask carries NOSA's state from step to step.  Each step is checked
    against the oracle on the grown inputs: summaries, scores, selections and the mask
    bit-exact, outputs and deltas as everywhere else."""
    g = 16
    pols = [HeadPolicy(MODE_RETRIEVAL, block=g, sub_block=4, budget=float(np.float32(0.1)),
                       force_sink=1, force_last=1),
            HeadPolicy(MODE_NOSA, block=g, sub_block=8, top_k=3, k_evict=5),
            HeadPolicy(MODE_STREAMING, block=g, sub_block=16, sink_tokens=4, local_tokens=40)]
    lens = [16 * 12 + 13, 16 * 7 + 15, 16 * 30]     # three phases within a block
    steps = 40
    w0 = _custom("grow", 3, 6, 3, 64, "bf16", max(lens) + steps + 8, lens, pols * 3)
    w0 = w0.replace(drift=(0.9, 0.44))
    inp = generate(w0, DEV)
    plan = make_plan(w0)
    bufs = fx.allocate_step_buffers(plan, DEV)
    fx.fx_build_summaries(plan, inp.K, inp.seq_lens, 0, INT32_MAX, bufs.summaries)   # prefill
    evicted = {u: None for u in range(w0.num_units)}
    prev = {u: np.zeros(0, np.int64) for u in range(w0.num_units)}
    filled = 0
    for t in range(steps):
        if t > 0:
            old = lens
            lens = append_tokens(inp, lens, t)
            filled += sum(1 for a, b in zip(old, lens) if b % g == 0 and b != a)
        w = w0.replace(seq_lens=tuple(lens))
        it = dataclasses.replace(inp, workload=w)
        q = query_at_step(w0, t, DEV)
        fx.fx_build_summaries(plan, inp.K, inp.seq_lens, -1, INT32_MAX, bufs.summaries)
        bufs.prev_idx.copy_(bufs.sel_idx)
        bufs.prev_cnt.copy_(bufs.sel_cnt)
        run_select_decode(plan, bufs, it, q, build=False)
        fx.fx_selection_delta(plan, bufs.prev_idx, bufs.prev_cnt, bufs.sel_idx, bufs.sel_cnt,
                              bufs.added, bufs.added_cnt, bufs.removed, bufs.removed_cnt)
        gv = GpuView(plan, bufs, w)
        added, added_cnt = bufs.added.cpu().numpy(), bufs.added_cnt.cpu().numpy()
        removed, removed_cnt = bufs.removed.cpu().numpy(), bufs.removed_cnt.cpu().numpy()
        for u in range(w.num_units):
            ref = oracle_unit(it, u, q, evicted[u])
            compare_unit(w, u, gv, ref)
            if w.policies[u].mode == MODE_NOSA:
                n_full = lens[u // w.num_kv_heads] // g
                got_ev = gv.evicted(u)
                assert np.array_equal(got_ev[:n_full], ref.evicted[:n_full]), f"unit {u} mask step {t}"
                assert not got_ev[n_full:].any()
                # Over all block slots: blocks that fill later start out not evicted.
                evicted[u] = np.pad(ref.evicted, (0, w.n_cap(u) - len(ref.evicted)))
            a_ref, r_ref = selection_delta(prev[u], ref.sel)
            assert list(added[u, :added_cnt[u]]) == list(a_ref), f"unit {u} added, step {t}"
            assert list(removed[u, :removed_cnt[u]]) == list(r_ref), f"unit {u} removed, step {t}"
            prev[u] = ref.sel
    assert filled >= 6, "the loop should fill several blocks"
    assert fx.fx_read_error(plan) == 0


def test_summary_is_rounded_once():
    """A sub-block mean just above a bfloat16 tie: one rounding gives 241/256, two give 240/256."""
    g = 16
    pol = HeadPolicy(MODE_RETRIEVAL, block=g, sub_block=16, top_k=1)
    w = _custom("single_rounding", 1, 1, 1, 64, "bf16", 2 * g, [2 * g], [pol])
    inp = generate(w, DEV)
    col = torch.zeros(g, dtype=torch.float64)
    col[:14] = 1.0
    col[14] = 1.0 + 2.0 ** -5
    col[15] = 2.0 ** -36
    inp.K[0, 0, :g, 5] = col.to(torch.bfloat16).to(DEV)
    plan = make_plan(w)
    bufs = fx.allocate_step_buffers(plan, DEV)
    fx.fx_build_summaries(plan, inp.K, inp.seq_lens, 0, INT32_MAX, bufs.summaries)
    torch.cuda.synchronize()
    assert bufs.summaries[5].item() == 241 * 2.0 ** -8
    ref = oracle_unit(inp, 0, inp.q)
    got = bufs.summaries.double().cpu().numpy().reshape(-1, 64)[:2]
    assert np.array_equal(got, ref.summaries)


def test_incremental_summary_build():
    w = small_workload("llama8b_layer")
    inp = generate(w, DEV)
    plan = make_plan(w)
    bufs = fx.allocate_step_buffers(plan, DEV)
    fx.fx_build_summaries(plan, inp.K, inp.seq_lens, 0, INT32_MAX, bufs.summaries)
    g = 64
    n_full = w.seq_lens[0] // g
    inp.K[0, :, (n_full - 1) * g:n_full * g] *= -2       # change the newest full block
    before = bufs.summaries.clone()
    fx.fx_build_summaries(plan, inp.K, inp.seq_lens, -1, INT32_MAX, bufs.summaries)
    incr = bufs.summaries.clone()
    fx.fx_build_summaries(plan, inp.K, inp.seq_lens, 0, INT32_MAX, bufs.summaries)
    assert torch.equal(incr, bufs.summaries)
    changed = (incr.view(-1, 128) != before.view(-1, 128)).any(dim=1).nonzero().flatten().cpu()
    offs = w.block_offsets()
    assert set(changed.tolist()) <= {int(offs[u]) + n_full - 1 for u in range(w.num_units)}
    assert len(changed) > 0


def test_selection_delta_random_lists():
    pol = HeadPolicy(MODE_RETRIEVAL, block=16, sub_block=16, top_k=200)
    w = _custom("delta", 4, 4, 2, 64, "bf16", 16 * 400, [6400] * 4, [pol] * 8)
    plan = make_plan(w)
    ms = plan.max_selected
    rng = np.random.default_rng(7)
    prev = np.full((8, ms), -1, np.int32)
    cur = np.full((8, ms), -1, np.int32)
    pc = np.zeros(8, np.int32)
    cc = np.zeros(8, np.int32)
    for u in range(8):
        a = np.sort(rng.choice(400, size=int(rng.integers(0, ms + 1)), replace=False))
        c = np.sort(rng.choice(400, size=int(rng.integers(0, ms + 1)), replace=False))
        prev[u, :a.size], pc[u] = a, a.size
        cur[u, :c.size], cc[u] = c, c.size
    bufs = fx.allocate_step_buffers(plan, DEV)
    t = lambda x: torch.from_numpy(x).to(DEV)
    fx.fx_selection_delta(plan, t(prev), t(pc), t(cur), t(cc), bufs.added, bufs.added_cnt,
                          bufs.removed, bufs.removed_cnt)
    torch.cuda.synchronize()
    for u in range(8):
        ar, rr = selection_delta(prev[u, :pc[u]], cur[u, :cc[u]])
        assert list(bufs.added[u, :bufs.added_cnt[u]].cpu()) == list(ar)
        assert list(bufs.removed[u, :bufs.removed_cnt[u]].cpu()) == list(rr)


@pytest.mark.parametrize("t_cap_blocks", [64, 320, 520])
def test_bad_device_data_is_flagged_not_faulting(t_cap_blocks):
    """seq_len beyond t_cap and out-of-range selection entries are clamped / skipped by the
    kernels' own checks and reported in the error word (64 and 320 block slots: the
    selection forms its own scores, with 256 and 512 threads; 520: the separate scoring
    kernel)."""
    w = small_workload("tiny")
    w = w.replace(t_cap=t_cap_blocks * w.policies[0].block)
    inp = generate(w, DEV)
    plan = make_plan(w)
    bufs = fx.allocate_step_buffers(plan, DEV)
    bad_lens = torch.tensor([w.t_cap + 100], dtype=torch.int32, device=DEV)
    fx.fx_build_summaries(plan, inp.K, bad_lens, 0, INT32_MAX, bufs.summaries)
    fx.fx_select(plan, inp.q, bufs.summaries, None, None, bad_lens, bufs.sel_idx, bufs.sel_cnt,
                 bufs.workspace)
    torch.cuda.synchronize()
    assert fx.fx_read_error(plan) & fx.FX_ERR_SEQ_LEN
    sel = bufs.sel_idx.clone()
    sel[0, 1] = 10_000                                      # outside the unit's blocks
    sel[1, 2] = sel[1, 1]                                   # not ascending
    fx.fx_sparse_decode(plan, inp.q, inp.K, inp.V, inp.seq_lens, sel, bufs.sel_cnt,
                        softmax_scale(w), bufs.out, bufs.lse, bufs.workspace)
    torch.cuda.synchronize()
    assert fx.fx_read_error(plan) & fx.FX_ERR_SEL_INDEX
    assert torch.isfinite(bufs.out).all()
