"""Delta-driven compaction (fx_compact_update) vs the CPU oracle.

[NOSA-DE] Methodik §2 (NOSI), "Optimierte Speicherlayout": blocks swapped by set
difference.  Slot maps and moved counts must match the oracle exactly, and every held
slot must hold its block's key and value rows bit for bit.
"""
import dataclasses

import numpy as np
import pytest
import torch

import block_sparse_decode_summary_amd as fx
from oracle.compaction import compact_update
from workloads import (HeadPolicy, MODE_NOSA, MODE_RETRIEVAL, MODE_STREAMING, Workload,
                       append_tokens, generate, query_at_step)

from gpu_harness import INT32_MAX, make_plan, oracle_unit, run_select_decode, say

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _custom(name, batch, Hq, Hkv, d, dtype, t_cap, lens, pols, seed=80):
    return Workload(name=name, batch=batch, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=d,
                    dtype=dtype, t_cap=t_cap, seq_lens=tuple(lens), policies=tuple(pols), seed=seed,
                    sink_scaled_tokens=4, needles_per_head=2)


class Mirror:
    """The oracle's side: one slot array per unit, updated by oracle.compaction."""

    def __init__(self, plan, w):
        self.w = w
        self.slots = [np.full(fx.fx_unit_max_selected(plan, u), -1) for u in range(w.num_units)]
        self.work_off = [fx.fx_unit_work_offset(plan, u) for u in range(w.num_units)]

    def step(self, u, sel, T):
        g = self.w.policies[u].block
        self.slots[u], moves = compact_update(self.slots[u], sel, T, g)
        return len(moves)


def _check(plan, w, inp, ws, mirror, lens, moved_ref, tag):
    torch.cuda.synchronize()
    smap = ws.slot_map.cpu().numpy()
    moved = ws.moved_cnt.cpu().numpy()
    wk = ws.work_K.cpu()
    wv = ws.work_V.cpu()
    Kc = inp.K.cpu()
    Vc = inp.V.cpu()
    for u in range(w.num_units):
        b_, h = divmod(u, w.num_kv_heads)
        g = w.policies[u].block
        n = len(mirror.slots[u])
        assert list(smap[u, :n]) == list(mirror.slots[u]), f"{tag} unit {u}: slot map"
        assert np.all(smap[u, n:] == -1), f"{tag} unit {u}: slots past max_sel(u)"
        assert moved[u] == moved_ref[u], f"{tag} unit {u}: moved {moved[u]} vs {moved_ref[u]}"
        off = mirror.work_off[u]
        for s, blk in enumerate(mirror.slots[u]):
            if blk < 0:
                continue
            rows = slice(off + s * g, off + (s + 1) * g)
            src = slice(blk * g, (blk + 1) * g)
            assert torch.equal(wk[rows], Kc[b_, h, src]), f"{tag} unit {u} slot {s}: K rows"
            assert torch.equal(wv[rows], Vc[b_, h, src]), f"{tag} unit {u} slot {s}: V rows"


@pytest.mark.parametrize("d,dtype", [(128, "bf16"), (64, "f32")])
def test_compaction_random_selections(d, dtype):
    """Seeded random selections over a context that grows by random amounts: held set,
    kept slots, lowest free slots, moved counts and slot contents."""
    pols = [HeadPolicy(MODE_RETRIEVAL, block=16, sub_block=4, top_k=12, force_sink=1,
                       force_last=1),
            HeadPolicy(MODE_NOSA, block=64, sub_block=16, top_k=3, k_evict=4),
            HeadPolicy(MODE_RETRIEVAL, block=256, sub_block=16, top_k=2, force_last=1),
            HeadPolicy(MODE_STREAMING, block=32, sub_block=8, sink_tokens=40, local_tokens=100)]
    lens0 = [0, 300, 1500]
    w = _custom(f"compact_{dtype}", 3, 8, 4, d, dtype, 4096, lens0, pols * 3)
    say(f"[compact] random selections {dtype} d={d}")
    inp = generate(w, DEV)
    plan = make_plan(w)
    bufs = fx.allocate_step_buffers(plan, DEV)
    ws = fx.allocate_working_set(plan, DEV)
    mirror = Mirror(plan, w)
    rng = np.random.default_rng(81)
    lens = list(lens0)
    ms = plan.max_selected
    for step in range(12):
        lens = [min(w.t_cap, T + int(rng.integers(0, 200))) for T in lens]
        inp.seq_lens.copy_(torch.tensor(lens, dtype=torch.int32))
        sel_idx = np.full((w.num_units, ms), -1, dtype=np.int32)
        sel_cnt = np.zeros(w.num_units, dtype=np.int32)
        moved_ref = np.zeros(w.num_units, dtype=np.int64)
        for u in range(w.num_units):
            T = lens[u // w.num_kv_heads]
            g = w.policies[u].block
            n_full, n_tot = T // g, -(-T // g)
            cap = len(mirror.slots[u])
            k = int(rng.integers(0, min(cap, n_full) + 1))
            sel = np.sort(rng.choice(n_full, size=k, replace=False)) if k else np.zeros(0, np.int64)
            if n_tot > n_full and len(sel) < cap:
                sel = np.append(sel, n_tot - 1)
            sel_idx[u, :len(sel)] = sel
            sel_cnt[u] = len(sel)
            moved_ref[u] = mirror.step(u, sel, T)
        bufs.sel_idx.copy_(torch.from_numpy(sel_idx))
        bufs.sel_cnt.copy_(torch.from_numpy(sel_cnt))
        fx.fx_compact_update(plan, inp.K, inp.V, inp.seq_lens, bufs.sel_idx, bufs.sel_cnt, ws,
                             bufs.workspace)
        _check(plan, w, inp, ws, mirror, lens, moved_ref, f"step {step}")
    assert fx.fx_read_error(plan) == 0


def test_compaction_in_the_growing_decode_loop():
    """End to end: select on the grown context each step (checked against the oracle),
    then compact; blocks that fill while selected become held."""
    g = 16
    pols = [HeadPolicy(MODE_RETRIEVAL, block=g, sub_block=4, budget=float(np.float32(0.1)),
                       force_sink=1, force_last=1),
            HeadPolicy(MODE_NOSA, block=g, sub_block=8, top_k=3, k_evict=5),
            HeadPolicy(MODE_STREAMING, block=g, sub_block=16, sink_tokens=4, local_tokens=40)]
    lens = [16 * 12 + 13, 16 * 7 + 15, 16 * 30]
    steps = 24
    w0 = _custom("compact_grow", 3, 6, 3, 64, "bf16", max(lens) + steps + 8, lens, pols * 3)
    w0 = w0.replace(drift=(0.9, 0.44))
    say("[compact] growing decode loop")
    inp = generate(w0, DEV)
    plan = make_plan(w0)
    bufs = fx.allocate_step_buffers(plan, DEV)
    ws = fx.allocate_working_set(plan, DEV)
    mirror = Mirror(plan, w0)
    fx.fx_build_summaries(plan, inp.K, inp.seq_lens, 0, INT32_MAX, bufs.summaries)
    evicted = {u: None for u in range(w0.num_units)}
    total_moved = 0
    for t in range(steps):
        if t > 0:
            lens = append_tokens(inp, lens, t)
        w = w0.replace(seq_lens=tuple(lens))
        it = dataclasses.replace(inp, workload=w)
        q = query_at_step(w0, t, DEV)
        fx.fx_build_summaries(plan, inp.K, inp.seq_lens, -1, INT32_MAX, bufs.summaries)
        run_select_decode(plan, bufs, it, q, build=False)
        fx.fx_compact_update(plan, inp.K, inp.V, inp.seq_lens, bufs.sel_idx, bufs.sel_cnt, ws,
                             bufs.workspace)
        torch.cuda.synchronize()
        sel_idx, sel_cnt = bufs.sel_idx.cpu().numpy(), bufs.sel_cnt.cpu().numpy()
        moved_ref = np.zeros(w.num_units, dtype=np.int64)
        for u in range(w.num_units):
            ref = oracle_unit(it, u, q, evicted[u])
            assert list(sel_idx[u, :sel_cnt[u]]) == list(ref.sel), f"unit {u} step {t}: selection"
            if w.policies[u].mode == MODE_NOSA:
                evicted[u] = np.pad(ref.evicted, (0, w.n_cap(u) - len(ref.evicted)))
            moved_ref[u] = mirror.step(u, ref.sel, lens[u // w.num_kv_heads])
        total_moved += int(moved_ref.sum())
        _check(plan, w, inp, ws, mirror, lens, moved_ref, f"step {t}")
    assert total_moved > 0
    assert fx.fx_read_error(plan) == 0


def test_compaction_bad_slot_map_is_flagged_not_faulting():
    """A slot row naming one block twice (state the call never writes) leaves blocks
    without a slot and sets FX_ERR_SLOT_MAP; out-of-range selection entries are skipped."""
    pols = [HeadPolicy(MODE_RETRIEVAL, block=16, sub_block=4, top_k=2)] * 2
    w = _custom("compact_bad", 1, 4, 2, 128, "bf16", 1024, [1000], pols)
    say("[compact] bad slot map")
    inp = generate(w, DEV)
    plan = make_plan(w)
    bufs = fx.allocate_step_buffers(plan, DEV)
    ws = fx.allocate_working_set(plan, DEV)
    n = fx.fx_unit_max_selected(plan, 0)
    assert n == 4
    bufs.sel_idx.fill_(-1)
    bufs.sel_idx[0, :4] = torch.tensor([1, 2, 3, 4], dtype=torch.int32)
    bufs.sel_cnt.copy_(torch.tensor([4, 2], dtype=torch.int32))
    bufs.sel_idx[1, :2] = torch.tensor([5, 900], dtype=torch.int32)     # 900: no such block
    ws.slot_map[0, :4] = torch.tensor([2, 2, -1, -1], dtype=torch.int32)
    fx.fx_compact_update(plan, inp.K, inp.V, inp.seq_lens, bufs.sel_idx, bufs.sel_cnt, ws,
                         bufs.workspace)
    torch.cuda.synchronize()
    err = fx.fx_read_error(plan)
    assert err == fx.FX_ERR_SLOT_MAP | fx.FX_ERR_SEL_INDEX, err
    row = ws.slot_map[0].cpu().tolist()
    assert row[:2] == [2, 2] and sorted(row[2:4]) == [1, 3]   # 1 and 3 placed; 4 left out
    assert ws.slot_map[1].cpu().tolist()[:1] == [5]


def test_compaction_refuses_large_selection_bounds():
    pols = [HeadPolicy(MODE_RETRIEVAL, block=1, sub_block=1, top_k=3000)]
    w = _custom("compact_big", 1, 1, 1, 64, "f32", 4096, [4096], pols)
    inp = generate(w, DEV)
    plan = make_plan(w)
    assert plan.max_selected > 2048
    bufs = fx.allocate_step_buffers(plan, DEV)
    ws = fx.allocate_working_set(plan, DEV)
    with pytest.raises(fx.FxError) as e:
        fx.fx_compact_update(plan, inp.K, inp.V, inp.seq_lens, bufs.sel_idx, bufs.sel_cnt, ws,
                             bufs.workspace)
    assert e.value.status == 2
