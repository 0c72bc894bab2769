"""Bad or extreme device data against the documented rules (needs an MI355X).

* fx_selection_delta and fx_select_delta read each list as its longest prefix that is
  strictly ascending within the unit's block slots; entries past it are ignored and set
  FX_ERR_SEL_INDEX.  The expected differences are the oracle's set differences of those
  prefixes.
* A +-inf score or eviction logit ranks as the largest / smallest value and sets
  FX_ERR_NONFINITE: the selection equals the one with the infinity replaced by a huge
  finite value of the same sign (which sets no flag).
"""
import numpy as np
import pytest
import torch

import block_sparse_decode_summary_amd as fx
from oracle.delta import selection_delta
from workloads import HeadPolicy, MODE_NOSA, MODE_RETRIEVAL, Workload, generate, small_workload

from gpu_harness import INT32_MAX, make_plan, say

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _valid_prefix(lst, n_cap):
    out = []
    for i, x in enumerate(lst):
        if not (0 <= x < n_cap) or (i > 0 and lst[i - 1] >= x):
            break
        out.append(int(x))
    return out


def _delta_case():
    pol = HeadPolicy(MODE_RETRIEVAL, block=16, sub_block=16, top_k=30)
    w = Workload(name="delta_prefix", batch=2, num_q_heads=4, num_kv_heads=2, head_dim=64,
                 dtype="bf16", t_cap=16 * 100, seq_lens=(1600, 1600), policies=(pol,) * 4,
                 seed=77, sink_scaled_tokens=4, needles_per_head=2)
    return w, make_plan(w)


def test_selection_delta_uses_the_valid_prefix():
    w, plan = _delta_case()
    ms, n_cap = plan.max_selected, 100
    rows = {
        # prev, cur
        0: ([1, 5, 9, 12], [1, 7, 9, 40]),                  # all valid
        1: ([2, 8, 500, 9, 30], [2, 9, 30]),                # out of range in the middle
        2: ([3, 6, 6, 10], [4, 3, 10]),                     # repeat in prev; cur not ascending
        3: ([-1, 4, 5], [0, 99, 100]),                      # negative first; 100 == n_cap
    }
    prev = np.full((4, ms), -1, np.int32)
    cur = np.full((4, ms), -1, np.int32)
    pc = np.zeros(4, np.int32)
    cc = np.zeros(4, np.int32)
    for u, (a, c) in rows.items():
        prev[u, :len(a)], pc[u] = a, len(a)
        cur[u, :len(c)], cc[u] = c, len(c)
    bufs = fx.allocate_step_buffers(plan, DEV)
    t = lambda x: torch.from_numpy(x).to(DEV)
    fx.fx_selection_delta(plan, t(prev), t(pc), t(cur), t(cc), bufs.added, bufs.added_cnt,
                          bufs.removed, bufs.removed_cnt)
    torch.cuda.synchronize()
    assert fx.fx_read_error(plan) == fx.FX_ERR_SEL_INDEX
    for u, (a, c) in rows.items():
        pa, ca = _valid_prefix(a, n_cap), _valid_prefix(c, n_cap)
        ar, rr = selection_delta(np.array(pa, np.int64), np.array(ca, np.int64))
        got_a = bufs.added[u, :bufs.added_cnt[u]].cpu().tolist()
        got_r = bufs.removed[u, :bufs.removed_cnt[u]].cpu().tolist()
        assert got_a == list(ar), (u, got_a, list(ar))
        assert got_r == list(rr), (u, got_r, list(rr))
        assert np.all(bufs.added[u, len(ar):].cpu().numpy() == -1)
    # Only valid lists: no flag.
    fx.fx_selection_delta(plan, t(prev[:1].repeat(4, 0)), t(pc[:1].repeat(4)),
                          t(cur[:1].repeat(4, 0)), t(cc[:1].repeat(4)), bufs.added,
                          bufs.added_cnt, bufs.removed, bufs.removed_cnt)
    assert fx.fx_read_error(plan) == 0


def test_fused_delta_uses_the_valid_prefix():
    """fx_select_delta on the register path reads the previous selection the same way."""
    w = small_workload("qwen7b_layer")
    say("[edges] fused delta, bad entry in the middle of the previous selection")
    inp = generate(w, DEV)
    plan = make_plan(w)
    B = fx.allocate_step_buffers(plan, DEV)
    fx.fx_build_summaries(plan, inp.K, inp.seq_lens, 0, INT32_MAX, B.summaries)
    fx.fx_select(plan, inp.q, B.summaries, None, None, inp.seq_lens, B.sel_idx, B.sel_cnt,
                 B.workspace)
    sel = B.sel_idx.cpu().numpy().copy()
    cnt = B.sel_cnt.cpu().numpy().copy()
    prev = sel.copy()
    mid = int(cnt[0]) // 2
    prev[0, mid] = prev[0, mid - 1]              # a repeat: entries from mid on are ignored
    B.prev_idx.copy_(torch.from_numpy(prev))
    B.prev_cnt.copy_(B.sel_cnt)
    fx.fx_select_delta(plan, inp.q, B.summaries, None, None, inp.seq_lens, B.prev_idx,
                       B.prev_cnt, B.sel_idx, B.sel_cnt, B.added, B.added_cnt, B.removed,
                       B.removed_cnt, B.workspace)
    torch.cuda.synchronize()
    assert fx.fx_read_error(plan) == fx.FX_ERR_SEL_INDEX
    assert np.array_equal(B.sel_idx.cpu().numpy(), sel)
    ac = B.added_cnt.cpu().numpy()
    rc = B.removed_cnt.cpu().numpy()
    assert list(B.added[0, :ac[0]].cpu()) == list(sel[0, mid:cnt[0]])
    assert rc[0] == 0 and np.all(ac[1:] == 0) and np.all(rc[1:] == 0)


def _plant(t: torch.Tensor, index, value: float):
    t.view(-1)[index] = value


@pytest.mark.parametrize("which", ["score", "logit"])
@pytest.mark.parametrize("sign", [1.0, -1.0])
def test_infinities_rank_by_sign_and_are_flagged(which, sign):
    pols = (HeadPolicy(MODE_RETRIEVAL, block=16, sub_block=16, top_k=6),
            HeadPolicy(MODE_NOSA, block=16, sub_block=16, top_k=3, k_evict=5))
    lens = (16 * 200, 16 * 200 - 3)
    w = Workload(name="inf", batch=2, num_q_heads=4, num_kv_heads=2, head_dim=128, dtype="bf16",
                 t_cap=16 * 200, seq_lens=lens, policies=pols * 2, seed=91,
                 sink_scaled_tokens=4, needles_per_head=2)
    inp = generate(w, DEV)
    plan = make_plan(w)
    say(f"[edges] {sign:+.0f} inf {which}")
    results = []
    for value in (sign * float("inf"), sign * 1.0e30):
        bufs = fx.allocate_step_buffers(plan, DEV)
        fx.fx_build_summaries(plan, inp.K, inp.seq_lens, 0, INT32_MAX, bufs.summaries)
        logits = inp.logits.clone()
        if which == "score":
            # Block 50 of unit 0 (retrieval): one summary element set so that the score
            # is +-value (the element's query-sum column is made positive).
            qs = inp.q[0, 0:2].float().sum(0)
            c = int(torch.argmax(qs).item())
            row = fx.fx_unit_summary_offset(plan, 0) + 50
            bufs.summaries.view(-1, w.head_dim)[row].zero_()
            bufs.summaries.view(-1, w.head_dim)[row, c] = value
        else:
            _plant(logits, plan.unit_block_offset(3) + 60, value)     # unit 3 (NOSA)
        fx.fx_select(plan, inp.q, bufs.summaries, logits, bufs.evicted_mask, inp.seq_lens,
                     bufs.sel_idx, bufs.sel_cnt, bufs.workspace)
        torch.cuda.synchronize()
        results.append((fx.fx_read_error(plan), bufs.sel_idx.cpu().numpy().copy(),
                        bufs.sel_cnt.cpu().numpy().copy(), bufs.evicted_mask.cpu().numpy().copy()))
    (err_inf, sel_inf, cnt_inf, ev_inf), (err_fin, sel_fin, cnt_fin, ev_fin) = results
    assert err_inf == fx.FX_ERR_NONFINITE and err_fin == 0
    assert np.array_equal(cnt_inf, cnt_fin) and np.array_equal(sel_inf, sel_fin)
    assert np.array_equal(ev_inf, ev_fin)
    if which == "score":
        assert (50 in sel_inf[0, :cnt_inf[0]]) == (sign > 0)
    elif sign > 0:
        assert 60 in sel_inf[3, :cnt_inf[3]]            # first in Γe
    else:
        word = int(w.mask_word_offsets()[3]) + 60 // 32   # last in Γe order: evicted
        assert (int(ev_inf[word]) >> (60 % 32)) & 1
