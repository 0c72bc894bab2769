"""Score-side pooling (FX_POOL_SCORE_SUM / FX_POOL_SCORE_MAX) vs the CPU oracle.

[NOSA-DE] Methodik §1, "Blockweise Implementierung", read with the block-level max taken
over scores: the summaries keep every sub-block mean (rounded once), and a block's score
is the max over them of the group's summed dot product, or of the max over the group's
rows.  Same bar as the key-side path: summaries, scores, selections, masks and deltas bit
for bit, out and lse within the decode tolerances.
"""
import numpy as np
import pytest
import torch

import block_sparse_decode_summary_amd as fx
from workloads import (HeadPolicy, MODE_NOSA, MODE_RETRIEVAL, MODE_STREAMING, Workload, generate,
                       get_workload, query_at_step, small_workload)

from gpu_harness import INT32_MAX, GpuView, compare_unit, make_plan, oracle_unit, say
from test_gpu_parity import _run_and_compare_all

pytestmark = pytest.mark.gpu
DEV = "cuda"
POOLS = [fx.FX_POOL_SCORE_SUM, fx.FX_POOL_SCORE_MAX]


def _custom(name, batch, Hq, Hkv, d, dtype, t_cap, lens, pols, pooling, seed=70):
    return Workload(name=name, batch=batch, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=d,
                    dtype=dtype, t_cap=t_cap, seq_lens=tuple(lens), policies=tuple(pols), seed=seed,
                    sink_scaled_tokens=4, needles_per_head=2, steps=2, drift=(0.9, 0.44),
                    pooling=pooling)


@pytest.mark.parametrize("pooling", POOLS)
@pytest.mark.parametrize("name", ["tiny", "llama8b_layer", "qwen7b_layer", "nosa_drift",
                                  "mixed_serving"])
def test_pooling_small_workloads(name, pooling):
    w = small_workload(name).replace(pooling=pooling)
    w = w.replace(name=f"{w.name}_pool{pooling}")
    _run_and_compare_all(w, steps=min(w.steps, 4))


@pytest.mark.parametrize("G,d,dtype", [(1, 128, "bf16"), (3, 64, "bf16"), (8, 128, "bf16"),
                                       (5, 128, "f32")])
@pytest.mark.parametrize("pooling", POOLS)
def test_pooling_rows_per_block_and_groups(G, d, dtype, pooling):
    """r = block / sub_block from 1 to 64, ragged and degenerate lengths, all modes."""
    lens = [0, 1, 63, 64, 700, 4000]
    pols = []
    for _ in lens:
        pols += [HeadPolicy(MODE_RETRIEVAL, block=64, sub_block=64, top_k=3, force_sink=1,
                            force_last=1),                                          # r = 1
                 HeadPolicy(MODE_RETRIEVAL, block=64, sub_block=32, top_k=4),         # r = 2
                 HeadPolicy(MODE_NOSA, block=64, sub_block=4, top_k=2, k_evict=3),    # r = 16
                 HeadPolicy(MODE_RETRIEVAL, block=256, sub_block=4, top_k=2,
                            force_last=1),                                          # r = 64
                 HeadPolicy(MODE_NOSA, block=16, sub_block=1, top_k=3, k_evict=2),    # r = 16
                 HeadPolicy(MODE_STREAMING, block=32, sub_block=8, sink_tokens=4, local_tokens=50)]
    w = _custom(f"pool{pooling}_g{G}_d{d}_{dtype}", len(lens), 6 * G, 6, d, dtype, 4096, lens,
                pols, pooling)
    _run_and_compare_all(w, steps=2)


@pytest.mark.parametrize("name,pooling", [("nosa_drift", fx.FX_POOL_SCORE_SUM),
                                          ("mixed_serving", fx.FX_POOL_SCORE_MAX)])
def test_pooling_full_size_sampled(name, pooling):
    """Full workload sizes in the benchmark's launch configuration; sampled units."""
    w = get_workload(name).replace(pooling=pooling)
    say(f"[pool] {name} pooling {pooling}: B={w.batch} t_cap={w.t_cap}")
    inp = generate(w, DEV)
    plan = make_plan(w)
    bufs = fx.allocate_step_buffers(plan, DEV)
    for u in (0, 7, w.num_units - 1):
        assert fx.fx_unit_summary_offset(plan, u) == int(w.summary_row_offsets()[u])
    assert plan.summary_bytes == int(w.summary_row_offsets()[-1]) * w.head_dim * w.elem_bytes
    rng = np.random.default_rng(400)
    units = sorted(set([0, w.num_units - 1] + list(rng.choice(w.num_units, 6, replace=False))))
    evicted = {u: None for u in units}
    for t in range(2 if w.drift else 1):
        q = query_at_step(w, t, DEV) if t > 0 else inp.q
        say(f"[pool] {name}: step {t}, units {units}")
        if t == 0:
            fx.fx_build_summaries(plan, inp.K, inp.seq_lens, 0, INT32_MAX, bufs.summaries)
        fx.fx_select(plan, q, bufs.summaries, inp.logits,
                     bufs.evicted_mask if w.has_nosa else None, inp.seq_lens, bufs.sel_idx,
                     bufs.sel_cnt, bufs.workspace)
        fx.fx_sparse_decode(plan, q, inp.K, inp.V, inp.seq_lens, bufs.sel_idx, bufs.sel_cnt,
                            w.head_dim ** -0.5, bufs.out, bufs.lse, bufs.workspace)
        gv = GpuView(plan, bufs, w)
        for u in units:
            ref = oracle_unit(inp, u, q, evicted[u])
            compare_unit(w, u, gv, ref)
            evicted[u] = ref.evicted
    assert fx.fx_read_error(plan) == 0
    del inp, bufs
    torch.cuda.empty_cache()


@pytest.mark.parametrize("pooling", POOLS)
def test_pooling_incremental_build(pooling):
    """Rebuilding only the newest block of each unit reproduces the full build."""
    w = small_workload("qwen7b_layer").replace(pooling=pooling)
    say(f"[pool] incremental build, pooling {pooling}")
    inp = generate(w, DEV)
    plan = make_plan(w)
    bufs = fx.allocate_step_buffers(plan, DEV)
    fx.fx_build_summaries(plan, inp.K, inp.seq_lens, 0, INT32_MAX, bufs.summaries)
    full = bufs.summaries.clone()
    bufs.summaries.zero_()
    fx.fx_build_summaries(plan, inp.K, inp.seq_lens, 0, -1, bufs.summaries)
    fx.fx_build_summaries(plan, inp.K, inp.seq_lens, -1, INT32_MAX, bufs.summaries)
    assert torch.equal(bufs.summaries, full)
    assert fx.fx_read_error(plan) == 0
