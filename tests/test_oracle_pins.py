"""The CPU oracle against its pins (no GPU)."""
import numpy as np
import pytest

from oracle import attention, compaction, delta, numerics, pooling, scoring, selection
from oracle.step import unit_step

import oracle_pins as pins


def test_bf16_rounding():
    pins.check_bf16_rounding(numerics.f64_to_bf16_bits, numerics.round_f64_to_bf16)


def test_pooling():
    pins.check_pooling(pooling.block_summaries)


def test_pooling_refuses_inexact_sums():
    K = np.zeros((16, 2))
    K[0, 0] = 1.0
    K[1, 0] = 2.0 ** -40          # float32 values whose float64 sum would need > 53 bits
    K[2, 0] = 2.0 ** 20
    with pytest.raises(ValueError):
        pooling.block_summaries(K, 16, 16, "f32")


def test_scoring():
    pins.check_scoring(scoring.block_scores)


def test_sub_block_means():
    pins.check_sub_block_means(pooling.sub_block_means, pooling.block_summaries)


def test_sub_block_scores():
    pins.check_sub_block_scores(scoring.sub_block_scores, scoring.block_scores,
                                scoring.POOL_SCORE_SUM, scoring.POOL_SCORE_MAX)


def test_forced_sets():
    pins.check_forced(selection.forced_blocks)


def test_budget():
    pins.check_budget(selection.budget_k)


def test_top_k():
    pins.check_top_k(selection.top_k)


def test_select_retrieval():
    pins.check_select_retrieval(selection.select_unit)


def test_select_nosa():
    pins.check_select_nosa(selection.select_unit)


def test_attention():
    pins.check_attention(attention.attend, attention.selected_tokens,
                         attention.merge_partials, attention.partial)


def test_biased_attention():
    pins.check_biased_attention(attention.attend, attention.token_bias, attention.selected_tokens,
                                attention.merge_partials, attention.partial)


def test_unit_step_ed_biases_nosa_units_only():
    """ED-DMA: a NOSA unit's tokens carry their block's eviction logit; the other modes
    have no eviction head, so the switch changes nothing for them."""
    rng = np.random.default_rng(22)
    G, d, T, g = 2, 16, 150, 16
    q = pins.random_bf16_values(rng, (G, d))
    K = pins.random_bf16_values(rng, (T, d))
    V = pins.random_bf16_values(rng, (T, d))
    logits = rng.standard_normal(-(-T // g)).astype(np.float32)
    scale = d ** -0.5
    for pol in (pins.Pol(mode=0, block=g, sub_block=4, top_k=3, force_sink=1, force_last=1),
                pins.Pol(mode=1, block=g, sub_block=4, sink_tokens=16, local_tokens=40)):
        a = unit_step(pol, T, "bf16", q, K, V, scale, logits=logits)
        b = unit_step(pol, T, "bf16", q, K, V, scale, logits=logits, ed=True)
        assert np.array_equal(a.out_exact, b.out_exact) and np.array_equal(a.lse, b.lse)
    pol = pins.Pol(mode=2, block=g, sub_block=4, top_k=2, k_evict=3, force_sink=1, force_last=1)
    ev = np.zeros(-(-T // g), dtype=bool)
    a = unit_step(pol, T, "bf16", q, K, V, scale, logits=logits, evicted=ev.copy())
    b = unit_step(pol, T, "bf16", q, K, V, scale, logits=logits, evicted=ev.copy(), ed=True)
    assert np.array_equal(a.sel, b.sel) and np.array_equal(a.evicted, b.evicted)
    tok = attention.selected_tokens(b.sel, g, T)
    bias = np.concatenate([np.full(min((j + 1) * g, T) - j * g, float(logits[j])) for j in b.sel])
    assert np.allclose(b.out_exact, pins._dense_additive(q, K, V, tok, bias, scale),
                       rtol=1e-12, atol=1e-12)
    assert not np.allclose(a.out_exact, b.out_exact)


def test_unit_step_score_side_pooling():
    """End to end: with sub_block = block the group-sum score-side pooling is key-side
    pooling; with smaller sub-blocks the summaries keep every mean and the max moves to
    the scores."""
    rng = np.random.default_rng(25)
    G, d, T = 4, 32, 700
    q = pins.random_bf16_values(rng, (G, d))
    K = pins.random_bf16_values(rng, (T, d))
    V = pins.random_bf16_values(rng, (T, d))
    scale = d ** -0.5
    pol = pins.Pol(mode=0, block=32, sub_block=32, top_k=4, force_sink=1, force_last=1)
    a = unit_step(pol, T, "bf16", q, K, V, scale)
    b = unit_step(pol, T, "bf16", q, K, V, scale, pooling=scoring.POOL_SCORE_SUM)
    assert np.array_equal(a.scores, b.scores) and np.array_equal(a.sel, b.sel)
    assert np.array_equal(b.summaries[:, 0, :], a.summaries)
    pol = pins.Pol(mode=0, block=32, sub_block=8, top_k=4)
    for pool in (scoring.POOL_SCORE_SUM, scoring.POOL_SCORE_MAX):
        r = unit_step(pol, T, "bf16", q, K, V, scale, pooling=pool)
        assert r.summaries.shape == (T // 32, 4, d)
        assert np.array_equal(r.scores, scoring.sub_block_scores(
            q, pooling.sub_block_means(K, 32, 8, "bf16"), pool))


def test_compaction():
    pins.check_compaction(compaction.compact_update, compaction.apply_moves, delta.selection_delta)


def test_delta():
    pins.check_delta(delta.selection_delta, delta.locality)


def test_unit_step_dense_when_budget_covers_everything():
    """End to end: budget >= all blocks, and block size 1 with k = n, are dense attention."""
    rng = np.random.default_rng(20)
    G, d, T = 2, 16, 100
    q = pins.random_bf16_values(rng, (G, d))
    K = pins.random_bf16_values(rng, (T, d))
    V = pins.random_bf16_values(rng, (T, d))
    scale = d ** -0.5
    dense = pins._dense_masked(q, K, V, np.arange(T), scale)
    for pol in (pins.Pol(mode=0, block=16, sub_block=4, top_k=1000),
                pins.Pol(mode=0, block=1, sub_block=1, top_k=T)):
        r = unit_step(pol, T, "bf16", q, K, V, scale)
        assert list(r.sel) == list(range(-(-T // pol.block)))
        assert np.allclose(r.out_exact, dense, rtol=1e-12, atol=1e-12)
