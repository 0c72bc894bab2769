"""Plant plausible mistakes in copies of oracle functions and check that the pins catch them.

Every mutant here is a CPU-only variant of an oracle function; a pin that let one
through would not be pinning that function.
"""
import math

import numpy as np
import pytest

from oracle import attention, compaction, delta, numerics, pooling, scoring, selection

import oracle_pins as pins


def _fails(check, *args):
    try:
        check(*args)
    except (AssertionError, ValueError, IndexError):
        return True
    return False


# ---- numerics -------------------------------------------------------------------------

def _bf16_via_f32(x):                     # double rounding through float32
    import torch
    t = torch.from_numpy(np.asarray(x, dtype=np.float64).astype(np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def _bf16_round_half_up(x):
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)
    q = np.maximum(e - 8, -133)
    return np.ldexp(np.floor(np.ldexp(x, -q) + 0.5), q)


def _bf16_truncate(x):
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)
    q = np.maximum(e - 8, -133)
    return np.ldexp(np.trunc(np.ldexp(x, -q)), q)


@pytest.mark.parametrize("mutant", ["double_rounding", "half_up", "truncate"])
def test_bf16_mutants(mutant):
    if mutant == "double_rounding":
        args = (_bf16_via_f32, lambda x: numerics.bf16_bits_to_f64(_bf16_via_f32(x)))
    elif mutant == "half_up":
        args = (lambda x: numerics.f64_to_bf16_bits(_bf16_round_half_up(x)), _bf16_round_half_up)
    else:
        args = (lambda x: numerics.f64_to_bf16_bits(_bf16_truncate(x)), _bf16_truncate)
    assert _fails(pins.check_bf16_rounding, *args)


# ---- pooling --------------------------------------------------------------------------

def _pool_swapped(K, g, s, dtype):        # max inside sub-blocks, mean across them
    n = K.shape[0] // g
    x = K[: n * g].reshape(n, g // s, s, -1)
    return numerics.round_to_storage(x.max(axis=2).mean(axis=1), dtype)


def _pool_off_by_one(K, g, s, dtype):     # drops the last row of each sub-block
    n = K.shape[0] // g
    x = K[: n * g].reshape(n, g // s, s, -1)
    return numerics.round_to_storage((x[:, :, : max(1, s - 1)].sum(axis=2) / s).max(axis=1), dtype)


def _pool_includes_partial(K, g, s, dtype):
    T = K.shape[0]
    pad = (-T) % g
    Kp = np.concatenate([K, np.repeat(K[-1:], pad, axis=0)]) if pad else K
    return pooling.block_summaries(Kp, g, s, dtype)


def _pool_double_round(K, g, s, dtype):   # rounds through float32 before bfloat16
    n = K.shape[0] // g
    x = K[: n * g].reshape(n, g // s, s, -1)
    m = (x.sum(axis=2) / s).max(axis=1)
    if dtype == "bf16":
        return numerics.bf16_bits_to_f64(_bf16_via_f32(m))
    return numerics.round_to_storage(m, dtype)


@pytest.mark.parametrize("mutant", [_pool_swapped, _pool_off_by_one, _pool_includes_partial])
def test_pooling_mutants(mutant):
    assert _fails(pins.check_pooling, mutant)


def test_pooling_double_rounding_is_a_real_difference():
    """A block whose exact sub-block mean sits just above a bfloat16 tie."""
    rows = np.zeros((16, 1))
    rows[:14, 0] = 1.0
    rows[14, 0] = 1.0 + 2 ** -5
    rows[15, 0] = 2.0 ** -36
    good = pooling.block_summaries(rows, 16, 16, "bf16")[0, 0]
    bad = _pool_double_round(rows, 16, 16, "bf16")[0, 0]
    assert good == 241 * 2.0 ** -8 and bad == 240 * 2.0 ** -8


# ---- scoring --------------------------------------------------------------------------

def _score_first_row_only(q, S):
    return scoring.block_scores(q[:1], S)


def _score_mean_of_rows(q, S):
    return (scoring.block_scores(q, S).astype(np.float64) / q.shape[0]).astype(np.float32)


def _score_wrong_column(q, S):
    return scoring.block_scores(q, np.roll(S, 1, axis=1))


def _score_accumulate_f32(q, S):
    qs = np.asarray(q, np.float64).sum(axis=0).astype(np.float32)
    acc = np.zeros(S.shape[0], dtype=np.float32)
    for c in range(S.shape[1]):
        acc = acc + qs[c] * S[:, c].astype(np.float32)
    return acc


@pytest.mark.parametrize("mutant", [_score_first_row_only, _score_mean_of_rows,
                                    _score_wrong_column, _score_accumulate_f32])
def test_scoring_mutants(mutant):
    assert _fails(pins.check_scoring, mutant)


# ---- selection ------------------------------------------------------------------------

def _forced_no_partial(pol, T):
    F = selection.forced_blocks(pol, T)
    g = pol.block
    if T % g and pol.mode != 1:
        n_tot = -(-T // g)
        if not pol.force_last:
            F = F[F != n_tot - 1]
    return F


def _forced_local_off_by_one(pol, T):
    if pol.mode != 1 or pol.local_tokens == 0:
        return selection.forced_blocks(pol, T)
    g = pol.block
    n_tot = -(-T // g)
    F = set(range(0, -(-min(pol.sink_tokens, T) // g)))
    F.update(range(max(0, T - pol.local_tokens) // g + 1, n_tot))
    if T % g:
        F.add(n_tot - 1)
    return np.array(sorted(F), dtype=np.int64)


@pytest.mark.parametrize("mutant", [_forced_no_partial, _forced_local_off_by_one])
def test_forced_mutants(mutant):
    assert _fails(pins.check_forced, mutant)


def _budget_floor(pol, n_tot):
    if pol.top_k > 0:
        return pol.top_k
    return int(math.floor(float(np.float32(pol.budget)) * n_tot))


def _budget_round(pol, n_tot):
    if pol.top_k > 0:
        return pol.top_k
    return int(round(float(np.float32(pol.budget)) * n_tot + 0.5))


@pytest.mark.parametrize("mutant", [_budget_floor, _budget_round])
def test_budget_mutants(mutant):
    assert _fails(pins.check_budget, mutant)


def _topk_ties_high(values, cand, k):
    cand = np.asarray(cand, dtype=np.int64)
    k = min(int(k), cand.size)
    if k <= 0:
        return np.zeros(0, np.int64)
    v = np.asarray(values, np.float32)[cand].astype(np.float64)
    order = np.lexsort((-cand, -v))
    return np.sort(cand[order[:k]])


def _topk_ascending(values, cand, k):
    cand = np.asarray(cand, dtype=np.int64)
    k = min(int(k), cand.size)
    if k <= 0:
        return np.zeros(0, np.int64)
    v = np.asarray(values, np.float32)[cand].astype(np.float64)
    order = np.lexsort((cand, v))
    return np.sort(cand[order[:k]])


def _topk_signed_zero(values, cand, k):   # orders -0.0 below +0.0 (bitwise order)
    cand = np.asarray(cand, dtype=np.int64)
    k = min(int(k), cand.size)
    if k <= 0:
        return np.zeros(0, np.int64)
    v = np.asarray(values, np.float32)[cand]
    key = v.astype(np.float64) + np.where(np.signbit(v) & (v == 0), -1e-300, 0.0)
    order = np.lexsort((cand, -key))
    return np.sort(cand[order[:k]])


@pytest.mark.parametrize("mutant", [_topk_ties_high, _topk_ascending, _topk_signed_zero])
def test_top_k_mutants(mutant):
    assert _fails(pins.check_top_k, mutant)


def _select_no_forced(pol, T, scores=None, logits=None, evicted=None):
    if pol.mode == 0:
        n_full = T // pol.block
        chosen = selection.top_k(scores, np.arange(n_full), selection.budget_k(pol, -(-T // pol.block)))
        return chosen, evicted
    return selection.select_unit(pol, T, scores, logits, evicted)


def _select_nosa_evicted_not_eligible(pol, T, scores=None, logits=None, evicted=None):
    if pol.mode != 2:
        return selection.select_unit(pol, T, scores, logits, evicted)
    n_full = T // pol.block
    ev = np.zeros(n_full, bool) if evicted is None else np.asarray(evicted, bool).copy()
    full = np.arange(n_full)
    E = full[~ev[:n_full]]
    ge = selection.top_k(logits, E, pol.k_evict)
    ev[np.setdiff1d(E, ge)] = True
    cand_q = full[~ev[:n_full]]
    cand_q = np.setdiff1d(cand_q, ge)
    gq = selection.top_k(scores, cand_q, pol.top_k)
    return np.union1d(ge, gq), ev


def _select_nosa_no_strict_eviction(pol, T, scores=None, logits=None, evicted=None):
    if pol.mode != 2:
        return selection.select_unit(pol, T, scores, logits, evicted)
    return selection.select_unit(pol, T, scores, logits, None)


@pytest.mark.parametrize("mutant,check", [
    (_select_no_forced, pins.check_select_retrieval),
    (_select_nosa_evicted_not_eligible, pins.check_select_nosa),
    (_select_nosa_no_strict_eviction, pins.check_select_nosa),
])
def test_select_mutants(mutant, check):
    assert _fails(check, mutant)


# ---- score-side pooling ---------------------------------------------------------------

def _means_unrounded(K, g, s, dtype):          # the exact means, never rounded
    return pooling._exact_means(K, g, s, dtype)


def _means_via_f32(K, g, s, dtype):            # double rounding through float32
    m = pooling._exact_means(K, g, s, dtype)
    if dtype != "bf16":
        return m
    return numerics.round_f64_to_bf16(m.astype(np.float32).astype(np.float64))


def _means_last_dropped(K, g, s, dtype):       # the last sub-block repeats the one before
    m = pooling.sub_block_means(K, g, s, dtype)
    if m.shape[1] > 1:
        m[:, -1] = m[:, -2]
    return m


@pytest.mark.parametrize("mutant", [_means_unrounded, _means_via_f32, _means_last_dropped])
def test_sub_block_means_mutants(mutant):
    assert _fails(pins.check_sub_block_means, mutant, pooling.block_summaries)


def _scores_key_side(q, M, pool):              # max over the means before scoring
    return scoring.block_scores(q, np.asarray(M).max(axis=1))


def _scores_mean_over_sub_blocks(q, M, pool):
    M = np.asarray(M, dtype=np.float64)
    if pool == scoring.POOL_SCORE_SUM:
        return scoring._chain(scoring.group_query_sum(q), M).mean(axis=1).astype(np.float32)
    return scoring.sub_block_scores(q, M, pool)


def _scores_aggregations_swapped(q, M, pool):
    other = scoring.POOL_SCORE_MAX if pool == scoring.POOL_SCORE_SUM else scoring.POOL_SCORE_SUM
    return scoring.sub_block_scores(q, M, other)


def _scores_max_agg_first_row_only(q, M, pool):
    if pool == scoring.POOL_SCORE_MAX:
        return scoring.sub_block_scores(np.asarray(q)[:1], M, scoring.POOL_SCORE_SUM)
    return scoring.sub_block_scores(q, M, pool)


def _scores_min_over_sub_blocks(q, M, pool):
    return -scoring.sub_block_scores(q, -np.asarray(M, dtype=np.float64), pool) \
        if pool == scoring.POOL_SCORE_SUM else scoring.sub_block_scores(q, M, pool)


@pytest.mark.parametrize("mutant", [_scores_key_side, _scores_mean_over_sub_blocks,
                                    _scores_aggregations_swapped, _scores_max_agg_first_row_only,
                                    _scores_min_over_sub_blocks])
def test_sub_block_scores_mutants(mutant):
    assert _fails(pins.check_sub_block_scores, mutant, scoring.block_scores,
                  scoring.POOL_SCORE_SUM, scoring.POOL_SCORE_MAX)


# ---- attention ------------------------------------------------------------------------

def _attend_no_scale(q, K, V, scale):
    return attention.attend(q, K, V, 1.0)


def _attend_no_max_shift_lse(q, K, V, scale):
    out, lse = attention.attend(q, K, V, scale)
    return out, lse - lse.max()


def _attend_keys_as_values(q, K, V, scale):
    return attention.attend(q, K, K, scale)


def _tokens_include_padding(sel, g, T):
    return np.concatenate([np.arange(j * g, (j + 1) * g) for j in np.asarray(sel)]) if len(sel) else np.zeros(0, np.int64)


@pytest.mark.parametrize("which", ["no_scale", "lse_shift", "kv_swap", "padding"])
def test_attention_mutants(which):
    att, tok = attention.attend, attention.selected_tokens
    if which == "no_scale":
        att = _attend_no_scale
    elif which == "lse_shift":
        att = _attend_no_max_shift_lse
    elif which == "kv_swap":
        att = _attend_keys_as_values
    else:
        tok = _tokens_include_padding
    assert _fails(pins.check_attention, att, tok, attention.merge_partials, attention.partial)


def _merge_no_rescale(parts):
    L = sum(p[1] for p in parts)
    O = sum(p[2] for p in parts)
    return O / L[:, None], np.log(L)


def test_merge_mutant():
    assert _fails(pins.check_attention, attention.attend, attention.selected_tokens,
                  _merge_no_rescale, attention.partial)


def _attend_bias_scaled(q, K, V, scale, bias=None):       # (q.k + b) * scale
    return attention.attend(q, K, V, scale, None if bias is None else np.asarray(bias) * scale)


def _attend_bias_ignored(q, K, V, scale, bias=None):
    return attention.attend(q, K, V, scale)


def _attend_bias_negated(q, K, V, scale, bias=None):
    return attention.attend(q, K, V, scale, None if bias is None else -np.asarray(bias))


def _attend_bias_after_exp(q, K, V, scale, bias=None):    # weights scaled by b, not e^b
    if bias is None or len(bias) == 0:
        return attention.attend(q, K, V, scale)
    s = (np.asarray(q) @ np.asarray(K).T) * scale
    p = np.exp(s - s.max(axis=1, keepdims=True)) * np.asarray(bias)[None, :]
    l = p.sum(axis=1, keepdims=True)
    return (p @ np.asarray(V)) / l, s.max(axis=1) + np.log(np.abs(l[:, 0]))


def _partial_bias_ignored(q, K, V, scale, bias=None):
    return attention.partial(q, K, V, scale)


def _token_bias_by_position(sel, g, T, logits):           # b indexed by selection rank
    sel = np.asarray(sel)
    parts = [np.full(min((j + 1) * g, T) - j * g, float(logits[i])) for i, j in enumerate(sel)]
    return np.concatenate(parts) if parts else np.zeros(0)


def _token_bias_full_blocks(sel, g, T, logits):           # ignores the partial last block
    parts = [np.full(g, float(logits[j])) for j in np.asarray(sel)]
    return np.concatenate(parts) if parts else np.zeros(0)


@pytest.mark.parametrize("which", ["scaled", "ignored", "negated", "after_exp", "partial",
                                   "by_position", "full_blocks"])
def test_biased_attention_mutants(which):
    att, tb, part = attention.attend, attention.token_bias, attention.partial
    if which == "scaled":
        att = _attend_bias_scaled
    elif which == "ignored":
        att = _attend_bias_ignored
    elif which == "negated":
        att = _attend_bias_negated
    elif which == "after_exp":
        att = _attend_bias_after_exp
    elif which == "partial":
        part = _partial_bias_ignored
    elif which == "by_position":
        tb = _token_bias_by_position
    else:
        tb = _token_bias_full_blocks
    assert _fails(pins.check_biased_attention, att, tb, attention.selected_tokens,
                  attention.merge_partials, part)


# ---- compaction -----------------------------------------------------------------------

def _compact_free_descending(slot_map, sel, T, g):
    slots = np.array(slot_map, dtype=np.int64, copy=True)
    target = compaction.held_target(sel, T, g)
    for s in range(slots.size):
        if slots[s] >= 0 and slots[s] not in target:
            slots[s] = -1
    added = [int(b) for b in target if b not in slots]
    free = [s for s in range(slots.size) if slots[s] < 0][::-1]
    moves = sorted(zip(free[:len(added)], added))
    for s, b in moves:
        slots[s] = b
    return slots, moves


def _compact_move_everything(slot_map, sel, T, g):          # re-copies held blocks too
    target = compaction.held_target(sel, T, g)
    slots = np.full(len(slot_map), -1)
    moves = [(i, int(b)) for i, b in enumerate(target)]
    for s, b in moves:
        slots[s] = b
    return slots, moves


def _compact_holds_partial(slot_map, sel, T, g):            # the growing block is held too
    return compaction.compact_update(slot_map, sel, T + g - 1 if T % g else T, g)


def _compact_no_free(slot_map, sel, T, g):                  # deselected blocks keep slots
    slots = np.array(slot_map, dtype=np.int64, copy=True)
    target = compaction.held_target(sel, T, g)
    added = [int(b) for b in target if b not in slots]
    free = [s for s in range(slots.size) if slots[s] < 0]
    if len(added) > len(free):
        raise ValueError("full")
    moves = list(zip(free[:len(added)], added))
    for s, b in moves:
        slots[s] = b
    return slots, moves


def _apply_moves_keys_only(wK, wV, K, V, moves, g):
    for s, b in moves:
        wK[s * g:(s + 1) * g] = K[b * g:(b + 1) * g]


@pytest.mark.parametrize("which", ["free_desc", "move_all", "partial", "no_free", "keys_only"])
def test_compaction_mutants(which):
    cu, am = compaction.compact_update, compaction.apply_moves
    if which == "free_desc":
        cu = _compact_free_descending
    elif which == "move_all":
        cu = _compact_move_everything
    elif which == "partial":
        cu = _compact_holds_partial
    elif which == "no_free":
        cu = _compact_no_free
    else:
        am = _apply_moves_keys_only
    assert _fails(pins.check_compaction, cu, am, delta.selection_delta)


# ---- delta ----------------------------------------------------------------------------

def _delta_swapped(prev, cur):
    return delta.selection_delta(cur, prev)


def _delta_symmetric(prev, cur):
    a, r = delta.selection_delta(prev, cur)
    both = np.union1d(a, r)
    return both, both


@pytest.mark.parametrize("mutant", [_delta_swapped, _delta_symmetric])
def test_delta_mutants(mutant):
    assert _fails(pins.check_delta, mutant, delta.locality)
