"""Pins for the CPU oracle, written as check functions.

Each ``check_*`` takes the oracle function(s) under test as arguments and raises
AssertionError when they disagree with something fixed independently of the
oracle: exact rational arithmetic (fractions.Fraction), brute force over tiny
inputs, closed forms, library routines (torch, numpy set algebra) or values
stated in the workload descriptions.  tests/test_oracle_pins.py runs them on the
real oracle; tests/test_oracle_mutations.py runs them on oracle copies with a
planted mistake and expects them to fail.
"""
from __future__ import annotations

import itertools
import json
import math
import os
from fractions import Fraction

import numpy as np
import torch

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def load_golden(name: str):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ----------------------------------------------------------------------------------------
# Exact rounding of rationals, written independently of oracle/numerics.py.
# ----------------------------------------------------------------------------------------

def fraction_round(x: Fraction, sig_bits: int, min_quantum_exp: int) -> Fraction:
    """Round a rational to ``sig_bits`` significant bits, ties to even (no overflow)."""
    if x == 0:
        return Fraction(0)
    sign = -1 if x < 0 else 1
    a = abs(x)
    # exponent E with 2**E <= a < 2**(E+1)
    E = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** E > a:
        E -= 1
    elif Fraction(2) ** (E + 1) <= a:
        E += 1
    qexp = max(E - (sig_bits - 1), min_quantum_exp)
    q = Fraction(2) ** qexp
    n = a / q
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return sign * fl * q


def fraction_to_bf16(x: Fraction) -> Fraction:
    return fraction_round(x, 8, -133)


def fraction_to_f32(x: Fraction) -> Fraction:
    return fraction_round(x, 24, -149)


def random_bf16_values(rng: np.random.Generator, shape, scale=1.0) -> np.ndarray:
    """float64 values that are exactly bfloat16 (via torch's float32 -> bfloat16 rounding)."""
    x = torch.from_numpy((rng.standard_normal(shape) * scale).astype(np.float32))
    return x.to(torch.bfloat16).to(torch.float64).numpy()


# ----------------------------------------------------------------------------------------
# numerics
# ----------------------------------------------------------------------------------------

def check_bf16_rounding(f64_to_bf16_bits, round_f64_to_bf16):
    rng = np.random.default_rng(11)
    # (1) float32-representable inputs: one rounding either way, so torch must agree.
    f32 = np.concatenate([
        rng.standard_normal(20000).astype(np.float32),
        (rng.standard_normal(2000) * 1e-39).astype(np.float32),     # float32 subnormals
        (rng.standard_normal(2000) * 1e37).astype(np.float32),
        np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8), 2 ** -126, 2 ** -133,
                  2 ** -134, 3 * 2 ** -134], dtype=np.float32),
    ])
    ref = torch.from_numpy(f32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = f64_to_bf16_bits(f32.astype(np.float64))
    assert np.array_equal(got, ref), "bf16 rounding disagrees with torch on float32 inputs"
    # (2) hand cases straight from the definition (ties to even, one rounding).
    cases = {
        1 + 2 ** -8: 1.0,                        # tie -> even (1.0)
        1 + 3 * 2 ** -8: 1 + 2 ** -6,             # tie -> even (fraction 0000010)
        1 + 2 ** -8 + 2 ** -40: 1 + 2 ** -7,      # above the tie; float32 first would tie to 1.0
        -(1 + 2 ** -8 + 2 ** -40): -(1 + 2 ** -7),
        2 ** -134: 0.0,                           # subnormal tie -> 0
        3 * 2 ** -134: 2 ** -132,                 # subnormal tie -> even
        3.39e38: 3.3895313892515355e38,           # largest finite bfloat16
    }
    for x, want in cases.items():
        assert round_f64_to_bf16(np.array([x]))[0] == want, (x, want)
    assert np.isinf(round_f64_to_bf16(np.array([3.4e38]))[0])
    # (3) random float64 inputs against exact rational rounding.
    xs = rng.standard_normal(3000) * np.exp2(rng.integers(-60, 60, 3000))
    got = round_f64_to_bf16(xs)
    for x, y in zip(xs, got):
        assert Fraction(float(y)) == fraction_to_bf16(Fraction(float(x))), x


# ----------------------------------------------------------------------------------------
# pooling
# ----------------------------------------------------------------------------------------

def _fraction_summary(block_rows: np.ndarray, s: int, to_storage) -> list:
    g, d = block_rows.shape
    out = []
    for c in range(d):
        means = [sum(Fraction(float(v)) for v in block_rows[u * s:(u + 1) * s, c]) / s
                 for u in range(g // s)]
        out.append(to_storage(max(means)))
    return out


def check_pooling(block_summaries):
    # Hand example (tests/golden/pooling_hand_example.json).
    gold = load_golden("pooling_hand_example.json")
    for case in gold["cases"]:
        K = np.array(gold["rows"], dtype=np.float64)
        S = block_summaries(K, case["block"], case["sub_block"], "f32")
        assert S.shape == (1, K.shape[1])
        assert np.array_equal(S[0], np.array(case["expected"], dtype=np.float64)), case

    rng = np.random.default_rng(12)
    # g = s = 1: every summary is its key row.
    K = random_bf16_values(rng, (37, 16))
    assert np.array_equal(block_summaries(K, 1, 1, "bf16"), K)
    # constant blocks: the summary is the constant.
    K = np.repeat(random_bf16_values(rng, (6, 1, 8)), 16, axis=1).reshape(96, 8)
    S = block_summaries(K, 16, 4, "bf16")
    assert np.array_equal(S, K[::16])
    # only full blocks get summaries.
    K = random_bf16_values(rng, (5 * 32 + 7, 8))
    assert block_summaries(K, 32, 16, "bf16").shape == (5, 8)
    # exact rational reference, bf16 and f32, several (g, s).
    for dtype, to_storage in (("bf16", fraction_to_bf16), ("f32", fraction_to_f32)):
        for g, s in ((16, 16), (32, 16), (64, 16), (16, 1), (8, 4)):
            if dtype == "bf16":
                K = random_bf16_values(rng, (3 * g, 6), scale=3.0)
            else:
                K = rng.standard_normal((3 * g, 6)).astype(np.float32).astype(np.float64)
            S = block_summaries(K, g, s, dtype)
            for j in range(3):
                want = _fraction_summary(K[j * g:(j + 1) * g], s, to_storage)
                assert [Fraction(float(v)) for v in S[j]] == want, (dtype, g, s, j)
    # invariances: permute rows inside each sub-block, and permute sub-blocks.
    K = random_bf16_values(rng, (64, 8))
    S = block_summaries(K, 64, 16, "bf16")
    sub = K.reshape(4, 16, 8)
    perm_rows = np.stack([sub[u][rng.permutation(16)] for u in range(4)]).reshape(64, 8)
    perm_sub = sub[rng.permutation(4)].reshape(64, 8)
    assert np.array_equal(block_summaries(perm_rows, 64, 16, "bf16"), S)
    assert np.array_equal(block_summaries(perm_sub, 64, 16, "bf16"), S)


# ----------------------------------------------------------------------------------------
# scoring
# ----------------------------------------------------------------------------------------

def check_scoring(block_scores):
    rng = np.random.default_rng(13)
    # exact rational reference: sum over the group and the columns, rounded once to float32.
    for G, d, n in ((1, 8, 40), (4, 16, 60), (7, 32, 50), (8, 128, 30)):
        q = random_bf16_values(rng, (G, d))
        S = random_bf16_values(rng, (n, d), scale=2.0)
        got = block_scores(q, S)
        assert got.dtype == np.float32 and got.shape == (n,)
        for j in range(n):
            exact = sum(Fraction(float(q[g, c])) * Fraction(float(S[j, c]))
                        for g in range(G) for c in range(d))
            assert Fraction(float(got[j])) == fraction_to_f32(exact), (G, d, j)
    # closed form: one-hot query rows and summaries.
    G, d = 4, 8
    q = np.zeros((G, d))
    q[:, 3] = 1.0
    S = np.zeros((5, d))
    S[:, 3] = [1.0, -2.0, 0.5, 4.0, 0.0]
    S[:, 5] = 7.0                         # a column the query does not see
    assert np.array_equal(block_scores(q, S), np.float32([4.0, -8.0, 2.0, 16.0, 0.0]))
    # distinct rows matter: q_0 = e_1 and q_1 = 2 e_2 against S = (0, 3, 5, 0).
    q = np.array([[0, 1, 0, 0], [0, 0, 2, 0]], dtype=np.float64)
    S = np.array([[0, 3, 5, 0]], dtype=np.float64)
    assert block_scores(q, S)[0] == np.float32(13.0)


def check_sub_block_means(sub_block_means, block_summaries):
    """Score-side pooling, first stage: every sub-block mean rounded once."""
    rng = np.random.default_rng(23)
    for dtype, to_storage in (("bf16", fraction_to_bf16), ("f32", fraction_to_f32)):
        for g, s in ((16, 16), (32, 8), (64, 16), (16, 1), (8, 4)):
            if dtype == "bf16":
                K = random_bf16_values(rng, (3 * g + 5, 6), scale=3.0)
            else:
                K = rng.standard_normal((3 * g + 5, 6)).astype(np.float32).astype(np.float64)
            M = sub_block_means(K, g, s, dtype)
            assert M.shape == (3, g // s, 6)
            for j in range(3):
                for u in range(g // s):
                    for c in range(6):
                        exact = sum(Fraction(float(v)) for v in
                                    K[j * g + u * s:j * g + (u + 1) * s, c]) / s
                        assert Fraction(float(M[j, u, c])) == to_storage(exact), (dtype, g, s)
            # rounding is monotone, so the max of the rounded means is the key-side summary.
            assert np.array_equal(M.max(axis=1), block_summaries(K, g, s, dtype))
    # the double-rounding trap, with bf16 rows (2, 2, 2^-6, 2^-27): the mean is
    # 1 + 2^-8 + 2^-29, just above the tie between the bf16 neighbours 1 and 1 + 2^-7, and
    # float32 would first round it onto that tie (then to the even neighbour, 1).
    rows = np.array([[2.0], [2.0], [2.0 ** -6], [2.0 ** -27]])
    M = sub_block_means(rows, 4, 4, "bf16")
    exact = sum(Fraction(float(v)) for v in rows[:, 0]) / 4
    assert Fraction(float(M[0, 0, 0])) == fraction_to_bf16(exact) == 1 + Fraction(1, 2 ** 7)


def check_sub_block_scores(sub_block_scores, block_scores, POOL_SCORE_SUM, POOL_SCORE_MAX):
    """Score-side pooling: block max over the sub-block means' scores; the group summed or
    maxed."""
    rng = np.random.default_rng(24)
    # exact rational reference for both group aggregations.
    for G, d, n, r in ((1, 8, 20, 4), (4, 16, 15, 2), (7, 32, 10, 4), (8, 128, 6, 16)):
        q = random_bf16_values(rng, (G, d))
        M = random_bf16_values(rng, (n, r, d), scale=2.0)
        got_s = sub_block_scores(q, M, POOL_SCORE_SUM)
        got_m = sub_block_scores(q, M, POOL_SCORE_MAX)
        assert got_s.dtype == np.float32 and got_s.shape == (n,) and got_m.shape == (n,)
        for j in range(n):
            dots = [[sum(Fraction(float(q[g, c])) * Fraction(float(M[j, u, c])) for c in range(d))
                     for u in range(r)] for g in range(G)]
            want_s = max(sum(dots[g][u] for g in range(G)) for u in range(r))
            want_m = max(max(row) for row in dots)
            assert Fraction(float(got_s[j])) == fraction_to_f32(want_s), (G, d, r, j)
            assert Fraction(float(got_m[j])) == fraction_to_f32(want_m), (G, d, r, j)
    # one sub-block per block: the group-sum variant is key-side scoring bit for bit.
    q = random_bf16_values(rng, (4, 64))
    S = random_bf16_values(rng, (30, 64))
    assert np.array_equal(sub_block_scores(q, S[:, None, :], POOL_SCORE_SUM), block_scores(q, S))
    # G = 1: the two group aggregations agree.
    M = random_bf16_values(rng, (12, 4, 32))
    q1 = random_bf16_values(rng, (1, 32))
    assert np.array_equal(sub_block_scores(q1, M, POOL_SCORE_SUM), sub_block_scores(q1, M, POOL_SCORE_MAX))
    # hand example where the two pooling sides differ: q = (1, 1), sub-block means
    # (1, 0) and (0, 1).  Key side: summary (1, 1), score 2.  Score side: max(1, 1) = 1.
    qh = np.array([[1.0, 1.0]])
    Mh = np.array([[[1.0, 0.0], [0.0, 1.0]]])
    assert sub_block_scores(qh, Mh, POOL_SCORE_SUM)[0] == np.float32(1.0)
    assert block_scores(qh, Mh.max(axis=1))[0] == np.float32(2.0)
    # group of two rows e_0 and 3 e_1 against means (2, 0) and (0, 1):
    # sum agg: max(2, 3) = 3; max agg: max(max(2, 0), max(0, 3)) = 3; with means (2, 0)
    # and (0, 0.5): sum agg max(2, 1.5) = 2, max agg max(2, 1.5) = 2; and with a third
    # row -e_0 the sum agg drops to max(0, 1.5) = 1.5 while the max agg stays 2.
    qg = np.array([[1.0, 0.0], [0.0, 3.0]])
    assert sub_block_scores(qg, np.array([[[2.0, 0.0], [0.0, 1.0]]]), POOL_SCORE_SUM)[0] == 3.0
    assert sub_block_scores(qg, np.array([[[2.0, 0.0], [0.0, 1.0]]]), POOL_SCORE_MAX)[0] == 3.0
    q3 = np.array([[1.0, 0.0], [0.0, 3.0], [-1.0, 0.0]])
    M3 = np.array([[[2.0, 0.0], [0.0, 0.5]]])
    assert sub_block_scores(q3, M3, POOL_SCORE_SUM)[0] == np.float32(1.5)
    assert sub_block_scores(q3, M3, POOL_SCORE_MAX)[0] == np.float32(2.0)
    # invariances: permuting the sub-blocks of a block, or the rows of the group.
    q = random_bf16_values(rng, (4, 16))
    M = random_bf16_values(rng, (10, 8, 16))
    for pool in (POOL_SCORE_SUM, POOL_SCORE_MAX):
        base = sub_block_scores(q, M, pool)
        assert np.array_equal(sub_block_scores(q, M[:, rng.permutation(8)], pool), base)
        assert np.array_equal(sub_block_scores(q[rng.permutation(4)], M, pool), base)
    # with a non-negative query the key-side score bounds the group-sum score from above.
    qp = np.abs(random_bf16_values(rng, (4, 16)))
    Mp = random_bf16_values(rng, (40, 4, 16))
    assert np.all(block_scores(qp, Mp.max(axis=1)) >= sub_block_scores(qp, Mp, POOL_SCORE_SUM))
    # empty block list.
    assert sub_block_scores(q, np.zeros((0, 8, 16)), POOL_SCORE_MAX).shape == (0,)


# ----------------------------------------------------------------------------------------
# selection
# ----------------------------------------------------------------------------------------

class Pol:
    def __init__(self, **kw):
        self.mode = 0
        self.block = 1
        self.sub_block = 1
        self.top_k = 0
        self.budget = 0.0
        self.k_evict = 0
        self.sink_tokens = 0
        self.local_tokens = 0
        self.force_sink = 0
        self.force_last = 0
        self.__dict__.update(kw)


def _forced_brute(pol, T):
    g = pol.block
    n_tot = -(-T // g)
    F = set()
    for j in range(n_tot):
        toks = set(range(j * g, min((j + 1) * g, T)))
        if pol.mode == 1:
            window = set(range(0, min(pol.sink_tokens, T))) | set(range(max(0, T - pol.local_tokens), T))
            if toks & window:
                F.add(j)
        else:
            if pol.force_sink and j == 0:
                F.add(j)
            if pol.force_last and j == n_tot - 1:
                F.add(j)
        if len(toks) < g:
            F.add(j)
    return sorted(F)


def check_forced(forced_blocks):
    gold = load_golden("selection_stated_sizes.json")
    st = gold["llama8b_streaming"]
    pol = Pol(mode=1, block=st["block"], sink_tokens=st["sink_tokens"], local_tokens=st["local_tokens"])
    assert list(forced_blocks(pol, st["context"])) == st["expected_forced"]
    rng = np.random.default_rng(14)
    for _ in range(300):
        g = int(rng.choice([1, 2, 4, 8, 16, 32]))
        T = int(rng.integers(1, 300))
        mode = int(rng.integers(0, 3))
        pol = Pol(mode=mode, block=g, sink_tokens=int(rng.integers(0, 70)),
                  local_tokens=int(rng.integers(0, 120)), force_sink=int(rng.integers(0, 2)),
                  force_last=int(rng.integers(0, 2)))
        assert list(forced_blocks(pol, T)) == _forced_brute(pol, T), (mode, g, T)


def check_budget(budget_k):
    gold = load_golden("selection_stated_sizes.json")
    b = gold["llama8b_retrieval"]
    pol = Pol(mode=0, block=b["block"], budget=float(np.float32(b["budget"])))
    assert budget_k(pol, b["context"] // b["block"]) == b["expected_k"]
    assert budget_k(Pol(mode=0, top_k=8), 64) == 8
    assert budget_k(Pol(mode=0, budget=0.25), 512) == 128          # exact product: no round-up
    assert budget_k(Pol(mode=0, budget=0.25), 500) == 125          # odd exact product
    assert budget_k(Pol(mode=0, budget=float(np.float32(0.3))), 10) == 4
    assert budget_k(Pol(mode=0, budget=float(np.float32(0.1))), 8192) == 820


def _precedes(a, b, v):
    return (v[a] > v[b]) or (v[a] == v[b] and a < b)


def check_top_k(top_k):
    rng = np.random.default_rng(15)
    for trial in range(200):
        n = int(rng.integers(1, 11))
        v = rng.integers(-3, 4, size=n).astype(np.float32)     # many ties on purpose
        if trial % 3 == 0:
            v = rng.standard_normal(n).astype(np.float32)
        cand = np.sort(rng.choice(n, size=int(rng.integers(0, n + 1)), replace=False))
        k = int(rng.integers(0, n + 2))
        got = top_k(v, cand, k)
        kk = min(k, cand.size)
        winners = [c for c in itertools.combinations(cand.tolist(), kk)
                   if all(_precedes(a, b, v) for a in c for b in cand.tolist() if b not in c)]
        assert len(winners) == 1
        assert list(got) == sorted(winners[0]), (v, cand, k, got, winners)
    # duplicated values: the lower index wins; -0.0 equals +0.0.
    v = np.float32([1.0, 5.0, 5.0, 5.0, 2.0])
    assert list(top_k(v, np.arange(5), 2)) == [1, 2]
    v = np.float32([-0.0, 0.0, -1.0])
    assert list(top_k(v, np.arange(3), 1)) == [0]
    assert list(top_k(np.float32([0.0, -0.0]), np.arange(2), 1)) == [0]


def check_select_retrieval(select_unit):
    gold = load_golden("selection_stated_sizes.json")
    t = gold["tiny"]
    pol = Pol(mode=0, block=t["block"], top_k=t["top_k"], force_sink=1, force_last=1)
    rng = np.random.default_rng(16)
    scores = rng.standard_normal(t["context"] // t["block"]).astype(np.float32)
    sel, _ = select_unit(pol, t["context"], scores)
    assert len(sel) == t["expected_selected"]
    assert sel[0] == 0 and sel[-1] == t["context"] // t["block"] - 1
    inner = [j for j in sel if j not in (0, t["context"] // t["block"] - 1)]
    order = sorted(range(1, 63), key=lambda j: (-float(scores[j]), j))
    assert sorted(order[:t["top_k"]]) == inner
    # a partial last block is always kept and never scored.
    pol = Pol(mode=0, block=16, top_k=2)
    scores = np.float32([0, 9, 1, 8, 2])
    sel, _ = select_unit(pol, 5 * 16 + 3, scores)
    assert list(sel) == [1, 3, 5]
    # budget covering everything keeps every block.
    sel, _ = select_unit(Pol(mode=0, block=16, top_k=100), 200, np.zeros(12, np.float32))
    assert list(sel) == list(range(13))


def check_select_nosa(select_unit):
    rng = np.random.default_rng(17)
    # growing context with eviction logits that change every step: strict eviction keeps
    # every dropped block out of Gamma_e for good, and Gamma_e only takes kept or new blocks.
    # (With logits that never change, a plain top-k over all blocks would already be
    # monotone, so the logits are redrawn to make the eviction state matter.)
    g, k_e, k_q = 4, 5, 3
    pol = Pol(mode=2, block=g, top_k=k_q, k_evict=k_e)
    n_max = 60
    ev = np.zeros(n_max, dtype=bool)
    prev_e = None
    ever_evicted = set()
    for step, T in enumerate(range(8 * g, n_max * g + 1, g)):
        n_full = T // g
        scores = rng.standard_normal(n_max).astype(np.float32)
        logits = rng.standard_normal(n_max).astype(np.float32)
        sel, ev_new = select_unit(pol, T, scores, logits, ev)
        assert np.all(ev_new[ev]), "an evicted block came back"
        full = np.arange(n_full)
        E = full[~ev[:n_full]]
        gamma_e = [j for j in sel if j in E and not ev_new[j]]
        # Gamma_e is exactly the top-k_e of the non-evicted blocks by logit.
        want_e = sorted(sorted(E, key=lambda j: (-float(logits[j]), j))[:k_e])
        assert gamma_e == want_e
        assert not (set(gamma_e) & ever_evicted)
        if prev_e is not None:
            assert set(gamma_e) <= set(prev_e) | {n_full - 1}
        assert len(sel) == min(n_full, k_e + k_q)
        newly = set(np.flatnonzero(ev_new[:n_full] & ~ev[:n_full]).tolist())
        assert newly == set(E.tolist()) - set(gamma_e)
        ever_evicted |= newly
        prev_e, ev = gamma_e, ev_new
    # fixed context: Gamma_e constant, evicted blocks still eligible for Gamma_q,
    # locality >= k_e / k every step.
    g, k_e, k_q, n = 8, 6, 2, 40
    pol = Pol(mode=2, block=g, top_k=k_q, k_evict=k_e)
    logits = rng.standard_normal(n).astype(np.float32)
    ev = np.zeros(n, dtype=bool)
    prev = None
    saw_evicted_in_q = False
    for step in range(30):
        scores = rng.standard_normal(n).astype(np.float32)
        sel, ev = select_unit(pol, n * g, scores, logits, ev)
        kept = [j for j in sel if not ev[j]]
        assert kept == sorted(sorted(range(n), key=lambda j: (-float(logits[j]), j))[:k_e])
        q_part = [j for j in sel if ev[j]]
        want_q = sorted(sorted([j for j in range(n) if j not in kept],
                               key=lambda j: (-float(scores[j]), j))[:k_q])
        assert q_part == want_q
        saw_evicted_in_q |= len(q_part) > 0
        if prev is not None:
            assert len(set(sel) & set(prev)) / len(sel) >= k_e / (k_e + k_q)
        prev = sel
    assert saw_evicted_in_q


# ----------------------------------------------------------------------------------------
# attention
# ----------------------------------------------------------------------------------------

def _dense_masked(q, K, V, keep_tokens, scale):
    """Reference: torch scaled_dot_product_attention in float64 over ALL tokens with a mask."""
    T = K.shape[0]
    mask = torch.zeros((q.shape[0], T), dtype=torch.bool)
    mask[:, torch.from_numpy(np.asarray(keep_tokens, dtype=np.int64))] = True
    out = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None], torch.from_numpy(K)[None], torch.from_numpy(V)[None],
        attn_mask=mask[None], scale=scale)
    return out[0].numpy()


def check_attention(attend, selected_tokens, merge_partials, partial):
    rng = np.random.default_rng(18)
    G, d, T, g = 4, 32, 203, 16
    q = rng.standard_normal((G, d))
    K = rng.standard_normal((T, d))
    V = rng.standard_normal((T, d))
    scale = 1 / math.sqrt(d)
    sel = np.array([0, 3, 4, 9, 12])               # 12 is the partial last block
    tok = selected_tokens(sel, g, T)
    assert list(tok) == [t for j in sel for t in range(j * g, min((j + 1) * g, T))]
    out, lse = attend(q, K[tok], V[tok], scale)
    assert np.allclose(out, _dense_masked(q, K, V, tok, scale), rtol=1e-12, atol=1e-12)
    s = (q @ K[tok].T) * scale
    assert np.allclose(lse, np.log(np.exp(s).sum(axis=1)), rtol=1e-12)
    # budget covering every block (and g = 1 with k = n) is dense attention.
    full = selected_tokens(np.arange(-(-T // g)), g, T)
    assert np.array_equal(full, np.arange(T))
    assert np.allclose(attend(q, K[full], V[full], scale)[0],
                       _dense_masked(q, K, V, np.arange(T), scale), rtol=1e-12, atol=1e-12)
    assert np.array_equal(selected_tokens(np.arange(T), 1, T), np.arange(T))
    # one selected token: out = v_t exactly, lse = its logit.
    out1, lse1 = attend(q, K[[7]], V[[7]], scale)
    assert np.array_equal(out1, np.repeat(V[[7]], G, axis=0))
    assert np.allclose(lse1, (q @ K[7]) * scale, rtol=1e-14)
    # identical keys: the mean of the selected values.
    Kc = np.repeat(K[[0]], 10, axis=0)
    outc, _ = attend(q, Kc, V[:10], scale)
    assert np.allclose(outc, np.repeat(V[:10].mean(axis=0)[None], G, axis=0), rtol=1e-12)
    # empty token set.
    oute, lsee = attend(q, K[:0], V[:0], scale)
    assert np.all(oute == 0) and np.all(np.isneginf(lsee))
    # split-K: merging partials over any split equals the whole.
    for cuts in ([50], [1, 2, 90], [0, 150, 150]):
        edges = [0] + cuts + [len(tok)]
        parts = [partial(q, K[tok[a:b]], V[tok[a:b]], scale) for a, b in zip(edges[:-1], edges[1:])]
        o2, l2 = merge_partials(parts)
        assert np.allclose(o2, out, rtol=1e-12, atol=1e-12) and np.allclose(l2, lse, rtol=1e-12)


def _dense_additive(q, K, V, keep_tokens, bias_tokens, scale):
    """Reference: torch scaled_dot_product_attention in float64 with a FLOAT mask, which the
    library adds to the scaled logits: the bias on the kept tokens, -inf elsewhere."""
    T = K.shape[0]
    mask = torch.full((q.shape[0], T), -math.inf, dtype=torch.float64)
    mask[:, torch.from_numpy(np.asarray(keep_tokens, dtype=np.int64))] = torch.from_numpy(
        np.asarray(bias_tokens, dtype=np.float64))[None, :]
    out = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None], torch.from_numpy(K)[None], torch.from_numpy(V)[None],
        attn_mask=mask[None], scale=scale)
    return out[0].numpy()


def check_biased_attention(attend, token_bias, selected_tokens, merge_partials, partial):
    """[NOSA-DE] Methodik §1, "ED-DMA", read as an additive pre-softmax term per block."""
    # token_bias by hand: g = 4, T = 10, blocks 0 and 2 (block 2 holds tokens 8, 9 only).
    assert list(token_bias(np.array([0, 2]), 4, 10, np.array([0.5, -1.0, 2.0]))) == \
        [0.5] * 4 + [2.0] * 2
    assert len(token_bias(np.zeros(0, np.int64), 4, 10, np.zeros(3))) == 0
    # Two tokens with equal keys, values 0 and 1, bias (0, b): out = sigmoid(b),
    # lse = ln(1 + e^b) (the key logits are 0).
    for b in (0.7, -2.0, 5.5):
        out, lse = attend(np.array([[1.0]]), np.zeros((2, 1)), np.array([[0.0], [1.0]]), 1.0,
                          np.array([0.0, b]))
        assert abs(out[0, 0] - 1.0 / (1.0 + math.exp(-b))) < 1e-15
        assert abs(lse[0] - math.log1p(math.exp(b))) < 1e-14

    rng = np.random.default_rng(21)
    G, d, T, g = 4, 32, 203, 16
    q = rng.standard_normal((G, d))
    K = rng.standard_normal((T, d))
    V = rng.standard_normal((T, d))
    scale = 1 / math.sqrt(d)
    sel = np.array([0, 3, 4, 9, 12])               # 12 is the partial last block
    logits = rng.standard_normal(-(-T // g))
    tok = selected_tokens(sel, g, T)
    bias = token_bias(sel, g, T, logits)
    out, lse = attend(q, K[tok], V[tok], scale, bias)
    # The library's additive float mask.
    assert np.allclose(out, _dense_additive(q, K, V, tok, bias, scale), rtol=1e-12, atol=1e-12)
    s = (q @ K[tok].T) * scale + bias[None, :]
    assert np.allclose(lse, np.log(np.exp(s).sum(axis=1)), rtol=1e-12)
    # A bias of ln 2 (ln 3) on one block weighs like that block's tokens present twice
    # (three times) without a bias.
    for reps in (2, 3):
        bl = np.zeros_like(logits)
        bl[4] = math.log(reps)
        bo, bls = attend(q, K[tok], V[tok], scale, token_bias(sel, g, T, bl))
        dup = np.concatenate([tok] + [np.arange(4 * g, 5 * g)] * (reps - 1))
        do, dls = attend(q, K[dup], V[dup], scale)
        assert np.allclose(bo, do, rtol=1e-12, atol=1e-12) and np.allclose(bls, dls, rtol=1e-12)
    # A constant bias leaves out unchanged and shifts lse by that constant; zero is no bias.
    oc, lc = attend(q, K[tok], V[tok], scale, np.full(len(tok), 1.75))
    o0, l0 = attend(q, K[tok], V[tok], scale)
    assert np.allclose(oc, o0, rtol=1e-12, atol=1e-12) and np.allclose(lc, l0 + 1.75, rtol=1e-12)
    oz, lz = attend(q, K[tok], V[tok], scale, np.zeros(len(tok)))
    assert np.array_equal(oz, o0) and np.array_equal(lz, l0)
    # A very negative bias on a block removes it.
    bl = logits.copy()
    bl[3] = -1e4
    on, ln_ = attend(q, K[tok], V[tok], scale, token_bias(sel, g, T, bl))
    keep = sel[sel != 3]
    tk = selected_tokens(keep, g, T)
    ok, lk = attend(q, K[tk], V[tk], scale, token_bias(keep, g, T, bl))
    assert np.allclose(on, ok, rtol=1e-12, atol=1e-12) and np.allclose(ln_, lk, rtol=1e-12)
    # split-K with the bias: merging partials over any split equals the whole.
    for cuts in ([50], [1, 2, 90], [0, 150, 150]):
        edges = [0] + cuts + [len(tok)]
        parts = [partial(q, K[tok[a:b]], V[tok[a:b]], scale, bias[a:b])
                 for a, b in zip(edges[:-1], edges[1:])]
        o2, l2 = merge_partials(parts)
        assert np.allclose(o2, out, rtol=1e-12, atol=1e-12) and np.allclose(l2, lse, rtol=1e-12)


# ----------------------------------------------------------------------------------------
# compaction
# ----------------------------------------------------------------------------------------

def check_compaction(compact_update, apply_moves, selection_delta):
    """Block-slot working set of the selected full blocks, moved by set difference."""
    # Hand example, g = 4, five slots.
    m, mv = compact_update(np.full(5, -1), np.array([0, 2, 5, 7]), 30, 4)   # block 7 partial
    assert list(m) == [0, 2, 5, -1, -1] and mv == [(0, 0), (1, 2), (2, 5)]
    m, mv = compact_update(m, np.array([0, 3, 5, 7]), 31, 4)                # 2 out, 3 in
    assert list(m) == [0, 3, 5, -1, -1] and mv == [(1, 3)]
    m, mv = compact_update(m, np.array([0, 5, 7]), 32, 4)                   # 7 became full
    assert list(m) == [0, 7, 5, -1, -1] and mv == [(1, 7)]
    m2, mv = compact_update(m, np.array([0, 5, 7]), 33, 4)                  # nothing new
    assert list(m2) == list(m) and mv == []
    m3, mv = compact_update(m, np.zeros(0, np.int64), 33, 4)
    assert list(m3) == [-1] * 5 and mv == []
    try:
        compact_update(np.full(2, -1), np.array([0, 1, 2]), 40, 4)
        raise AssertionError("capacity not enforced")
    except ValueError:
        pass

    # Random growing sequences against independent characterisations.
    rng = np.random.default_rng(26)
    for trial in range(60):
        g = int(rng.choice([1, 4, 16]))
        n_slots = int(rng.integers(3, 12))
        T = int(rng.integers(0, 6 * g))
        d = 3
        K = rng.standard_normal((T + 80 * g, d))
        V = rng.standard_normal((T + 80 * g, d))
        slots = np.full(n_slots, -1)
        wK = np.full((n_slots * g, d), np.nan)
        wV = np.full((n_slots * g, d), np.nan)
        prev_full = np.zeros(0, np.int64)
        for step in range(12):
            T += int(rng.integers(0, 2 * g))
            n_tot, n_full = -(-T // g), T // g
            k = int(rng.integers(0, min(n_slots, n_full) + 1))
            sel = np.sort(rng.choice(n_full, size=k, replace=False)) if k else np.zeros(0, np.int64)
            if n_tot > n_full and rng.random() < 0.7:
                sel = np.append(sel, n_tot - 1)                   # the partial last block
            before = slots.copy()
            slots, mv = compact_update(slots, sel, T, g)
            target = sel[sel < n_full]
            held_before = before[before >= 0]
            assert sorted(slots[slots >= 0].tolist()) == sorted(target.tolist())
            for s_, b in enumerate(before):                      # kept blocks stay put
                if b >= 0 and b in target:
                    assert slots[s_] == b
            added = np.setdiff1d(target, held_before)
            assert [b for _, b in mv] == list(added)             # ascending, only the new ones
            free_after_removal = [s_ for s_ in range(n_slots)
                                  if before[s_] < 0 or before[s_] not in target]
            assert [s_ for s_, _ in mv] == free_after_removal[:len(added)]
            apply_moves(wK, wV, K, V, mv, g)
            for s_, b in enumerate(slots):                       # contents: brute force
                if b >= 0:
                    assert np.array_equal(wK[s_ * g:(s_ + 1) * g], K[b * g:(b + 1) * g])
                    assert np.array_equal(wV[s_ * g:(s_ + 1) * g], V[b * g:(b + 1) * g])
            # with only full blocks on both sides, the moves are the selection delta's adds.
            assert list(added) == list(selection_delta(prev_full, target)[0]) or \
                len(np.setdiff1d(held_before, prev_full)) > 0
            prev_full = target


# ----------------------------------------------------------------------------------------
# delta
# ----------------------------------------------------------------------------------------

def check_delta(selection_delta, locality):
    rng = np.random.default_rng(19)
    for _ in range(200):
        prev = np.sort(rng.choice(50, size=int(rng.integers(0, 20)), replace=False))
        cur = np.sort(rng.choice(50, size=int(rng.integers(0, 20)), replace=False))
        added, removed = selection_delta(prev, cur)
        assert list(added) == sorted(set(cur.tolist()) - set(prev.tolist()))
        assert list(removed) == sorted(set(prev.tolist()) - set(cur.tolist()))
        assert cur.size == prev.size - removed.size + added.size
        if cur.size:
            assert locality(prev, cur) == len(set(cur.tolist()) & set(prev.tolist())) / cur.size
    added, removed = selection_delta(np.zeros(0, np.int64), np.array([2, 5]))
    assert list(added) == [2, 5] and removed.size == 0
