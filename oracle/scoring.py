"""Block scores against the GQA query group (oracle; test infrastructure only).

[NOSA-DE] Methodik §1, "Query-Aware Selection (Γq)": the current query decides
which (possibly distant) blocks are fetched.  [Fluxion-NL] Systeemcomponenten,
"Granularity-Budget Selector": GQA is handled at the level of the query group,
so one selection per kv head serves all G query heads that share it.
[NOSA-DE] Methodik §1, "ED-DMA": selection is made on pre-exponential scores.

Readings:
* Group aggregation is the SUM of the raw dot products of the G query rows with
  the block summary.  No 1/sqrt(d) factor and no softmax: a positive scale does
  not change the ranking, and selection is made before any exponential.
* The score is a float32 number.  Its value is defined as the float64
  evaluation below, rounded once to float32 (ties to even):
      qs     = ((q_0 + q_1) + q_2) + ... + q_{G-1}          (float64, row order)
      acc    = (((0 + qs[0]*S[0]) + qs[1]*S[1]) + ... )      (float64, column order,
                                                              product and sum each
                                                              rounded, no fused
                                                              multiply-add)
      score  = float32(acc)
  Summing the rows first is the same quantity as sum_g (q_g . S) in exact
  arithmetic (linearity); the fixed float64 order makes the float32 result a
  single well-defined number.
* Score-side pooling ([NOSA-DE] Methodik §1, "Blockweise Implementierung", its
  other reading): the block's score is the max over its sub-block means of their
  scores; the group is aggregated by the sum above or, as an alternative, by a max
  over the G rows (sub_block_scores).
"""
from __future__ import annotations

import numpy as np


def group_query_sum(q_rows: np.ndarray) -> np.ndarray:
    """Sum of the G query rows [G][d] in float64, in row order."""
    q_rows = np.asarray(q_rows, dtype=np.float64)
    acc = q_rows[0].copy()
    for g in range(1, q_rows.shape[0]):
        acc = acc + q_rows[g]
    return acc


def _chain(vec: np.ndarray, rows: np.ndarray) -> np.ndarray:
    """float64 dot products of vec [d] with rows [..., d], columns in order, each product
    and sum rounded on its own."""
    rows = np.asarray(rows, dtype=np.float64)
    acc = np.zeros(rows.shape[:-1], dtype=np.float64)
    for c in range(rows.shape[-1]):
        prod = vec[c] * rows[..., c]
        acc = acc + prod
    return acc


def block_scores(q_rows: np.ndarray, S: np.ndarray) -> np.ndarray:
    """float32 scores [n] of the summaries S [n][d] against the query group q_rows [G][d]."""
    return _chain(group_query_sum(q_rows), S).astype(np.float32)


POOL_KEY, POOL_SCORE_SUM, POOL_SCORE_MAX = 0, 1, 2


def sub_block_scores(q_rows: np.ndarray, M: np.ndarray, pooling: int) -> np.ndarray:
    """float32 scores [n] from the sub-block means M [n][r][d] (score-side pooling).

    POOL_SCORE_SUM: score_j = float32( max over u of chain(qs, M[j, u]) ), the group's
                    summed dot product of every sub-block mean, then the block max.
    POOL_SCORE_MAX: score_j = float32( max over u and g of chain(q_g, M[j, u]) ), the
                    group aggregated by a max instead of a sum.
    chain is block_scores' float64 evaluation; rounding once after the max equals the
    max of the rounded values (rounding is monotone)."""
    q_rows = np.asarray(q_rows, dtype=np.float64)
    M = np.asarray(M, dtype=np.float64)
    if pooling == POOL_SCORE_SUM:
        v = _chain(group_query_sum(q_rows), M)                           # [n][r]
        return v.max(axis=1).astype(np.float32)
    if pooling == POOL_SCORE_MAX:
        v = np.stack([_chain(q_rows[g], M) for g in range(q_rows.shape[0])])   # [G][n][r]
        return v.max(axis=(0, 2)).astype(np.float32)
    raise ValueError(f"not a score-side pooling: {pooling}")
