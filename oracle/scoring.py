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


def block_scores(q_rows: np.ndarray, S: np.ndarray) -> np.ndarray:
    """float32 scores [n] of the summaries S [n][d] against the query group q_rows [G][d]."""
    qs = group_query_sum(q_rows)
    S = np.asarray(S, dtype=np.float64)
    acc = np.zeros(S.shape[0], dtype=np.float64)
    for c in range(S.shape[1]):
        prod = qs[c] * S[:, c]
        acc = acc + prod
    return acc.astype(np.float32)
