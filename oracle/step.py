"""One decode step of one unit, end to end (oracle; test infrastructure only).

Chains the oracle's pieces in the order the hot path runs them:
summaries -> scores -> selection -> attention over the selected tokens.
A unit is one (sequence, kv head); its G query rows share the selection
([Fluxion-NL] Systeemcomponenten, "Granularity-Budget Selector": selection is
made per GQA group).  ``pol`` is any object with the fields of a head policy
(mode, block, sub_block, top_k, budget, k_evict, sink_tokens, local_tokens,
force_sink, force_last).
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np

from .attention import attend, selected_tokens, token_bias
from .numerics import round_to_storage
from .pooling import block_summaries, sub_block_means
from .scoring import POOL_KEY, block_scores, sub_block_scores
from .selection import MODE_NOSA, MODE_STREAMING, select_unit


@dataclass
class UnitResult:
    summaries: np.ndarray           # float64 [n_full][d] ([n_full][r][d] under score-side
                                    # pooling), representable in the storage dtype
    scores: Optional[np.ndarray]    # float32 [n_full] (None for streaming units)
    sel: np.ndarray                 # int64 ascending block indices
    evicted: Optional[np.ndarray]   # bool eviction state after the step (NOSA units)
    out: np.ndarray                 # float64 [G][d], rounded to the storage dtype
    out_exact: np.ndarray           # float64 [G][d] before rounding
    lse: np.ndarray                 # float64 [G]


def unit_step(pol, T: int, dtype: str, q_rows: np.ndarray, K: np.ndarray, V: np.ndarray,
              scale: float, logits: Optional[np.ndarray] = None,
              evicted: Optional[np.ndarray] = None,
              summaries: Optional[np.ndarray] = None, ed: bool = False,
              pooling: int = POOL_KEY) -> UnitResult:
    """q_rows float64 [G][d]; K, V float64 [T][d] (the unit's valid rows).

    ``ed``: a NOSA unit adds each selected block's eviction logit (``logits``, one per
    block slot of the unit) to its tokens' attention logits ([NOSA-DE] Methodik §1,
    "ED-DMA"); other modes have no eviction head and are unaffected.
    ``pooling``: POOL_KEY pools the keys into one vector per block (summaries [n_full][d]);
    POOL_SCORE_SUM / POOL_SCORE_MAX keep the sub-block means (summaries
    [n_full][block/sub_block][d]) and take the block max over their scores."""
    if pooling == POOL_KEY:
        S = block_summaries(K, pol.block, pol.sub_block, dtype) if summaries is None else summaries
        scores = None if pol.mode == MODE_STREAMING else block_scores(q_rows, S)
    else:
        S = sub_block_means(K, pol.block, pol.sub_block, dtype) if summaries is None else summaries
        scores = None if pol.mode == MODE_STREAMING else sub_block_scores(q_rows, S, pooling)
    sel, ev = select_unit(pol, T, scores, logits, evicted)
    tok = selected_tokens(sel, pol.block, T)
    bias = None
    if ed and pol.mode == MODE_NOSA:
        bias = token_bias(sel, pol.block, T, logits)
    out, lse = attend(q_rows, K[tok], V[tok], scale, bias)
    return UnitResult(S, scores, sel, ev, round_to_storage(out, dtype), out, lse)
