"""Attention over the selected blocks (oracle; test infrastructure only).

[Fluxion-NL] Probleemstelling item 1: after top-k selection, attention runs
over the selected KV blocks only.  [NOSA-DE] Methodik §1, "ED-DMA": the
exponential belongs to the attention computation.

Definition used (standard scaled dot-product attention restricted to a token
set): for a query row q and the selected tokens t,
    s_t = (q . k_t) * scale          (scale = 1/sqrt(d) unless given)
    m   = max_t s_t,  l = sum_t exp(s_t - m)
    out = sum_t exp(s_t - m) v_t / l,  lse = m + ln l
computed in float64; out is rounded once to the storage dtype by the caller.
An empty token set gives out = 0 and lse = -inf.

Exp-delayed eviction scores in attention ([NOSA-DE] Methodik §1, "ED-DMA").  The
page says only that the eviction head's exponential is taken in the attention
phase and that selection ranks the values before it.  Reading used here: the raw
eviction logit b_j of block j is added to the attention logit of each of the
block's tokens before the softmax,
    s_t = (q . k_t) * scale + b_{block(t)},
so exp(b_j) multiplies the block's unnormalised weights and is never formed on its
own.  ``bias`` below is that per-token term (None: no term).

The split-K merge states how partial results over disjoint token sets combine:
    M = max_i m_i,  L = sum_i l_i exp(m_i - M),
    out = sum_i o_i exp(m_i - M) / L,  lse = M + ln L,
where o_i is the unnormalised sum_t exp(s_t - m_i) v_t of part i.
"""
from __future__ import annotations

from typing import List, Optional, Tuple

import numpy as np


def selected_tokens(sel: np.ndarray, g: int, T: int) -> np.ndarray:
    """Ascending token indices covered by the selected blocks (valid tokens only)."""
    parts = [np.arange(j * g, min((j + 1) * g, T), dtype=np.int64) for j in np.asarray(sel)]
    if not parts:
        return np.zeros(0, dtype=np.int64)
    return np.concatenate(parts)


def token_bias(sel: np.ndarray, g: int, T: int, block_logits: np.ndarray) -> np.ndarray:
    """Per-token term of the selected tokens (order of selected_tokens): b_j repeated
    over the valid tokens of block j."""
    b = np.asarray(block_logits, dtype=np.float64)
    parts = [np.full(min((j + 1) * g, T) - j * g, b[j]) for j in np.asarray(sel)]
    return np.concatenate(parts) if parts else np.zeros(0)


def _logits(q_rows: np.ndarray, K_rows: np.ndarray, scale: float, bias) -> np.ndarray:
    s = (q_rows @ np.asarray(K_rows, dtype=np.float64).T) * scale     # [G][n]
    if bias is not None:
        s = s + np.asarray(bias, dtype=np.float64)[None, :]
    return s


def attend(q_rows: np.ndarray, K_sel: np.ndarray, V_sel: np.ndarray, scale: float,
           bias: Optional[np.ndarray] = None) -> Tuple[np.ndarray, np.ndarray]:
    """(out [G][d], lse [G]) of the query rows over the given key/value rows, float64.
    ``bias`` (float64 [n] or None) is added to every row's logits."""
    q_rows = np.asarray(q_rows, dtype=np.float64)
    G, d = q_rows.shape
    if K_sel.shape[0] == 0:
        return np.zeros((G, V_sel.shape[1])), np.full(G, -np.inf)
    s = _logits(q_rows, K_sel, scale, bias)
    m = s.max(axis=1, keepdims=True)
    p = np.exp(s - m)
    l = p.sum(axis=1, keepdims=True)
    out = (p @ np.asarray(V_sel, dtype=np.float64)) / l
    lse = m[:, 0] + np.log(l[:, 0])
    return out, lse


def partial(q_rows: np.ndarray, K_part: np.ndarray, V_part: np.ndarray, scale: float,
            bias: Optional[np.ndarray] = None) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Unnormalised partial (m [G], l [G], o [G][d]) over one part of the token set."""
    q_rows = np.asarray(q_rows, dtype=np.float64)
    G = q_rows.shape[0]
    if K_part.shape[0] == 0:
        return np.full(G, -np.inf), np.zeros(G), np.zeros((G, V_part.shape[1]))
    s = _logits(q_rows, K_part, scale, bias)
    m = s.max(axis=1)
    p = np.exp(s - m[:, None])
    return m, p.sum(axis=1), p @ np.asarray(V_part, dtype=np.float64)


def merge_partials(parts: List[Tuple[np.ndarray, np.ndarray, np.ndarray]]
                   ) -> Tuple[np.ndarray, np.ndarray]:
    """Combine partials of disjoint token sets into (out, lse)."""
    ms = np.stack([p[0] for p in parts])                # [n][G]
    M = ms.max(axis=0)
    if np.all(np.isneginf(M)):
        G, d = parts[0][2].shape
        return np.zeros((G, d)), np.full(G, -np.inf)
    w = np.where(np.isneginf(ms), 0.0, np.exp(ms - M))  # [n][G]
    L = sum(w[i] * parts[i][1] for i in range(len(parts)))
    O = sum(w[i][:, None] * parts[i][2] for i in range(len(parts)))
    return O / L[:, None], M + np.log(L)
