"""Per-kv-head block selection (oracle; test infrastructure only).

Sources:
* [Fluxion-NL] Kerninzichten item 2 and Systeemcomponenten: heads are either
  streaming heads, which make do with the default retained KV, or retrieval heads,
  which need top-k selection at a per-head granularity (block size) and budget.
  [Fluxion-KO] section 해결책, strategy 2: streamers look only at the most
  recent pages, retrievers dig into the archive.
* [Fluxion-NL] Probleemstelling item 1: top-k selection followed by sparse
  attention is the GPU-side procedure.
* [NOSA-DE] Methodik §1, "Dual-Selection-Mechanismus": the selection is the
  union of a query-aware part Γq and a query-agnostic part Γe chosen by an
  eviction head, with strict eviction: what Γe drops at step t can never
  re-enter Γe later.  "Lokalitätsgarantie": Γe has a fixed budget k_e.
  "ED-DMA": blocks are chosen on pre-exponential scores, so the eviction logits
  are ranked as they are, never exponentiated.

Readings (the pages give no formulas):
* Blocks of one unit: block j covers tokens [j*g, min((j+1)*g, T)).
  n_full = T // g full blocks, n_tot = ceil(T / g) blocks in all.
* Forced set F:
    streaming : every block overlapping [0, min(sink, T)) or [max(0, T - local), T);
    retrieval, NOSA : {0} if force_sink, {n_tot - 1} if force_last;
    all modes : the partial last block, if any (it has no summary, so it can be
                neither scored nor evicted, and it holds the newest tokens).
* Retrieval budget: k = top_k if top_k > 0, else ceil(budget * n_tot), evaluated
  in float64 from the float32 budget (the product is exact).  Forced blocks come on
  top of k; k is clamped to the number of candidates (full blocks not in F).
* Order: larger value first, equal values by lower block index; -0.0 == +0.0.
* NOSA: E = full blocks not in F and not yet evicted; Γe = top k_e of E by
  logit; every block of E outside Γe becomes evicted.  Γq = top top_k by score
  among full blocks in neither F nor Γe -- evicted blocks stay eligible for Γq.
  Selection = F ∪ Γe ∪ Γq.
* Output: the selected block indices in ascending order.
"""
from __future__ import annotations

import math
from typing import Optional, Tuple

import numpy as np

MODE_RETRIEVAL, MODE_STREAMING, MODE_NOSA = 0, 1, 2


def block_counts(T: int, g: int) -> Tuple[int, int]:
    """(n_full, n_tot) for a context of T tokens in blocks of g."""
    return T // g, -(-T // g)


def forced_blocks(pol, T: int) -> np.ndarray:
    """Ascending forced block indices F of one unit (see module docstring)."""
    g = pol.block
    n_full, n_tot = block_counts(T, g)
    F = set()
    if n_tot == 0:
        return np.zeros(0, dtype=np.int64)
    if pol.mode == MODE_STREAMING:
        sink_end = min(pol.sink_tokens, T)
        F.update(range(0, -(-sink_end // g)))                  # blocks with j*g < sink_end
        if pol.local_tokens > 0:
            start = max(0, T - pol.local_tokens)
            F.update(range(start // g, n_tot))                  # blocks with end > start
    else:
        if pol.force_sink:
            F.add(0)
        if pol.force_last:
            F.add(n_tot - 1)
    if n_full < n_tot:
        F.add(n_tot - 1)
    return np.array(sorted(F), dtype=np.int64)


def budget_k(pol, n_tot: int) -> int:
    """Blocks the retrieval budget asks for (before clamping to the candidates)."""
    if pol.top_k > 0:
        return int(pol.top_k)
    beta = float(np.float32(pol.budget))
    return int(math.ceil(beta * float(n_tot)))


def top_k(values: np.ndarray, cand: np.ndarray, k: int) -> np.ndarray:
    """The k best candidates (value descending, index ascending), returned ascending.

    values: float32 per block index; cand: candidate block indices.
    """
    cand = np.asarray(cand, dtype=np.int64)
    k = min(int(k), cand.size)
    if k <= 0:
        return np.zeros(0, dtype=np.int64)
    v = np.asarray(values, dtype=np.float32)[cand].astype(np.float64)
    if not np.all(np.isfinite(v)):
        raise ValueError("top_k: non-finite value")
    order = np.lexsort((cand, -v))       # primary key -v (value desc), then index asc
    return np.sort(cand[order[:k]])


def select_unit(pol, T: int, scores: Optional[np.ndarray] = None,
                logits: Optional[np.ndarray] = None,
                evicted: Optional[np.ndarray] = None):
    """Selection of one unit at one step.

    scores : float32 [>= n_full] block scores (retrieval and NOSA modes)
    logits : float32 [>= n_full] eviction logits (NOSA mode)
    evicted: bool [>= n_full] eviction state before this step (NOSA mode)
    Returns (selected ascending int64 array, evicted after this step or None).
    """
    g = pol.block
    n_full, n_tot = block_counts(T, g)
    F = forced_blocks(pol, T)
    if pol.mode == MODE_STREAMING:
        return F, evicted
    full = np.arange(n_full, dtype=np.int64)
    not_forced = full[~np.isin(full, F)]
    if pol.mode == MODE_RETRIEVAL:
        chosen = top_k(scores, not_forced, budget_k(pol, n_tot))
        return np.union1d(F, chosen).astype(np.int64), evicted
    if pol.mode == MODE_NOSA:
        ev = np.zeros(n_full, dtype=bool) if evicted is None else np.asarray(evicted, dtype=bool).copy()
        E = not_forced[~ev[not_forced]]
        gamma_e = top_k(logits, E, pol.k_evict)
        ev[np.setdiff1d(E, gamma_e)] = True
        cand_q = np.setdiff1d(not_forced, gamma_e)
        gamma_q = top_k(scores, cand_q, pol.top_k)
        sel = np.union1d(np.union1d(F, gamma_e), gamma_q).astype(np.int64)
        return sel, ev
    raise ValueError(f"unknown mode {pol.mode}")
