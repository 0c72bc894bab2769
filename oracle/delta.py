"""Selection set differences and locality (oracle; test infrastructure only).

[NOSA-DE] Methodik §2 (NOSI), "Optimierte Speicherlayout": the KV cache is kept
in minimal block units, and set differences between consecutive selections
decide which blocks are swapped.  Methodik §1, "Lokalitätsgarantie": the share
of step-t blocks that were already selected at step t-1 is at least k_e / k.

Definitions used:
    added   = cur \\ prev   (ascending)
    removed = prev \\ cur   (ascending)
    gamma   = |cur ∩ prev| / |cur|        (locality of step t against step t-1)
An empty previous selection (the first step) makes every current block "added".
"""
from __future__ import annotations

from typing import Tuple

import numpy as np


def selection_delta(prev: np.ndarray, cur: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    prev = np.asarray(prev, dtype=np.int64)
    cur = np.asarray(cur, dtype=np.int64)
    added = np.setdiff1d(cur, prev)
    removed = np.setdiff1d(prev, cur)
    return added, removed


def locality(prev: np.ndarray, cur: np.ndarray) -> float:
    cur = np.asarray(cur, dtype=np.int64)
    if cur.size == 0:
        return 1.0
    return float(np.intersect1d(prev, cur).size) / float(cur.size)
