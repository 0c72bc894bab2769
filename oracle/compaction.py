"""Delta-driven compaction of the selected blocks into a block-slot working set
(oracle; test infrastructure only).

[NOSA-DE] Methodik §2 (NOSI), "Optimierte Speicherlayout": the KV cache is held in
minimal block units, and the set difference between what is selected and what is
already held decides which blocks are swapped, so no contiguous allocation is needed.
Here the held copy is a per-unit array of block slots in the same HBM; a step moves
only the blocks that became selected.

Readings (the page gives no algorithm):
* The working set of a unit holds its selected FULL blocks (j < n_full).  The partial
  last block is not held: it still grows, and attention reads it from the cache.
* A slot whose block is no longer a selected full block becomes free (-1).
* The selected full blocks not yet held ("added", ascending) take the free slots in
  ascending slot order, the i-th added block the i-th free slot.  Held blocks never
  change slot.
* Moving a block copies its g key rows and g value rows into the slot.
"""
from __future__ import annotations

from typing import List, Tuple

import numpy as np


def held_target(sel: np.ndarray, T: int, g: int) -> np.ndarray:
    """The selected full blocks (ascending)."""
    sel = np.asarray(sel, dtype=np.int64)
    return sel[sel < T // g]


def compact_update(slot_map: np.ndarray, sel: np.ndarray, T: int, g: int
                   ) -> Tuple[np.ndarray, List[Tuple[int, int]]]:
    """New slot map and the moves [(slot, block)] of one unit, in slot order."""
    slots = np.array(slot_map, dtype=np.int64, copy=True)
    target = held_target(sel, T, g)
    if target.size > slots.size:
        raise ValueError("more selected full blocks than slots")
    tset = set(int(b) for b in target)
    for s in range(slots.size):
        if slots[s] >= 0 and int(slots[s]) not in tset:
            slots[s] = -1
    held = set(int(b) for b in slots if b >= 0)
    added = [int(b) for b in target if int(b) not in held]
    free = [s for s in range(slots.size) if slots[s] < 0]
    moves = list(zip(free[:len(added)], added))
    for s, b in moves:
        slots[s] = b
    return slots, moves


def apply_moves(work_K: np.ndarray, work_V: np.ndarray, K: np.ndarray, V: np.ndarray,
                moves: List[Tuple[int, int]], g: int) -> None:
    """Copy block b's rows into slot s for every move (work_* are [slots * g][d])."""
    for s, b in moves:
        work_K[s * g:(s + 1) * g] = K[b * g:(b + 1) * g]
        work_V[s * g:(s + 1) * g] = V[b * g:(b + 1) * g]
