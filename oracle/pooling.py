"""Two-stage block summaries (oracle; test infrastructure only).

[NOSA-DE] Methodik §1, bullet "Blockweise Implementierung": selection works on
blocks of tokens, and the selection scores come from a two-stage pooling: a mean
inside each sub-block, followed by a max at block level.

Readings taken where the page is silent:
* The pooling acts on the key rows and the max is elementwise over the
  sub-block mean vectors, giving one query-independent d-vector per full block
  (block_summaries).  The other reading, the max taken over the scores of the
  sub-block means, keeps every mean (sub_block_means) and leaves the max to
  scoring.sub_block_scores.
* Only full blocks get a summary; a partial last block has none.
* Precision: the sub-block sums are formed in float64, where they are exact for
  the inputs used here (checked below, the function refuses otherwise); the
  division by the power-of-two sub-block size is exact too.  The block maximum
  is then rounded ONCE, to nearest with ties to even, into the KV storage dtype.
  Rounding is monotone, so max-then-round equals round-then-max.
"""
from __future__ import annotations

import numpy as np

from .numerics import round_to_storage, significant_bits


def _check_exact_sums(x: np.ndarray, p: int) -> None:
    """Refuse inputs whose float64 sub-block sums could be inexact.

    x has shape [..., s, d] and holds values with at most p significant bits.
    Every partial sum is a multiple of 2**L, L = the smallest ulp exponent among
    the nonzero terms, and is bounded by sum |x|; if that bound is below 2**(L+52)
    every partial sum fits in float64's 53-bit significand.
    """
    nz = x != 0
    _, e = np.frexp(x)
    ulp_e = np.where(nz, e - p, np.iinfo(np.int32).max)
    L = ulp_e.min(axis=-2)
    bound = np.abs(x).sum(axis=-2)
    ok = (bound == 0) | (bound < np.ldexp(1.0, np.minimum(L, 960) + 52))
    if not np.all(ok):
        raise ValueError("pooling: a float64 sub-block sum would be inexact for these inputs")


def _exact_means(K: np.ndarray, block: int, sub_block: int, dtype: str) -> np.ndarray:
    """m[j, u] = (sum of the sub_block rows of sub-block u of block j) / sub_block, exact,
    float64 [n_full][block/sub_block][d]."""
    if block % sub_block != 0:
        raise ValueError("sub_block must divide block")
    T, d = K.shape
    n_full = T // block
    x = K[: n_full * block].reshape(n_full, block // sub_block, sub_block, d)
    _check_exact_sums(x, significant_bits(dtype))
    return x.sum(axis=2) / sub_block


def block_summaries(K: np.ndarray, block: int, sub_block: int, dtype: str) -> np.ndarray:
    """Summaries S[j] for the full blocks of one (sequence, kv head).

    K: float64 [T][d], the unit's valid key rows (exact widening of the stored keys).
    Returns float64 [T // block][d], exactly representable in ``dtype``:
        m[j, u] = (sum of the sub_block rows of sub-block u of block j) / sub_block
        S[j]    = round_once(elementwise max over u of m[j, u])
    """
    means = _exact_means(K, block, sub_block, dtype)
    return round_to_storage(means.max(axis=1), dtype)


def sub_block_means(K: np.ndarray, block: int, sub_block: int, dtype: str) -> np.ndarray:
    """The first pooling stage alone, for score-side pooling (the block-level max is
    then taken over scores, not over vectors; see scoring.sub_block_scores).

    Returns float64 [T // block][block // sub_block][d]: every m[j, u] rounded once into
    ``dtype`` (to nearest, ties to even)."""
    return round_to_storage(_exact_means(K, block, sub_block, dtype), dtype)
