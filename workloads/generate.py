"""Seeded input generation.

Recipe (identical for the HIP library and the oracle, which both receive these
tensors):

* q  : N(0, 1), drawn on the host (numpy PCG64, float64), stored in the
       workload dtype (float32, or float32 then round-to-nearest-even bfloat16).
       With query drift, q_t = a * q_{t-1} + b * N(0, 1) on the float64 state,
       and step t stores the rounded q_t.
* K,V: N(0, 1) noise drawn with torch's generator on the target device (float32),
       then:
         - needles: per (seq, kv head), ``needles_per_head`` distinct full blocks
           other than block 0 and the last block get keys 3 * qbar + noise, where
           qbar is the mean of the group's G stored query rows at step 0;
         - sink: the first ``sink_scaled_tokens`` tokens get keys x8, values x0.1;
       then rounded to the workload dtype.  Rows at or beyond a sequence's length
       stay zero.
* eviction logits (workloads with NOSA heads): N(0, 1) float32 per block slot.
* decode-loop growth (append_tokens): step t appends to sequence b one key row and one
  value row per kv head, N(0, 1) from torch's generator seeded by (seed, append, b, t),
  rounded to the workload dtype, at position seq_len(b).

Sub-streams come from np.random.SeedSequence([seed, purpose, ...]) so that any
(sequence, kv head) can be regenerated on its own.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Optional, Tuple

import numpy as np
import torch

from .configs import (Workload, MODE_NOSA, P_QUERY, P_KV, P_NEEDLE, P_LOGITS, P_DRIFT,
                      P_APPEND, _rng)


def storage_dtype(w: Workload) -> torch.dtype:
    return torch.float32 if w.dtype == "f32" else torch.bfloat16


def _seed32(seed: int, *keys: int) -> int:
    return int(np.random.SeedSequence([seed, *keys]).generate_state(1, dtype=np.uint64)[0]
               & 0x7FFF_FFFF_FFFF_FFFF)


_DRIFT_CACHE: Dict[Tuple, List[np.ndarray]] = {}


def _query_states(w: Workload, upto: int) -> List[np.ndarray]:
    """float64 query states q_0 .. q_upto (inclusive)."""
    key = (w.name, w.seed, w.batch, w.num_q_heads, w.head_dim, w.drift)
    states = _DRIFT_CACHE.setdefault(key, [])
    shape = (w.batch, w.num_q_heads, w.head_dim)
    if not states:
        states.append(_rng(w.seed, P_QUERY).standard_normal(shape))
    if upto > 0 and w.drift is None:
        raise ValueError(f"workload {w.name} has no query drift")
    while len(states) <= upto:
        t = len(states)
        a, b = w.drift
        eps = _rng(w.seed, P_DRIFT, t).standard_normal(shape)
        states.append(a * states[-1] + b * eps)
    return states


def query_at_step(w: Workload, step: int, device="cpu") -> torch.Tensor:
    """Stored query [B][Hq][d] at decode step ``step`` in the workload dtype."""
    q64 = _query_states(w, step)[step]
    return torch.from_numpy(q64.astype(np.float32)).to(device=device).to(storage_dtype(w))


@dataclass
class Inputs:
    workload: Workload
    device: torch.device
    q: torch.Tensor                       # [B][Hq][d], step 0
    K: torch.Tensor                       # [B][Hkv][t_cap][d]
    V: torch.Tensor                       # [B][Hkv][t_cap][d]
    seq_lens: torch.Tensor                # int32 [B]
    logits: Optional[torch.Tensor]        # float32 [total_blocks] or None
    needles: Dict[Tuple[int, int], List[int]] = field(default_factory=dict)


def _needle_blocks(w: Workload, b: int, h: int) -> List[int]:
    u = b * w.num_kv_heads + h
    g = w.policies[u].block
    T = w.seq_lens[b]
    n_full, n_tot = T // g, -(-T // g)
    cand = [j for j in range(1, n_full) if j != n_tot - 1]
    n = min(w.needles_per_head, len(cand))
    if n == 0:
        return []
    r = _rng(w.seed, P_NEEDLE, b, h)
    return sorted(int(x) for x in r.choice(np.array(cand), size=n, replace=False))


def generate(w: Workload, device="cpu") -> Inputs:
    device = torch.device(device)
    B, Hq, Hkv, d, G = w.batch, w.num_q_heads, w.num_kv_heads, w.head_dim, w.group
    sdt = storage_dtype(w)
    q = query_at_step(w, 0, device)
    qbar = q.to(torch.float32).reshape(B, Hkv, G, d).mean(dim=2)   # [B][Hkv][d]

    K = torch.zeros((B, Hkv, w.t_cap, d), dtype=sdt, device=device)
    V = torch.zeros((B, Hkv, w.t_cap, d), dtype=sdt, device=device)
    needles: Dict[Tuple[int, int], List[int]] = {}
    for b in range(B):
        T = w.seq_lens[b]
        gk = torch.Generator(device=device)
        gk.manual_seed(_seed32(w.seed, P_KV, b, 0))
        kb = torch.randn((Hkv, T, d), generator=gk, device=device, dtype=torch.float32)
        gv = torch.Generator(device=device)
        gv.manual_seed(_seed32(w.seed, P_KV, b, 1))
        vb = torch.randn((Hkv, T, d), generator=gv, device=device, dtype=torch.float32)
        for h in range(Hkv):
            g = w.policies[b * Hkv + h].block
            blocks = _needle_blocks(w, b, h)
            needles[(b, h)] = blocks
            for j in blocks:
                kb[h, j * g:(j + 1) * g] += 3.0 * qbar[b, h]
        ns = min(w.sink_scaled_tokens, T)
        kb[:, :ns] *= 8.0
        vb[:, :ns] *= 0.1
        K[b, :, :T] = kb.to(sdt)
        V[b, :, :T] = vb.to(sdt)
        del kb, vb

    logits = None
    if w.has_nosa:
        off = w.block_offsets()
        lg = np.zeros(int(off[-1]), dtype=np.float32)
        for u in range(w.num_units):
            n = int(off[u + 1] - off[u])
            lg[off[u]:off[u + 1]] = _rng(w.seed, P_LOGITS, u).standard_normal(n).astype(np.float32)
        logits = torch.from_numpy(lg).to(device)

    seq_lens = torch.tensor(w.seq_lens, dtype=torch.int32, device=device)
    return Inputs(workload=w, device=device, q=q, K=K, V=V, seq_lens=seq_lens,
                  logits=logits, needles=needles)


def append_tokens(inp: Inputs, lens: List[int], step: int) -> List[int]:
    """Append one decode token to every sequence shorter than t_cap (seeded key and
    value rows at position lens[b]) and store the new lengths in inp.seq_lens.  Returns
    the new host-side lengths; inp.workload keeps the lengths it was generated with."""
    w = inp.workload
    new = list(lens)
    for b in range(w.batch):
        T = lens[b]
        if T >= w.t_cap:
            continue
        gen = torch.Generator(device=inp.device)
        gen.manual_seed(_seed32(w.seed, P_APPEND, b, step))
        kv = torch.randn((2, w.num_kv_heads, w.head_dim), generator=gen, device=inp.device,
                         dtype=torch.float32)
        inp.K[b, :, T] = kv[0].to(inp.K.dtype)
        inp.V[b, :, T] = kv[1].to(inp.V.dtype)
        new[b] = T + 1
    inp.seq_lens.copy_(torch.tensor(new, dtype=torch.int32, device=inp.device))
    return new


def unit_arrays(inp: Inputs, b: int, h: int, q: Optional[torch.Tensor] = None
                ) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Host float64 copies of one unit's query rows [G][d] and valid K, V rows [T][d].

    Widening float32 / bfloat16 to float64 is exact.
    """
    w = inp.workload
    G = w.group
    T = w.seq_lens[b]
    qq = inp.q if q is None else q
    q_rows = qq[b, h * G:(h + 1) * G].to("cpu").to(torch.float64).numpy()
    K = inp.K[b, h, :T].to("cpu").to(torch.float64).numpy()
    V = inp.V[b, h, :T].to("cpu").to(torch.float64).numpy()
    return q_rows, K, V


def unit_logits(inp: Inputs, u: int) -> Optional[np.ndarray]:
    if inp.logits is None:
        return None
    off = inp.workload.block_offsets()
    return inp.logits[int(off[u]):int(off[u + 1])].to("cpu").numpy().astype(np.float32)
