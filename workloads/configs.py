"""Workload shapes and per-(sequence, kv-head) policies.

A *unit* is one (sequence b, kv head h), numbered u = b * num_kv_heads + h.
Query head hq belongs to kv head hq // G with G = num_q_heads // num_kv_heads.

Per-block arrays (summaries rows, eviction logits, scores) are packed per unit:
unit u owns n_cap(u) = ceil(t_cap / block(u)) consecutive block slots starting
at block_offset(u) = sum of n_cap over earlier units.  The eviction mask packs
ceil(n_cap(u) / 32) uint32 words per unit the same way.  These layout rules are
the ones the C ABI states; they are repeated here only so the generator can lay
out the eviction logits.
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass, field
from typing import Optional, Tuple

import numpy as np

MODE_RETRIEVAL = 0
MODE_STREAMING = 1
MODE_NOSA = 2

_MODE_NAMES = {MODE_RETRIEVAL: "retrieval", MODE_STREAMING: "streaming", MODE_NOSA: "nosa"}

# Sub-stream purposes for np.random.SeedSequence([seed, purpose, ...]).
P_POLICY, P_QUERY, P_KV, P_NEEDLE, P_LOGITS, P_DRIFT, P_LENS, P_APPEND = 1, 2, 3, 4, 5, 6, 7, 8


@dataclass(frozen=True)
class HeadPolicy:
    """Per-unit selection policy (mirrors fx_head_policy in include/fx.h)."""
    mode: int
    block: int
    sub_block: int
    top_k: int = 0
    budget: float = 0.0        # stored as float32 by the library
    k_evict: int = 0
    sink_tokens: int = 0
    local_tokens: int = 0
    force_sink: int = 0
    force_last: int = 0

    @property
    def mode_name(self) -> str:
        return _MODE_NAMES[self.mode]


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    dtype: str                          # "f32" or "bf16"
    t_cap: int
    seq_lens: Tuple[int, ...]
    policies: Tuple[HeadPolicy, ...]    # one per unit, u = b * Hkv + h
    seed: int
    sink_scaled_tokens: int             # leading tokens whose keys x8 and values x0.1
    needles_per_head: int
    steps: int = 1
    drift: Optional[Tuple[float, float]] = None   # (decay, noise) of the query drift
    description: str = ""
    pooling: int = 0                    # 0 key-side; 1 / 2 score-side with group sum / max

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def num_units(self) -> int:
        return self.batch * self.num_kv_heads

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2

    def n_cap(self, u: int) -> int:
        g = self.policies[u].block
        return -(-self.t_cap // g)

    def block_offsets(self) -> np.ndarray:
        caps = np.array([self.n_cap(u) for u in range(self.num_units)], dtype=np.int64)
        off = np.zeros(self.num_units + 1, dtype=np.int64)
        off[1:] = np.cumsum(caps)
        return off

    def summary_rows_per_block(self, u: int) -> int:
        p = self.policies[u]
        return 1 if self.pooling == 0 else p.block // p.sub_block

    def summary_row_offsets(self) -> np.ndarray:
        rows = np.array([self.n_cap(u) * self.summary_rows_per_block(u)
                         for u in range(self.num_units)], dtype=np.int64)
        off = np.zeros(self.num_units + 1, dtype=np.int64)
        off[1:] = np.cumsum(rows)
        return off

    def mask_word_offsets(self) -> np.ndarray:
        words = np.array([-(-self.n_cap(u) // 32) for u in range(self.num_units)], dtype=np.int64)
        off = np.zeros(self.num_units + 1, dtype=np.int64)
        off[1:] = np.cumsum(words)
        return off

    @property
    def total_blocks(self) -> int:
        return int(self.block_offsets()[-1])

    @property
    def has_nosa(self) -> bool:
        return any(p.mode == MODE_NOSA for p in self.policies)

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


def _rng(seed: int, *keys: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, *keys])))


def _f32(x: float) -> float:
    return float(np.float32(x))


# --------------------------------------------------------------------------------------
# The five workloads.
# --------------------------------------------------------------------------------------

def _tiny(t: int = 2048) -> Workload:
    B, Hq, Hkv, d, g = 1, 4, 2, 64, 32
    pol = HeadPolicy(MODE_RETRIEVAL, block=g, sub_block=16, top_k=8, force_sink=1, force_last=1)
    return Workload(
        name="tiny", batch=B, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=d, dtype="f32",
        t_cap=t, seq_lens=(t,) * B, policies=(pol,) * (B * Hkv), seed=1,
        sink_scaled_tokens=g, needles_per_head=2,
        description="1 seq, 4q/2kv, d64, fp32, T2048, block 32, top-8 + sink block 0 + last block")


def _llama8b_layer(t: int = 32768) -> Workload:
    B, Hq, Hkv, d, g = 1, 32, 8, 128, 64
    stream = HeadPolicy(MODE_STREAMING, block=g, sub_block=16, sink_tokens=64, local_tokens=1024)
    retr = HeadPolicy(MODE_RETRIEVAL, block=g, sub_block=16, budget=_f32(0.05),
                      force_sink=1, force_last=1)
    pols = tuple(stream if h < 4 else retr for _ in range(B) for h in range(Hkv))
    return Workload(
        name="llama8b_layer", batch=B, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=d,
        dtype="bf16", t_cap=t, seq_lens=(t,) * B, policies=pols, seed=2,
        sink_scaled_tokens=4, needles_per_head=8,
        description="1 seq, 32q/8kv, d128, bf16, T32768, block 64; kv 0-3 streaming "
                    "(sink 64 + local 1024), kv 4-7 retrieval budget 5%")


def _qwen7b_layer(batch: int = 4, t: int = 131072) -> Workload:
    B, Hq, Hkv, d = batch, 28, 4, 128
    r = _rng(3, P_POLICY)
    blocks = r.choice(np.array([16, 32, 64, 128]), size=Hkv)
    budgets = r.uniform(0.02, 0.10, size=Hkv)
    head_pol = [HeadPolicy(MODE_RETRIEVAL, block=int(blocks[h]), sub_block=min(16, int(blocks[h])),
                           budget=_f32(budgets[h]), force_sink=1, force_last=1)
                for h in range(Hkv)]
    pols = tuple(head_pol[h] for _ in range(B) for h in range(Hkv))
    return Workload(
        name="qwen7b_layer", batch=B, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=d,
        dtype="bf16", t_cap=t, seq_lens=(t,) * B, policies=pols, seed=3,
        sink_scaled_tokens=4, needles_per_head=8,
        description="4 seqs, 28q/4kv (GQA 7), d128, bf16, T131072; per-kv-head block in "
                    "{16,32,64,128}, budget U[2%,10%]")


def _nosa_drift(batch: int = 32, t: int = 16384, steps: int = 64) -> Workload:
    B, Hq, Hkv, d, g = batch, 32, 8, 128, 64
    pol = HeadPolicy(MODE_NOSA, block=g, sub_block=16, top_k=16, k_evict=48)
    return Workload(
        name="nosa_drift", batch=B, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=d,
        dtype="bf16", t_cap=t, seq_lens=(t,) * B, policies=(pol,) * (B * Hkv), seed=4,
        sink_scaled_tokens=4, needles_per_head=8, steps=steps, drift=(0.9, 0.44),
        description="32 seqs, 32q/8kv, d128, bf16, T16384, block 64 / sub 16; query-aware "
                    "top-16 + eviction top-48 on N(0,1) logits; 64 drift steps")


def _mixed_serving(batch: int = 64, t_min: int = 8192, t_max: int = 131072) -> Workload:
    B, Hq, Hkv, d, g = batch, 32, 8, 128, 64
    r = _rng(5, P_POLICY)
    streaming = r.random(Hkv) < 0.5
    budgets = r.uniform(0.02, 0.10, size=Hkv)
    lens = _rng(5, P_LENS).integers(t_min, t_max, endpoint=True, size=B)
    head_pol = []
    for h in range(Hkv):
        if streaming[h]:
            head_pol.append(HeadPolicy(MODE_STREAMING, block=g, sub_block=16,
                                       sink_tokens=64, local_tokens=1024))
        else:
            head_pol.append(HeadPolicy(MODE_RETRIEVAL, block=g, sub_block=16,
                                       budget=_f32(budgets[h]), force_sink=1, force_last=1))
    pols = tuple(head_pol[h] for _ in range(B) for h in range(Hkv))
    return Workload(
        name="mixed_serving", batch=B, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=d,
        dtype="bf16", t_cap=t_max, seq_lens=tuple(int(x) for x in lens), policies=pols,
        seed=5, sink_scaled_tokens=4, needles_per_head=8,
        description="64 seqs, T U{8192..131072}, 32q/8kv, d128, bf16, block 64; per-kv-head "
                    "streaming/retrieval coin flip, budget U[2%,10%]; ragged")


WORKLOAD_NAMES = ("tiny", "llama8b_layer", "qwen7b_layer", "nosa_drift", "mixed_serving")


def get_workload(name: str) -> Workload:
    """The full-size workload."""
    return {
        "tiny": _tiny,
        "llama8b_layer": _llama8b_layer,
        "qwen7b_layer": _qwen7b_layer,
        "nosa_drift": _nosa_drift,
        "mixed_serving": _mixed_serving,
    }[name]()


def small_workload(name: str) -> Workload:
    """A reduced workload with the same structure that the oracle finishes in seconds.

    Every reduced size spans several split-K chunks and scoring tiles and, except
    for nosa_drift (whose context is block-aligned), ends in a ragged partial block.
    """
    if name == "tiny":
        return _tiny()
    if name == "llama8b_layer":
        w = _llama8b_layer(t=8192 + 37)
        return w.replace(name="llama8b_layer_small")
    if name == "qwen7b_layer":
        w = _qwen7b_layer(batch=2, t=16384 + 5)
        return w.replace(name="qwen7b_layer_small")
    if name == "nosa_drift":
        w = _nosa_drift(batch=2, t=8192, steps=6)
        return w.replace(name="nosa_drift_small")
    if name == "mixed_serving":
        w = _mixed_serving(batch=6, t_min=1000, t_max=20000)
        return w.replace(name="mixed_serving_small")
    raise KeyError(name)
