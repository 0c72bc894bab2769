"""Glue between the HIP library (through its Python binding), the seeded inputs
and the CPU oracle, for the GPU parity tests."""
from __future__ import annotations

import math
import sys
from dataclasses import dataclass
from typing import Dict, List, Optional

import numpy as np
import torch

import block_sparse_decode_summary_amd as fx
from oracle.delta import selection_delta
from oracle.step import unit_step
from workloads import Workload, generate, unit_arrays
from workloads.generate import unit_logits

INT32_MAX = 2 ** 31 - 1

# Output tolerances: |gpu - ref| <= atol + rtol * |ref|
TOL = {"bf16": (2e-2, 1e-2), "f32": (1e-4, 1e-4)}
LSE_TOL = (1e-5, 1e-4)      # (rtol, atol) on the natural-log lse


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def make_plan(w: Workload, split_tokens: int = 0) -> fx.Plan:
    dt = fx.FX_F32 if w.dtype == "f32" else fx.FX_BF16
    return fx.fx_plan_create(w.batch, w.num_q_heads, w.num_kv_heads, w.head_dim, w.t_cap, dt,
                             list(w.policies), split_tokens, w.pooling)


def softmax_scale(w: Workload) -> float:
    return 1.0 / math.sqrt(w.head_dim)


def run_select_decode(plan: fx.Plan, bufs: fx.StepBuffers, inp, q: torch.Tensor,
                      build: bool = True) -> None:
    w = inp.workload
    if build:
        fx.fx_build_summaries(plan, inp.K, inp.seq_lens, 0, INT32_MAX, bufs.summaries)
    fx.fx_select(plan, q, bufs.summaries, inp.logits, bufs.evicted_mask if w.has_nosa else None,
                 inp.seq_lens, bufs.sel_idx, bufs.sel_cnt, bufs.workspace)
    fx.fx_sparse_decode(plan, q, inp.K, inp.V, inp.seq_lens, bufs.sel_idx, bufs.sel_cnt,
                        softmax_scale(w), bufs.out, bufs.lse, bufs.workspace)


@dataclass
class GpuUnit:
    summaries: np.ndarray     # float64 [n_full][d] ([n_full][r][d] under score-side pooling)
    scores: Optional[np.ndarray]
    sel: np.ndarray
    out: np.ndarray           # float64 [G][d]
    lse: np.ndarray           # float64 [G]


class GpuView:
    """Host copies of every GPU output of one step, indexed per unit."""

    def __init__(self, plan: fx.Plan, bufs: fx.StepBuffers, w: Workload):
        torch.cuda.synchronize()
        self.w = w
        self.plan = plan
        self.summ = bufs.summaries.to("cpu").to(torch.float64).numpy().reshape(-1, w.head_dim)
        nb = w.total_blocks
        self.scores = bufs.workspace[: nb * 4].to("cpu").view(torch.float32).numpy().copy()
        self.sel_idx = bufs.sel_idx.to("cpu").numpy().copy()
        self.sel_cnt = bufs.sel_cnt.to("cpu").numpy().copy()
        self.out = bufs.out.to("cpu").to(torch.float64).numpy().copy()
        self.lse = bufs.lse.to("cpu").to(torch.float64).numpy().copy()
        self.mask = bufs.evicted_mask.to("cpu").numpy().view(np.uint32).copy()
        self.block_off = w.block_offsets()
        self.sum_off = w.summary_row_offsets()
        self.mask_off = w.mask_word_offsets()

    def unit(self, u: int) -> GpuUnit:
        w = self.w
        b, h = divmod(u, w.num_kv_heads)
        G = w.group
        T = w.seq_lens[b]
        g = w.policies[u].block
        n_full = T // g
        o = int(self.block_off[u])
        so, r = int(self.sum_off[u]), w.summary_rows_per_block(u)
        summ = self.summ[so:so + n_full * r]
        cnt = int(self.sel_cnt[u])
        return GpuUnit(
            summaries=summ if w.pooling == 0 else summ.reshape(n_full, r, w.head_dim),
            scores=self.scores[o:o + n_full] if w.policies[u].mode != fx.FX_STREAMING else None,
            sel=self.sel_idx[u, :cnt].astype(np.int64),
            out=self.out[b, h * G:(h + 1) * G],
            lse=self.lse[b, h * G:(h + 1) * G],
        )

    def padding_ok(self, u: int) -> bool:
        cnt = int(self.sel_cnt[u])
        return bool(np.all(self.sel_idx[u, cnt:] == -1))

    def evicted(self, u: int) -> np.ndarray:
        n = self.w.n_cap(u)
        words = self.mask[int(self.mask_off[u]):int(self.mask_off[u + 1])]
        bits = np.unpackbits(words.view(np.uint8), bitorder="little")[:n]
        return bits.astype(bool)


def oracle_unit(inp, u: int, q: torch.Tensor, evicted: Optional[np.ndarray] = None,
                ed: bool = False):
    w = inp.workload
    b, h = divmod(u, w.num_kv_heads)
    q_rows, K, V = unit_arrays(inp, b, h, q=q)
    return unit_step(w.policies[u], w.seq_lens[b], w.dtype, q_rows, K, V, softmax_scale(w),
                     logits=unit_logits(inp, u), evicted=evicted, ed=ed, pooling=w.pooling)


def assert_close(name: str, got: np.ndarray, ref: np.ndarray, rtol: float, atol: float) -> float:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    both_neginf = np.isneginf(got) & np.isneginf(ref)
    with np.errstate(invalid="ignore"):
        err = np.where(both_neginf, 0.0, np.abs(got - ref))
    lim = atol + rtol * np.abs(np.where(both_neginf, 0.0, ref))
    bad = ~(err <= lim)
    if np.any(bad):
        i = np.argwhere(bad)[0]
        raise AssertionError(f"{name}: {bad.sum()} elements out of tolerance; first at {tuple(i)}: "
                             f"got {got[tuple(i)]} ref {ref[tuple(i)]} (rtol {rtol}, atol {atol})")
    return float(np.max(err / np.maximum(lim, 1e-300))) if err.size else 0.0


def compare_unit(w: Workload, u: int, gv: GpuView, ref, check_scores: bool = True) -> None:
    g = gv.unit(u)
    tag = f"{w.name} unit {u}"
    assert np.array_equal(g.summaries, ref.summaries), f"{tag}: summaries differ"
    if check_scores and ref.scores is not None:
        assert np.array_equal(g.scores.view(np.uint32) if g.scores.dtype == np.float32 else g.scores,
                              ref.scores.view(np.uint32)), f"{tag}: scores differ"
    assert np.array_equal(g.sel, ref.sel), f"{tag}: selection differs: {g.sel} vs {ref.sel}"
    assert gv.padding_ok(u), f"{tag}: sel_idx padding"
    rtol, atol = TOL[w.dtype]
    assert_close(f"{tag} out", g.out, ref.out_exact, rtol, atol)
    assert_close(f"{tag} lse", g.lse, ref.lse, *LSE_TOL)
