#!/usr/bin/env python3
"""Benchmark one block-sparse decode step on one MI355X.

A step is one pass of the whole hot path over one batch of synthetic input:
  fx_build_summaries  (the newest full block of every unit, as when a block fills)
  fx_select_delta     (scores + per-kv-head selection + the differences against the
                       previous step's selection, formed by the selection kernel)
  fx_sparse_decode    (attention over the selected blocks in equal segments + merge)
(`--separate-delta`: fx_select, fx_sparse_decode, then fx_selection_delta.)
Inputs are resident in HBM before timing starts.  The timed steps carry events only at
their boundaries (an event between two kernels delays the second by a few microseconds);
the decode time, the select + decode time and the phase split are each measured in a
further pass over the same steps with events around just that part; those passes use
fx_select and fx_selection_delta as separate calls, so that select + decode is the pair
fx_select + fx_sparse_decode alone.  The default workload is the mixed serving batch
(64 sequences of U{8192..131072} tokens, 32 q / 8 kv heads, d 128, bf16, block 64,
streaming/retrieval kv heads), the largest of the five workloads.

Prints ONE JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "effective KV GB/s read (and µs) per sparse decode step, % of HBM peak"
HBM_PEAK_GBS = 8000.0      # MI355X HBM3E, published
INT32_MAX = 2 ** 31 - 1


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def algorithmic_bytes(w, max_sel, sel_idx, sel_cnt, ed=False):
    """The method's own HBM traffic for one step (decode partials and scores excluded).

    Per unit: KV = 2 d e N (N = valid tokens of the selected blocks); summaries read by
    scoring = n_full r d e (retrieval / NOSA units; r summary rows per block, 1 unless
    pooling is score-side); newest-block summary build = g d e read + r d e write; NOSA logits n_full * 4 and mask words read + written (with the eviction
    term in attention, also 4 bytes per selected block of a NOSA unit).  Shared: q read by
    select and decode, out written, lse written, selection indices written by select,
    read by decode, read twice and written twice (padded) by the delta.
    """
    import numpy as np
    e, d = w.elem_bytes, w.head_dim
    parts = dict(kv=0, summaries=0, build=0, logits_mask=0, q=0, out=0, lse=0, indices=0,
                 ed_logits=0)
    n_q = w.batch * w.num_q_heads
    tot_cnt = 0
    for u in range(w.num_units):
        b = u // w.num_kv_heads
        p = w.policies[u]
        T, g = w.seq_lens[b], p.block
        n_full = T // g
        r = w.summary_rows_per_block(u)
        cnt = int(sel_cnt[u])
        tot_cnt += cnt
        sel = sel_idx[u, :cnt].astype(np.int64)
        N = int(np.minimum(g, T - sel * g).clip(min=0).sum())
        parts["kv"] += 2 * d * e * N
        if p.mode != 1:
            parts["summaries"] += n_full * r * d * e
        if n_full >= 1:
            parts["build"] += g * d * e + r * d * e
        if p.mode == 2:
            parts["logits_mask"] += n_full * 4 + 2 * 4 * (-(-n_full // 32))
            if ed:
                parts["ed_logits"] += cnt * 4
    parts["q"] = 2 * n_q * d * e
    parts["out"] = n_q * d * e
    parts["lse"] = n_q * 4
    parts["indices"] = (w.num_units * max_sel * 4) + tot_cnt * 4 + 2 * tot_cnt * 4 \
        + 2 * w.num_units * max_sel * 4
    total = sum(parts.values())
    decode = (parts["kv"] + n_q * d * e + parts["out"] + parts["lse"] + tot_cnt * 4
              + parts["ed_logits"])
    # fx_select + fx_sparse_decode alone: no summary build, no delta.
    sel_dec = (parts["kv"] + parts["summaries"] + parts["logits_mask"] + parts["q"] + parts["out"]
               + parts["lse"] + w.num_units * max_sel * 4 + tot_cnt * 4 + parts["ed_logits"])
    return total, decode, sel_dec, parts


def decode_source_hash() -> str:
    import hashlib
    path = os.path.join(ROOT, "block_sparse_decode_summary_amd", "csrc", "k_decode.hip")
    return hashlib.sha256(open(path, "rb").read()).hexdigest()[:16]


def measured_traffic(workload: str):
    """HBM bytes per fx_sparse_decode call from the committed counter summary, or None
    when no summary exists for this workload or the decode source changed since."""
    path = os.path.join(ROOT, "profiles", f"k_decode_{workload}_hbm_traffic.md")
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line and line.startswith("- "):
            k, v = line[2:].rsplit(":", 1)
            fields[k.strip()] = v.strip().strip("`")
    if fields.get("k_decode.hip sha256[:16]") != decode_source_hash():
        return None
    try:
        return int(fields["traffic bytes per call"])
    except (KeyError, ValueError):
        return None


# ---- CPU baseline: the oracle on the host's cores ----------------------------------------
#
# A pool of worker processes, started before this process touches the GPU (spawned
# interpreters that import only NumPy and the oracle, one BLAS thread each).  After the GPU
# timing, each worker receives its share of a seeded sample of the workload's units (the
# same tensors the GPU read), widens them to float64 and builds their summaries (untimed,
# as the GPU's are resident), then runs the oracle's decode step over them a given number
# of times; the wall time runs from the "run" message to the last worker's answer.

def _oracle_worker(conn) -> None:
    import time as _time

    import numpy as np
    from threadpoolctl import threadpool_limits

    from oracle.delta import selection_delta
    from oracle.pooling import block_summaries, sub_block_means
    from oracle.step import unit_step

    def widen(a, dtype):
        if dtype == "bf16":
            return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        return a.astype(np.float64)

    held = []
    with threadpool_limits(limits=1):
        while True:
            msg = conn.recv()
            if msg[0] == "load":
                for sp in msg[1]:
                    K, V = widen(sp["K"], sp["dtype"]), widen(sp["V"], sp["dtype"])
                    pool_fn = block_summaries if sp["pooling"] == 0 else sub_block_means
                    summ = pool_fn(K, sp["pol"].block, sp["pol"].sub_block, sp["dtype"])
                    held.append((sp, K, V, summ, pool_fn))
                conn.send(("loaded", len(held)))
            elif msg[0] == "run":
                reps, done, nbytes = msg[1], 0, 0
                t0 = _time.perf_counter()
                for _ in range(reps):
                    for sp, K, V, summ, pool_fn in held:
                        pol, T, g = sp["pol"], sp["T"], sp["pol"].block
                        n_full = T // g
                        if n_full >= 1:
                            pool_fn(K[(n_full - 1) * g:n_full * g], g, pol.sub_block, sp["dtype"])
                        r = unit_step(pol, T, sp["dtype"], sp["q"], K, V, sp["scale"],
                                      logits=sp["logits"], summaries=summ, ed=sp["ed"],
                                      pooling=sp["pooling"])
                        selection_delta(np.zeros(0, np.int64), r.sel)
                        N = int(np.minimum(g, T - r.sel * g).clip(min=0).sum())
                        nbytes += 2 * sp["d"] * sp["e"] * N + sp["fixed_bytes"]
                        done += 1
                conn.send(("done", _time.perf_counter() - t0, nbytes, done))
            else:
                conn.close()
                return


class OraclePool:
    """Worker processes for the CPU baseline (start before the GPU is touched)."""

    def __init__(self, n: int):
        import multiprocessing as mp
        ctx = mp.get_context("spawn")
        saved = {k: os.environ.get(k) for k in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS",
                                                "MKL_NUM_THREADS")}
        os.environ.update({k: "1" for k in saved})
        self.conns, self.procs = [], []
        try:
            for _ in range(n):
                a, b = ctx.Pipe()
                p = ctx.Process(target=_oracle_worker, args=(b,), daemon=True)
                p.start()
                self.conns.append(a)
                self.procs.append(p)
        finally:
            for k, v in saved.items():
                if v is None:
                    os.environ.pop(k, None)
                else:
                    os.environ[k] = v

    def close(self) -> None:
        for c in self.conns:
            try:
                c.send(("stop",))
            except Exception:
                pass
        for p in self.procs:
            p.join(timeout=10)
            if p.is_alive():
                p.terminate()


def cpu_baseline(pool: OraclePool, w, inp, seconds: float, seed: int = 0, ed: bool = False,
                 max_units: int = 128):
    """Time the oracle on a bounded sample of this workload's units on the pool's cores."""
    import numpy as np
    import torch

    from workloads.generate import unit_logits

    n = len(pool.conns)
    rng = np.random.default_rng(seed)
    units = sorted(rng.permutation(w.num_units)[:max_units].tolist())
    scale = 1.0 / math.sqrt(w.head_dim)
    e, d, G = w.elem_bytes, w.head_dim, w.group
    raw = torch.int16 if w.dtype == "bf16" else torch.float32
    shares = [[] for _ in range(n)]
    load = [0] * n
    # Longest first, each to the least loaded worker (a unit's cost grows with its length).
    units.sort(key=lambda u: -w.seq_lens[u // w.num_kv_heads])
    for u in units:
        i = load.index(min(load))
        b, h = divmod(int(u), w.num_kv_heads)
        load[i] += w.seq_lens[b] + 1
        p = w.policies[u]
        T, g = w.seq_lens[b], p.block
        n_full = T // g
        rr = w.summary_rows_per_block(int(u))
        host = lambda x: x.to("cpu").view(raw).numpy()
        shares[i].append(dict(
            pol=p, T=T, dtype=w.dtype, pooling=w.pooling, ed=ed, scale=scale, d=d, e=e,
            q=inp.q[b, h * G:(h + 1) * G].to("cpu").to(torch.float64).numpy(),
            K=host(inp.K[b, h, :T]).view(np.uint16) if w.dtype == "bf16" else host(inp.K[b, h, :T]),
            V=host(inp.V[b, h, :T]).view(np.uint16) if w.dtype == "bf16" else host(inp.V[b, h, :T]),
            logits=unit_logits(inp, int(u)),
            fixed_bytes=(n_full * rr * d * e if p.mode != 1 else 0)
            + (g * d * e + rr * d * e if n_full else 0) + 3 * G * d * e + G * 4))
    for c, sh in zip(pool.conns, shares):
        c.send(("load", sh))
    for c in pool.conns:
        assert c.recv()[0] == "loaded"
    # One pass to size the repetitions to about `seconds` of CPU work in total.
    t0 = time.perf_counter()
    for c in pool.conns:
        c.send(("run", 1))
    cpu_one = sum(c.recv()[1] for c in pool.conns)
    reps = max(1, int(round(seconds / max(cpu_one, 1e-6))))
    t0 = time.perf_counter()
    for c in pool.conns:
        c.send(("run", reps))
    res = [c.recv() for c in pool.conns]
    wall = time.perf_counter() - t0
    nbytes = sum(r[2] for r in res)
    steps = sum(r[3] for r in res)
    cpu = sum(r[1] for r in res)
    return {
        "value": nbytes / wall / 1e9, "unit": "GB/s", "cores": n, "kind": "oracle",
        "sample": f"{len(units)} of {w.num_units} (sequence, kv head) units of {w.name} (seeded "
                  f"sample), each run {reps} times ({steps} unit-steps: newest-block summary + "
                  f"scores + selection + attention + delta; the other summaries precomputed as "
                  f"on the GPU), float64 NumPy oracle in {n} worker processes with 1 BLAS "
                  f"thread each; {nbytes / 1e6:.1f} MB algorithmic in {wall:.2f} s wall "
                  f"({cpu:.1f} s of CPU time)",
    }


def graph_replay(fx, plan, w, inp, A, Bsel, q, logits, mask, scale, flush_buf, reps):
    """Median microseconds of one step (newest-block build, fx_select_delta, fx_sparse_decode)
    and of fx_select + fx_sparse_decode, each captured once in a HIP graph and replayed,
    with the cache flush (when on) between replays, outside the graph.  Kernel arguments
    are fixed at capture, so every replay repeats the same step."""
    import numpy as np
    import torch

    def capture(fn):
        fn()                                     # warm-up outside the capture
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn()
        torch.cuda.synchronize()
        return g

    def full_step():
        fx.fx_build_summaries(plan, inp.K, inp.seq_lens, -1, INT32_MAX, A.summaries)
        fx.fx_select_delta(plan, q, A.summaries, logits, mask, inp.seq_lens, Bsel.sel_idx,
                           Bsel.sel_cnt, A.sel_idx, A.sel_cnt, A.added, A.added_cnt, A.removed,
                           A.removed_cnt, A.workspace)
        fx.fx_sparse_decode(plan, q, inp.K, inp.V, inp.seq_lens, A.sel_idx, A.sel_cnt, scale,
                            A.out, A.lse, A.workspace)

    def select_decode():
        fx.fx_select(plan, q, A.summaries, logits, mask, inp.seq_lens, A.sel_idx, A.sel_cnt,
                     A.workspace)
        fx.fx_sparse_decode(plan, q, inp.K, inp.V, inp.seq_lens, A.sel_idx, A.sel_cnt, scale,
                            A.out, A.lse, A.workspace)

    res = {}
    for key, fn in (("step", full_step), ("select_decode", select_decode)):
        g = capture(fn)
        times = []
        for i in range(reps + 3):
            if flush_buf is not None:
                flush_buf.fill_(i & 0xFF)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            g.replay()
            e1.record()
            torch.cuda.synchronize()
            if i >= 3:
                times.append(e0.elapsed_time(e1))
        res[key + "_us_median"] = round(float(np.median(times)) * 1e3, 2)
        del g
    if fx.fx_read_error(plan) != 0:
        raise SystemExit("device error word set during the graph replays")
    return res


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="mixed_serving")
    ap.add_argument("--split", type=int, default=0, help="minimum decode segment (tokens), 0 = plan default")
    ap.add_argument("--grow", action="store_true",
                    help="decode loop: append one token to every sequence before each step "
                         "(outside the timed events; t_cap grows by the number of steps)")
    ap.add_argument("--no-flush", action="store_true",
                    help="skip the 1 GiB overwrite between steps (outside the timed events) "
                         "that keeps the 256 MB Infinity Cache from holding the previous step")
    ap.add_argument("--ed", action="store_true",
                    help="attention adds each NOSA block's eviction logit to its tokens' logits "
                         "(fx_sparse_decode_ed)")
    ap.add_argument("--pooling", choices=["key", "score_sum", "score_max"], default="key",
                    help="where the block max of the two-stage pooling acts: over key vectors "
                         "(one summary row per block) or over the scores of the sub-block means")
    ap.add_argument("--compact", action="store_true",
                    help="after the delta, keep the selected full blocks in a block-slot working "
                         "set (fx_compact_update), timed as its own phase")
    ap.add_argument("--separate-delta", action="store_true",
                    help="fx_select then fx_selection_delta instead of fx_select_delta")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="CPU time (summed over the workers) the oracle baseline runs for")
    ap.add_argument("--cpu-workers", type=int, default=16,
                    help="most oracle worker processes (the pool takes min(this, usable cores))")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-reference", action="store_true",
                    help="after timing, run one plain 1 GiB device copy (scales HBM counters)")
    ap.add_argument("--graph", action="store_true",
                    help="also time the step, and fx_select + fx_sparse_decode, replayed from a "
                         "captured HIP graph (launches without the host in between)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py: the benchmark runs on exactly one GPU (asked for --gpus {args.gpus}); "
              f"units (sequence, kv head) are independent, so each GPU would run the same calls "
              f"on its own share of sequences or kv heads with no exchange",
              file=sys.stderr)
        return 2

    # The oracle's worker processes start before this process touches the GPU.
    pool = None
    if not args.no_cpu_baseline:
        pool = OraclePool(min(len(os.sched_getaffinity(0)), args.cpu_workers))
    try:
        return run(args, pool)
    finally:
        if pool is not None:
            pool.close()


def run(args, pool) -> int:
    import numpy as np
    import torch

    import block_sparse_decode_summary_amd as fx
    from workloads import WORKLOAD_NAMES, append_tokens, generate, get_workload, query_at_step

    if args.workload not in WORKLOAD_NAMES:
        raise SystemExit(f"unknown workload {args.workload}; one of {WORKLOAD_NAMES}")
    w = get_workload(args.workload)
    pooling = {"key": fx.FX_POOL_KEY, "score_sum": fx.FX_POOL_SCORE_SUM,
               "score_max": fx.FX_POOL_SCORE_MAX}[args.pooling]
    w = w.replace(pooling=pooling)
    if args.grow:
        w = w.replace(t_cap=w.t_cap + args.warmup + args.steps)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    t0 = time.time()
    inp = generate(w, dev)
    torch.cuda.synchronize()
    log(f"[bench] {w.name}: inputs generated in {time.time() - t0:.1f} s "
        f"(K+V {2 * inp.K.numel() * inp.K.element_size() / 1e9:.1f} GB)")

    dt = fx.FX_F32 if w.dtype == "f32" else fx.FX_BF16
    plan = fx.fx_plan_create(w.batch, w.num_q_heads, w.num_kv_heads, w.head_dim, w.t_cap, dt,
                             list(w.policies), args.split, pooling)
    A = fx.allocate_step_buffers(plan, dev)
    Bsel = fx.allocate_step_buffers(plan, dev)     # second selection buffer for the delta
    scale = 1.0 / math.sqrt(w.head_dim)
    qs = [query_at_step(w, t, dev) for t in range(w.steps)] if w.drift else [inp.q]
    logits = inp.logits
    mask = A.evicted_mask if w.has_nosa else None
    fx.fx_build_summaries(plan, inp.K, inp.seq_lens, 0, INT32_MAX, A.summaries)   # prefill
    flush_buf = None if args.no_flush else torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    wset = fx.allocate_working_set(plan, dev) if args.compact else None

    cur, prev = A, Bsel
    lens = list(w.seq_lens)

    # Events between the kernels of a step delay the next dispatch by a few microseconds,
    # so the timed loop records events only at step boundaries.  Phase times come from
    # separate loops over the same steps, each with events only around what it measures.
    plain_select = False      # True: fx_select and fx_selection_delta as two calls

    def step(i, ev=None):
        """One step; ev maps marks ("b1" after the build, "d0" / "d1" around the decode,
        "c0" / "c1" around the compaction) to per-step event lists."""
        nonlocal cur, prev
        ev = ev or {}
        mark = lambda k: ev[k][i].record() if k in ev else None
        q = qs[i % len(qs)]
        fx.fx_build_summaries(plan, inp.K, inp.seq_lens, -1, INT32_MAX, A.summaries)
        mark("b1")
        fused = not args.separate_delta and not plain_select
        if fused:
            fx.fx_select_delta(plan, q, A.summaries, logits, mask, inp.seq_lens, prev.sel_idx,
                               prev.sel_cnt, cur.sel_idx, cur.sel_cnt, A.added, A.added_cnt,
                               A.removed, A.removed_cnt, A.workspace)
        else:
            fx.fx_select(plan, q, A.summaries, logits, mask, inp.seq_lens, cur.sel_idx,
                         cur.sel_cnt, A.workspace)
        mark("d0")
        if args.ed:
            fx.fx_sparse_decode_ed(plan, q, inp.K, inp.V, inp.seq_lens, cur.sel_idx, cur.sel_cnt,
                                   logits, scale, A.out, A.lse, A.workspace)
        else:
            fx.fx_sparse_decode(plan, q, inp.K, inp.V, inp.seq_lens, cur.sel_idx, cur.sel_cnt,
                                scale, A.out, A.lse, A.workspace)
        mark("d1")
        if not fused:
            fx.fx_selection_delta(plan, prev.sel_idx, prev.sel_cnt, cur.sel_idx, cur.sel_cnt,
                                  A.added, A.added_cnt, A.removed, A.removed_cnt)
        if wset is not None:
            mark("c0")
            fx.fx_compact_update(plan, inp.K, inp.V, inp.seq_lens, cur.sel_idx, cur.sel_cnt, wset,
                                 A.workspace)
            mark("c1")
            hist_moved[i].copy_(wset.moved_cnt)
        cur, prev = prev, cur

    n_ev = args.warmup + args.steps
    mk = lambda: [torch.cuda.Event(enable_timing=True) for _ in range(n_ev)]
    ev_s0, ev_s1 = mk(), mk()
    hist_moved = torch.zeros(n_ev, w.num_units, dtype=torch.int32, device=dev) if args.compact else None
    # Per-step selection statistics of multi-step (drifting query) workloads, copied out
    # after each step's end event.
    multi = len(qs) > 1
    if multi:
        hist_cnt = torch.zeros(n_ev, w.num_units, dtype=torch.int32, device=dev)
        hist_add = torch.zeros_like(hist_cnt)
        hist_rem = torch.zeros_like(hist_cnt)
    for i in range(args.warmup):
        if args.grow:
            lens = append_tokens(inp, lens, i + 1)
        ev_s0[i].record()
        step(i)
        ev_s1[i].record()
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    for i in range(args.warmup, n_ev):
        if args.grow:
            lens = append_tokens(inp, lens, i + 1)
        if flush_buf is not None:
            flush_buf.fill_(i & 0xFF)
        ev_s0[i].record()
        step(i)
        ev_s1[i].record()
        if multi:
            hist_cnt[i].copy_(prev.sel_cnt)      # prev: this step's selection after the swap
            hist_add[i].copy_(A.added_cnt)
            hist_rem[i].copy_(A.removed_cnt)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    timed = range(args.warmup, n_ev)
    moved_main = hist_moved.clone() if args.compact else None   # the later loops overwrite it
    step_ms = [ev_s0[i].elapsed_time(ev_s1[i]) for i in timed]
    ms_per_step = float(np.median(step_ms))
    ms_per_step_mean = float(np.mean(step_ms))

    def marked_loop(marks, separate=False):
        """The timed steps again (no token appends), with events at the given marks;
        separate: fx_select and fx_selection_delta as two calls."""
        nonlocal plain_select
        plain_select = separate
        ev = {k: mk() for k in marks}
        for i in timed:
            if flush_buf is not None:
                flush_buf.fill_(i & 0xFF)
            ev_s0[i].record()
            step(i, ev)
            ev_s1[i].record()
        torch.cuda.synchronize()
        plain_select = False
        return ev

    ev = marked_loop(["d0", "d1"])
    dec_ms = [ev["d0"][i].elapsed_time(ev["d1"][i]) for i in timed]
    dec_avg = float(np.mean(dec_ms))
    ev = marked_loop(["b1", "d1"], separate=True)     # fx_select + fx_sparse_decode alone
    sd_ms = [ev["b1"][i].elapsed_time(ev["d1"][i]) for i in timed]
    pm = ["b1", "d0", "d1"] + (["c0", "c1"] if args.compact else [])
    ev = marked_loop(pm, separate=True)
    phases = {
        "build": [ev_s0[i].elapsed_time(ev["b1"][i]) for i in timed],
        "select": [ev["b1"][i].elapsed_time(ev["d0"][i]) for i in timed],
        "decode": [ev["d0"][i].elapsed_time(ev["d1"][i]) for i in timed],
        "delta": [ev["d1"][i].elapsed_time(ev["c0"][i] if args.compact else ev_s1[i])
                  for i in timed],
    }
    if args.compact:
        phases["compact"] = [ev["c0"][i].elapsed_time(ev["c1"][i]) for i in timed]
    ev_c0, ev_c1 = (ev["c0"], ev["c1"]) if args.compact else (None, None)
    if fx.fx_read_error(plan) != 0:
        raise SystemExit("device error word set during the benchmark")

    # Attainable-bandwidth reference: a plain streaming read of 2 GiB of the K cache.
    ref_bytes = min(2 << 30, inp.K.numel() * inp.K.element_size()) // 16 * 16
    ref_src = inp.K.view(torch.uint8).reshape(-1)[:ref_bytes]
    sink = torch.empty(fx.load_library().fx_stream_read_sink_words(ref_bytes), dtype=torch.int32,
                       device=dev)
    for _ in range(2):
        fx.fx_stream_read(ref_src, sink)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ref_ms = []
    for _ in range(5):
        if flush_buf is not None:
            flush_buf.fill_(1)
        e0.record()
        fx.fx_stream_read(ref_src, sink)
        e1.record()
        torch.cuda.synchronize()
        ref_ms.append(e0.elapsed_time(e1))
    stream_gbs = ref_bytes / (float(np.median(ref_ms)) * 1e-3) / 1e9

    drift = None
    if multi:
        c = hist_cnt[args.warmup:].cpu().numpy().astype(np.float64)
        a = hist_add[args.warmup:].cpu().numpy().astype(np.float64)
        r = hist_rem[args.warmup:].cpu().numpy().astype(np.float64)
        with np.errstate(invalid="ignore", divide="ignore"):
            gamma = np.where(c > 0, (c - a) / c, 1.0)
        drift = {"added_mean": round(float(a.mean()), 3), "added_max": int(a.max()),
                 "removed_mean": round(float(r.mean()), 3), "removed_max": int(r.max()),
                 "locality_min": round(float(gamma.min()), 4),
                 "steps_per_query_cycle": len(qs)}

    graph = None
    if args.graph:
        graph = graph_replay(fx, plan, w, inp, A, Bsel, qs[0], logits, mask, scale, flush_buf,
                             args.steps)
        log(f"[bench] graph replay: {graph}")

    if args.copy_reference:
        src = torch.ones(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    sel_idx = prev.sel_idx.cpu().numpy()      # the last step's selection
    sel_cnt = prev.sel_cnt.cpu().numpy()
    w_last = w.replace(seq_lens=tuple(lens))      # the lengths of the last timed step
    compact = None
    if args.compact:
        # Per step: each moved block's g key and value rows read and written, plus the slot
        # rows read and written and the selection read by the planning kernel.
        mv = moved_main[args.warmup:].cpu().numpy().astype(np.int64)
        blk = np.array([2 * 2 * p.block * w.head_dim * w.elem_bytes for p in w.policies])
        moved_bytes = (mv * blk[None, :]).sum(axis=1) + 3 * w.num_units * plan.max_selected * 4
        c_ms = np.array([ev_c0[i].elapsed_time(ev_c1[i]) for i in timed])
        compact = {"us_median": round(float(np.median(c_ms)) * 1e3, 2),
                   "moved_blocks_per_step_mean": round(float(mv.sum(axis=1).mean()), 1),
                   "moved_blocks_per_unit_max": int(mv.max()),
                   "alg_bytes_per_step_mean": int(moved_bytes.mean()),
                   "achieved": round(float((moved_bytes / (c_ms * 1e-3)).mean() / 1e9), 1),
                   "unit": "GB/s"}
        log(f"[bench] compaction: {compact}")
    total_b, dec_b, sd_b, parts = algorithmic_bytes(w_last, plan.max_selected, sel_idx, sel_cnt,
                                                    ed=args.ed)
    if compact:
        parts["compaction"] = compact["alg_bytes_per_step_mean"]
        total_b += compact["alg_bytes_per_step_mean"]
    value = total_b / (ms_per_step * 1e-3) / 1e9
    achieved = dec_b / (dec_avg * 1e-3) / 1e9
    sd_med = float(np.median(sd_ms))
    sd_gbs = sd_b / (sd_med * 1e-3) / 1e9
    log(f"[bench] {w.name}: {ms_per_step * 1e3:.1f} us/step (p10 {np.percentile(step_ms, 10) * 1e3:.1f},"
        f" p90 {np.percentile(step_ms, 90) * 1e3:.1f}), decode {dec_avg * 1e3:.1f} us; "
        f"{total_b / 1e6:.1f} MB/step -> {value:.0f} GB/s ({100 * value / HBM_PEAK_GBS:.1f}% of peak); "
        f"decode {achieved:.0f} GB/s; wall {wall / args.steps * 1e3:.3f} ms/step")
    log(f"[bench] bytes/step: " + ", ".join(f"{k} {v / 1e6:.2f} MB" for k, v in parts.items()))
    log(f"[bench] phase medians (us): " + ", ".join(
        f"{k} {float(np.median(v)) * 1e3:.1f}" for k, v in phases.items())
        + f"; select+decode {sd_gbs:.0f} GB/s; streaming-read reference {stream_gbs:.0f} GB/s")
    if drift:
        log(f"[bench] selection drift: {drift}")

    cpu = None
    if not args.no_cpu_baseline:
        log(f"[bench] timing the CPU oracle on a sample (~{args.cpu_seconds:.0f} s)")
        cpu = cpu_baseline(pool, w, inp, args.cpu_seconds, ed=args.ed)
        log(f"[bench] oracle: {cpu['value']:.4f} GB/s ({cpu['sample']})")

    shapes = {
        "workload": w.name, "batch": w.batch, "q_heads": w.num_q_heads, "kv_heads": w.num_kv_heads,
        "head_dim": w.head_dim, "t_cap": w.t_cap,
        "seq_lens": "U{8192..131072}" if w.name == "mixed_serving" else w.seq_lens[0],
        "blocks": sorted({p.block for p in w.policies}), "split_tokens": plan.split_tokens,
        "cache_flush_between_steps": not args.no_flush,
        "decode_loop_growth": bool(args.grow),
        "eviction_logit_in_attention": bool(args.ed),
        "pooling": args.pooling,
    }
    line = {
        "metric": METRIC, "value": round(value, 2), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5),
        "ms_per_step_mean": round(ms_per_step_mean, 5),
        "us_per_step": round(ms_per_step * 1e3, 2),
        "step_us_p10_p50_p90": [round(float(np.percentile(step_ms, p)) * 1e3, 2) for p in (10, 50, 90)],
        "frac_of_hbm_peak": round(value / HBM_PEAK_GBS, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": w.dtype,
        "data": "synthetic (seeded; shapes and value distributions of the workload definition)",
        "config": shapes,
        "alg_bytes_per_step": int(total_b),
        "roofline": {"bound": "hbm",
                     "kernel": ("fx_sparse_decode_ed" if args.ed else "fx_sparse_decode")
                     + " (k_decode + k_combine)",
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": None if args.ed else measured_traffic(w.name),
                     "alg_bytes_per_launch": int(dec_b), "avg_launch_us": round(dec_avg * 1e3, 2),
                     "k_decode_sha256_16": decode_source_hash()},
        "cpu_baseline": cpu,
        "select_decode": {"us_median": round(sd_med * 1e3, 2), "alg_bytes": int(sd_b),
                          "achieved": round(sd_gbs, 1), "unit": "GB/s",
                          "frac": round(sd_gbs / HBM_PEAK_GBS, 4)},
        "phases_us_median": {k: round(float(np.median(v)) * 1e3, 2) for k, v in phases.items()},
        "stream_read_reference": {"achieved": round(stream_gbs, 1), "unit": "GB/s",
                                  "bytes": int(ref_bytes)},
    }
    if drift:
        line["selection_drift"] = drift
    if graph:
        line["graph_replay"] = graph
    if compact:
        line["compaction"] = compact
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
