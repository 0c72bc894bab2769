"""Seeded synthetic workloads for block-sparse decode attention.

This package only describes shapes and draws inputs. It holds none of the
method's arithmetic (no pooling, scoring, selection or attention): the HIP
library and the CPU oracle both receive exactly the tensors built here.

Workloads follow five benchmark shapes:

  tiny            1 seq, 4 q / 2 kv heads, d 64, fp32, context 2048, block 32
  llama8b_layer   1 seq, 32 / 8, d 128, bf16, context 32768, block 64,
                  kv heads 0-3 streaming (sink 64 + local 1024), 4-7 retrieval 5 %
  qwen7b_layer    4 seqs, 28 / 4 (GQA 7), d 128, bf16, context 131072,
                  per-kv-head block in {16,32,64,128}, budget U[2 %, 10 %]
  nosa_drift      32 seqs, 32 / 8, d 128, bf16, context 16384, block 64 / sub 16,
                  query-aware top-16 + eviction top-48, 64 steps of query drift
  mixed_serving   64 seqs of length U{8192..131072}, 32 / 8, d 128, bf16, block 64,
                  per-kv-head streaming/retrieval coin flip, budget U[2 %, 10 %]
"""
from .configs import (HeadPolicy, Workload, get_workload, small_workload,
                      WORKLOAD_NAMES, MODE_RETRIEVAL, MODE_STREAMING, MODE_NOSA)
from .generate import Inputs, append_tokens, generate, query_at_step, unit_arrays

__all__ = [
    "HeadPolicy", "Workload", "get_workload", "small_workload", "WORKLOAD_NAMES",
    "MODE_RETRIEVAL", "MODE_STREAMING", "MODE_NOSA",
    "Inputs", "append_tokens", "generate", "query_at_step", "unit_arrays",
]
