"""CPU oracle for block-sparse decode attention -- TEST INFRASTRUCTURE ONLY.

This package is a plain, slow, float64 NumPy statement of what the hot path
computes.  It exists to check the HIP library.  Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it; the product path never does, and it shares no code with the HIP
sources (its only common dependency is the seeded input generator in
``workloads/``, which holds none of the method's arithmetic).

Sources, cited by page title and section:

  [Fluxion-NL]  "Technische Samenvatting: Fluxion"
                (gist.science/nl/paper/2605.07719)
  [NOSA-DE]     "Technisches Resümee: NOSA: Native und Offloadable Sparse Attention"
                (gist.science/de/paper/2510.13602)
  [Fluxion-KO]  "An Efficient Hybrid Sparse Attention with CPU-GPU Parallelism for
                Long-Context Inference" (gist.science/ko/paper/2605.07719)

The pages give the method in prose only (no equations, listings or worked
numbers).  Where they leave a step open, each module states the reading it
takes.  Every function here is pinned by a CPU test in tests/test_oracle_*.py
against closed forms, brute force, exact rational arithmetic or library
routines; none is "parity unpinned".

Modules
  numerics   float64 -> bfloat16 / float32 rounding (round to nearest, ties to even)
  pooling    two-stage block summaries (mean over sub-blocks, max over the block), or
             the sub-block means alone for score-side pooling
  scoring    block scores against the GQA query group (key-side or score-side pooling)
  selection  forced sets, top-k per kv head, NOSA eviction selection
  attention  attention over the selected tokens; split-K partial merge
  delta      selection set differences and locality
  compaction the selected full blocks kept in a block-slot working set (moves by set
             difference)
  step       one decode step for one unit / a whole workload
"""
