"""Oracle for the decode-step mega-kernel.

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import, call or
execute anything in this package: only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` use it.

Two independent parts, written from the MPK paper summary ("MPK: A Compiler
and Runtime for Mega-Kernelizing Tensor Programs", L2 notes) and the
author's HN comments on "Compiling LLMs into a MegaKernel":

* ``oracle.numerics`` -- a plain CPU decoder forward (numpy) of one decode
  step of a Qwen3-shaped transformer over a paged KV cache.  It is the
  definition of what the hot path computes, written out without blocking,
  fusion or reordering.
* ``oracle.tgraph`` -- the canonical task/event-graph spec (decomposition,
  overlap dependencies, event fusion Def 4.1 / Def 4.2, normalisation,
  BFS linearisation, JIT/AOT classification) in plain Python, plus
  brute-force semantic checks that do not depend on the spec.

The two share no code with the HIP path (``task_graph_runtime_amd``) and
neither imports it.
"""
