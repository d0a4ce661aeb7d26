"""CPU oracle for one RoundPipe GPU-worker stage -- TEST INFRASTRUCTURE ONLY.

This package is the slow, plain, obviously-correct CPU statement of what an
offloaded pipeline stage computes. It exists to check the HIP path; the
product never imports, calls or links it. Only the test suite, the smoke
entry point and the benchmark's CPU-baseline leg may use it.

Sources (the RoundPipe paper, "Efficient Training on Multiple Consumer GPUs
with RoundPipe", as published on paperpeel.com, plus the paperlayer.ai
summary of its appendices):

* ``oracle.stage``  -- the decoder-layer / LM-head math of a stage: forward
  written out operation by operation in torch CPU tensors (fp64 by default),
  gradients as the exact derivative of that forward (torch autograd used as a
  library primitive). The paper changes where and when a layer runs, never what
  it computes (section 3.2, asymmetric stage splitting; section 2.1.1,
  recomputation re-executes the same forward).
* ``oracle.sched``  -- the host-side algorithms: RoundPipe's bubble formula and a
  brute-force schedule simulator (section 3.3), the partition objective and
  the O(L^3) greedy partitioner with an exhaustive-search cross-check
  (section 4.4), longest-processing-time-first window packing (section 4.2.2),
  and the per-layer activation-memory model (appendix B.1).

Readings of points the pages leave open are listed in each function's
docstring. Every function here is pinned by a CPU test to something other than
itself (finite differences, closed forms, textbook/library special cases,
brute force); none is "parity unpinned".
"""
