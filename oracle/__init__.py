"""Plain fp64 CPU oracle for the vertical-slash (VS) sparse attention path.

TEST INFRASTRUCTURE ONLY. Nothing on the product path imports this package:
only the tests, the smoke check and the CPU-baseline leg of the benchmark use
it. It shares no code with the HIP library; both sides consume the same seeded
inputs from ``synth``.

Sources are the MTraining review page (xllm-io paper-review, "MTraining:
分布式动态稀疏注意力高效超长上下文训练") and the Ring Attention overview page
(intelliparadigm, "Ring Attention：突破长序列训练的分布式架构"). Each function
names the section it follows.

Modules:
  layout    -- shard maps (contiguous / striped / zigzag) and ring order
  index     -- online sparse-index approximation: row statistics, vertical and
               slash attention mass, top-p budget selection
  mask      -- the active set M and the per-query-block tile / vertical lists
  attention -- masked softmax attention forward, log-sum-exp merge, backward

Every function here has at least one pin in tests/test_oracle_*.py against
something other than itself (closed forms, brute force, library routines,
finite differences, planted structure); none is "parity unpinned".
"""
