"""CPU oracle for the ragged step compile, the paged K/V write and the
hidden-state gather.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, links or runs
anything in this package: only the tests, the smoke check and the benchmark's
CPU-baseline leg do.  It shares no code, headers, tables or constants with the
HIP library; the two meet only at the seeded input generators (``workloads``),
which draw inputs and hold none of the method's arithmetic.

Sources (web pages; cited by title and section):

* [P1] "vLLM 源码完全拆解（五）：GPUModelRunner 如何把动态请求拼成一次 GPU 前向"
  (pinghaoyang.com.cn)
* [P2] "第8章 ModelRunner：从 SchedulerOutput 到 GPU Kernel" (yangyitao.com)
* [P3] "变长批处理与一次混合前向" (anrans.github.io, inference-engine handbook)
* [P4] "04 · 模型执行与 CUDA Graph" (ai-reference-codex)
* [P5] "Nano-VLLM全代码解析笔记(4)-model_runner" (lbrq.cn)

Modules:

* ``step``        per-token Python loops: the plain definition (P1, P3), and
                  the routines of the next rows (kernel-block expansion, padded
                  tables, per-group slots, sampled-token append, the correction
                  of optimistic computed counts, speculative-decoding indices).
* ``vectorised``  the same outputs from numpy library routines
                  (cumsum / repeat / take), as P2 section 8.3 describes them.
* ``batch``       the persistent row-compacted batch: add, remove, append,
                  replace and condense (P1, P2 section 8.2).
* ``nano_oracle.c`` plain C, the nano-vllm block-range slot loop (P5) and a
                  row-by-row K/V scatter; loaded through ``cbind``.

Pinning: every function is checked in ``tests/test_oracle_*.py`` against
values the pages print (``tests/golden``), closed forms, invariants and brute
force.  One part is "parity unpinned": the content of the reserved null block
after padded tokens write to it (several pad tokens write the same slot; the
pages leave the winner open), so it is excluded from every comparison.  The pad
tail values of the per-token outputs (0, 0, -1, null slot) and of the
per-request outputs are fixed by this package's own reading, not by the pages.
"""
