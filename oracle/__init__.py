"""CPU oracle for bucketed gradient synchronisation (plain Python + NumPy).

TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check in
``__graft_entry__`` and the bench's ``cpu_baseline`` leg may import this
package. The product path (``ddp_bucketed_gradient_amd``) never imports it and
shares no code, table or constant with it.

It is written from the method as these pages describe it:

* [Li] "PyTorch Distributed: Experiences on Accelerating Data Parallel
  Training" (paper-graph-ui summary of arXiv 2006.15704), §3.4 subsections
  "Gradient Bucketing", "Overlapping Computation with Communication",
  "Gradient Accumulation (no_sync)", and the correctness discussion.
* [TP] "Distributed Data Parallel" (tensorplay.cn notes), sections "Example",
  "Internal Design", "When a parameter never receives a gradient",
  "Gradient sync you can turn off".
* [C30] "NCCL 专家课程 30：DDP Reducer、Bucket 与计算通信重叠" (blog.cptz.space),
  sections "Variable 到 Bucket", "Bucket 必须按序发起", "bucket_cap_mb 不是张量切分器",
  "参数粒度实验", "从 Bucket 到 AllReduce Future", "未检测的失败".
* [PDTI] "PyTorch Distributed Training Internals" (sandeep007734.github.io),
  §2 "What DDP Does at Construction", §3 "The All-Reduce Itself".

Modules:
  plan      -- bucket assignment under the cap and the variable locator
  reducer   -- readiness state machine, pack, fixed-order mean, copy-back,
               finalize, no_sync accumulation
  linear10  -- the nn.Linear(10, 10) example in closed form

Pins (all in ``tests/test_oracle_*.py``): the pages' printed layouts, the
sequence of the in-order launch example, closed forms, exact rational means on
dyadic inputs, error bounds, brute force over permutations, and planted-mistake
checks. No function here is "parity unpinned".
"""
from . import plan, reducer, linear10  # noqa: F401
