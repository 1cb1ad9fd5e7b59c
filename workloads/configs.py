"""The five workloads: shapes, replica count R, bucket cap and hook order.

Workload definitions only; nothing here plans buckets or reduces anything.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Callable, List

from . import shapes as S

MiB = S.MiB
DEFAULT_CAP = 25 * MiB          # bucket_cap_mb = 25, read as MiB
CAP_SWEEP_MIB = [0, 1, 5, 10, 25, 50, 100, 200]   # 0 = one bucket per tensor


@dataclass(frozen=True)
class Workload:
    cfg: int                      # seed namespace
    name: str
    params: Callable[[], List[S.Param]]
    R: int
    cap_bytes: int = DEFAULT_CAP
    micro_steps: int = 1          # k local steps (no_sync) before one sync
    step_dtype: str = "f32"       # dtype of the per-micro-step gradients
    note: str = ""

    def numels(self) -> List[int]:
        return S.numels(self.params())

    def ready_order(self) -> List[int]:
        """Hooks fire last-defined parameter first (reverse index)."""
        return list(range(len(self.params())))[::-1]


LINEAR10 = Workload(1, "linear10_r2", S.linear10, R=2,
                    note="nn.Linear(10,10), 20x10 batch per rank, loss mean(out^2)")
RESNET50 = Workload(2, "resnet50_r8", S.resnet50, R=8)
BERT_LARGE = Workload(3, "bert_large_r8_cap25", S.bert_large, R=8)
BERT_BASE_NOSYNC = Workload(4, "bert_base_r16_nosync_k8", S.bert_base, R=16,
                            micro_steps=8, step_dtype="bf16")
# the blog's 48 MiB payload per rank on 4 ranks, as 12 x 4 MiB or 48 x 1 MiB parameters
BLOG_COARSE4 = Workload(6, "blog48mib_12x4mib_r4", S.blog_coarse4, R=4, cap_bytes=4 * MiB)
BLOG_FINE1 = Workload(6, "blog48mib_48x1mib_r4", S.blog_fine1, R=4, cap_bytes=4 * MiB)
MLP_OVERLAP = Workload(5, "mlp24_d2048_f8192_r8_overlap", S.mlp, R=8,
                       note="bf16 backward GEMMs over 8192 tokens on the compute stream")

ALL = {w.cfg: w for w in (LINEAR10, RESNET50, BERT_LARGE, BERT_BASE_NOSYNC, MLP_OVERLAP)}


def bert_large_cap(cap_mib: int) -> Workload:
    return Workload(3, f"bert_large_r8_cap{cap_mib}", S.bert_large, R=8, cap_bytes=cap_mib * MiB)
