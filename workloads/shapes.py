"""Parameter shape lists, in definition (``Model.parameters()``) order, for the
synthetic gradient sets used by the tests and the bench.

This module holds workload *definitions* only: names, shapes and element
counts. It does no arithmetic of the bucketing method.

The gradient sets stand in for the models the pages evaluate (ResNet50 and BERT
in "PyTorch Distributed: Experiences on Accelerating Data Parallel Training",
§5 Evaluation; the nn.Linear(10, 10) example in the tensorplay "Distributed Data
Parallel" notes, section "Example"; the 48 MiB payload of the blog "NCCL 专家课程
30: DDP Reducer, Bucket 与计算通信重叠", table in "参数粒度实验"). The pages do not
list the parameter order of ResNet50 or BERT; the order used here is the order
in which the standard architectures register their parameters.
"""
from __future__ import annotations

from dataclasses import dataclass
from math import prod
from typing import List, Tuple

MiB = 1 << 20


@dataclass(frozen=True)
class Param:
    name: str
    shape: Tuple[int, ...]

    @property
    def numel(self) -> int:
        return int(prod(self.shape)) if self.shape else 1


def numels(params: List[Param]) -> List[int]:
    return [p.numel for p in params]


def shapes(params: List[Param]) -> List[Tuple[int, ...]]:
    return [p.shape for p in params]


def linear10() -> List[Param]:
    """nn.Linear(10, 10): weight [out, in] then bias."""
    return [Param("weight", (10, 10)), Param("bias", (10,))]


def resnet50(num_classes: int = 1000) -> List[Param]:
    """ResNet-50 (bottleneck blocks [3, 4, 6, 3], widths 64/128/256/512,
    expansion 4). 161 tensors, 25,557,032 parameters."""
    ps: List[Param] = [Param("conv1.weight", (64, 3, 7, 7)),
                       Param("bn1.weight", (64,)), Param("bn1.bias", (64,))]
    in_ch = 64
    for si, (blocks, width) in enumerate([(3, 64), (4, 128), (6, 256), (3, 512)]):
        out_ch = width * 4
        for bi in range(blocks):
            pre = f"layer{si + 1}.{bi}."
            ps.append(Param(pre + "conv1.weight", (width, in_ch, 1, 1)))
            ps += [Param(pre + "bn1.weight", (width,)), Param(pre + "bn1.bias", (width,))]
            ps.append(Param(pre + "conv2.weight", (width, width, 3, 3)))
            ps += [Param(pre + "bn2.weight", (width,)), Param(pre + "bn2.bias", (width,))]
            ps.append(Param(pre + "conv3.weight", (out_ch, width, 1, 1)))
            ps += [Param(pre + "bn3.weight", (out_ch,)), Param(pre + "bn3.bias", (out_ch,))]
            if bi == 0:
                ps.append(Param(pre + "downsample.0.weight", (out_ch, in_ch, 1, 1)))
                ps += [Param(pre + "downsample.1.weight", (out_ch,)),
                       Param(pre + "downsample.1.bias", (out_ch,))]
            in_ch = out_ch
    ps += [Param("fc.weight", (num_classes, 2048)), Param("fc.bias", (num_classes,))]
    return ps


def bert(layers: int, hidden: int, ffn: int, vocab: int = 30522,
         max_pos: int = 512, type_vocab: int = 2) -> List[Param]:
    """BERT encoder with pooler, no pre-training heads. Linear weights are
    [out, in]."""
    h, f = hidden, ffn
    ps = [Param("embeddings.word_embeddings.weight", (vocab, h)),
          Param("embeddings.position_embeddings.weight", (max_pos, h)),
          Param("embeddings.token_type_embeddings.weight", (type_vocab, h)),
          Param("embeddings.LayerNorm.weight", (h,)),
          Param("embeddings.LayerNorm.bias", (h,))]
    for i in range(layers):
        pre = f"encoder.layer.{i}."
        for nm in ("query", "key", "value"):
            ps += [Param(pre + f"attention.self.{nm}.weight", (h, h)),
                   Param(pre + f"attention.self.{nm}.bias", (h,))]
        ps += [Param(pre + "attention.output.dense.weight", (h, h)),
               Param(pre + "attention.output.dense.bias", (h,)),
               Param(pre + "attention.output.LayerNorm.weight", (h,)),
               Param(pre + "attention.output.LayerNorm.bias", (h,)),
               Param(pre + "intermediate.dense.weight", (f, h)),
               Param(pre + "intermediate.dense.bias", (f,)),
               Param(pre + "output.dense.weight", (h, f)),
               Param(pre + "output.dense.bias", (h,)),
               Param(pre + "output.LayerNorm.weight", (h,)),
               Param(pre + "output.LayerNorm.bias", (h,))]
    ps += [Param("pooler.dense.weight", (h, h)), Param("pooler.dense.bias", (h,))]
    return ps


def bert_large() -> List[Param]:
    """24 layers, hidden 1024, FFN 4096: 391 tensors, 335,141,888 parameters."""
    return bert(24, 1024, 4096)


def bert_base() -> List[Param]:
    """12 layers, hidden 768, FFN 3072: 199 tensors, 109,482,240 parameters."""
    return bert(12, 768, 3072)


def mlp(layers: int = 24, d: int = 2048, ffn: int = 8192) -> List[Param]:
    """Stack of [Linear(d, ffn), Linear(ffn, d)] blocks with biases:
    fc1.weight [ffn, d], fc1.bias [ffn], fc2.weight [d, ffn], fc2.bias [d]."""
    ps: List[Param] = []
    for i in range(layers):
        pre = f"layers.{i}."
        ps += [Param(pre + "fc1.weight", (ffn, d)), Param(pre + "fc1.bias", (ffn,)),
               Param(pre + "fc2.weight", (d, ffn)), Param(pre + "fc2.bias", (d,))]
    return ps


def blog_fine1() -> List[Param]:
    """48 independent 1 MiB fp32 parameters (48 MiB payload)."""
    return [Param(f"p{i}", (MiB // 4,)) for i in range(48)]


def blog_coarse4() -> List[Param]:
    """12 independent 4 MiB fp32 parameters (48 MiB payload)."""
    return [Param(f"p{i}", (MiB,)) for i in range(12)]
