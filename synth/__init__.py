"""Seeded synthetic inputs shared by the tests, the bench and the oracle checks.

This module holds NO arithmetic of the attention method: it only draws random tensors of the
shapes the workloads use.  Q, K and V are N(0, 1) (unit variance, the stated input
distribution of every workload), gate values are sigmoid(N(0, 1)) in (0, 1).  The gates'
sigmoid belongs to the gate projection that sits upstream of the operator, not to it.

The permutation sigma is NOT drawn here: it is a step of the method, implemented on each side
from the published generator (splitmix64 + Fisher-Yates); ``sigma_seed`` only fixes the seed.
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Tuple

import torch


@dataclass(frozen=True)
class Workload:
    """One synthetic workload: an attention-layer shape plus the paths to run on it."""
    name: str
    index: int          # 1-based position in the workload table (used in seeds)
    B: int
    n: int
    Hq: int
    Hkv: int
    d: int
    dtype: str          # "f32" | "bf16"
    windows: Tuple[int, ...]
    layers: int
    paths: Tuple[str, ...]  # subset of {"sa", "swa", "gated"}
    causal_modes: Tuple[bool, ...] = (True,)


# The five layer shapes: a tiny parity case, then attention layers shaped like the models the
# pages evaluate (a 360M pretraining model, Qwen3-8B, Qwen3-30B-A3B) at their windows.
WORKLOADS: List[Workload] = [
    Workload("tiny-sa-n256-d64-w16-f32", 1, 1, 256, 1, 1, 64, "f32", (16,), 1,
             ("sa", "swa", "gated"), (False, True)),
    Workload("qwen3-8b-layer-n4096-w128", 2, 1, 4096, 32, 8, 128, "bf16", (128,), 4,
             ("gated",)),
    Workload("360m-layer-b8-n2048-w256", 3, 8, 2048, 16, 16, 64, "bf16", (256,), 1,
             ("gated",)),
    Workload("long-n32768-w128", 4, 1, 32768, 32, 8, 128, "bf16", (32, 64, 128), 1,
             ("sa", "gated", "swa")),
    Workload("qwen3-30b-a3b-layer-n131072-w64", 5, 1, 131072, 32, 4, 128, "bf16", (64,), 2,
             ("gated",)),
]


def workload(index: int) -> Workload:
    for wl in WORKLOADS:
        if wl.index == index:
            return wl
    raise KeyError(index)


def sigma_seed(index: int, layer: int) -> int:
    """Seed of the permutation of layer ``layer`` of workload ``index``."""
    return 1000 * index + layer


def data_seed(index: int, layer: int) -> int:
    """Seed of the Q/K/V/gate draw of layer ``layer`` of workload ``index``."""
    return 1000 * index + 100 + layer


_DT = {"f32": torch.float32, "bf16": torch.bfloat16}


def torch_dtype(name: str) -> torch.dtype:
    return _DT[name]


def qkv(seed: int, B: int, n: int, Hq: int, Hkv: int, d: int, dtype: str = "bf16"):
    """Q [B, n, Hq, d], K and V [B, n, Hkv, d], each N(0, 1), cast to ``dtype`` (CPU tensors)."""
    g = torch.Generator().manual_seed(seed)
    dt = _DT[dtype]
    q = torch.randn(B, n, Hq, d, generator=g, dtype=torch.float32).to(dt)
    k = torch.randn(B, n, Hkv, d, generator=g, dtype=torch.float32).to(dt)
    v = torch.randn(B, n, Hkv, d, generator=g, dtype=torch.float32).to(dt)
    return q, k, v


def gates(seed: int, B: int, n: int, Hq: int):
    """Gate values float32 [2, B, n, Hq] (g_sa first), each sigmoid(N(0, 1))."""
    g = torch.Generator().manual_seed(seed ^ 0x5A5A)
    return torch.sigmoid(torch.randn(2, B, n, Hq, generator=g, dtype=torch.float32))


def upstream_grad(seed: int, B: int, n: int, Hq: int, d: int, dtype: str = "bf16"):
    """An upstream gradient dL/dY [B, n, Hq, d], N(0, 1), cast to ``dtype`` (CPU tensor).

    Stands in for whatever the layers above would send back; the backward's cost and numerics do
    not depend on its distribution beyond its scale.
    """
    g = torch.Generator().manual_seed(seed ^ 0x3C3C)
    return torch.randn(B, n, Hq, d, generator=g, dtype=torch.float32).to(_DT[dtype])


def gate_inputs(seed: int, rows: int, Hm: int, Hq: int):
    """Layer input x [rows, Hm] ~ N(0, 1) (bf16), projection weight w_t [2 Hq, Hm] ~ N(0, 1/Hm)
    (bf16, so each logit is ~ N(0, 1)) and bias [2 Hq] ~ N(0, 1) (fp32), CPU tensors."""
    g = torch.Generator().manual_seed(seed ^ 0x6B6B)
    x = torch.randn(rows, Hm, generator=g, dtype=torch.float32).to(torch.bfloat16)
    w_t = (torch.randn(2 * Hq, Hm, generator=g, dtype=torch.float32) / Hm ** 0.5).to(torch.bfloat16)
    bias = torch.randn(2 * Hq, generator=g, dtype=torch.float32)
    return x, w_t, bias
