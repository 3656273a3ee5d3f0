"""Seeded synthetic inputs for the attention-KL workloads.

This module draws random tensors and nothing else: it holds none of the
method's arithmetic, so both the GPU path (tests, bench) and the CPU oracle
can take their inputs from it.

Recipe (every workload): the teacher tensors Q1, K1 are fp32 draws from
N(0, 1) with a generator seeded ``seed``; the student tensors Q2, K2 are
``teacher + noise * N(0, 1)`` with an independent generator seeded
``100 + seed`` (or, for workloads whose two models have different head
dimensions, fresh N(0, 1) draws from that second generator).  Each tensor is
then rounded once to the workload dtype (round-to-nearest-even for bf16).
Layout is contiguous [B, H, N, d].
"""
from __future__ import annotations

from dataclasses import dataclass, replace

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    n_q: int
    n_k: int
    d1: int
    d2: int
    dtype: str          # "f32" or "bf16"
    causal: bool
    noise: float        # student = teacher + noise * N(0,1); ignored if independent
    independent: bool   # draw the student independently (different head dims)
    seed: int
    settings: tuple = (1,)  # backward settings one step runs (empty: forward only)
    kv_heads: int = 0       # key heads of both models (0: one per query head)
    lengths: tuple = ()     # ragged batch: per batch element lengths (query = key), () for none

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


# The workloads the pages' experiments are shaped like (32 heads, head dim
# 128, contexts from 4K to 512K, causal and non-causal, decode-shaped rows).
WORKLOADS = {
    w.name: w for w in [
        Workload("h1-n512-d64-f32", 1, 1, 512, 512, 64, 64, "f32", False, 0.3, False, 1),
        Workload("h32-n8k-d128-bf16-causal", 1, 32, 8192, 8192, 128, 128, "bf16", True, 0.5, False, 2, (1, 2)),
        Workload("h32-n64k-d128-bf16-causal", 1, 32, 65536, 65536, 128, 128, "bf16", True, 0.5, False, 3),
        Workload("h32-n64k-d128-bf16", 1, 32, 65536, 65536, 128, 128, "bf16", False, 0.5, False, 3),
        Workload("decode-h32-q1-k128k-d128-bf16", 1, 32, 1, 131072, 128, 128, "bf16", False, 0.5, False, 4, ()),
        Workload("decode-h32-q16-k128k-d128-bf16", 1, 32, 16, 131072, 128, 128, "bf16", False, 0.5, False, 4, ()),
        Workload("decode-h32-q1-k512k-d128-bf16", 1, 32, 1, 524288, 128, 128, "bf16", False, 0.5, False, 4, ()),
        Workload("decode-h32-q16-k512k-d128-bf16", 1, 32, 16, 524288, 128, 128, "bf16", False, 0.5, False, 4, ()),
        # the decode-shaped forward followed by the backward of one setting
        Workload("decode-bwd-h32-q1-k512k-d128-bf16", 1, 32, 1, 524288, 128, 128, "bf16", False, 0.5, False, 4, (1,)),
        Workload("decode-bwd-h32-q16-k512k-d128-bf16", 1, 32, 16, 524288, 128, 128, "bf16", False, 0.5, False, 4, (1,)),
        Workload("h32-n512k-d128x64-bf16-causal", 1, 32, 524288, 524288, 128, 64, "bf16", True, 0.0, True, 5, (2,)),
        # grouped key heads: 32 query heads read 8 key heads
        Workload("h32-kv8-n64k-d128-bf16-causal", 1, 32, 65536, 65536, 128, 128, "bf16", True, 0.5, False, 3,
                 kv_heads=8),
        # ragged batch: four sequences padded to 32K
        Workload("ragged-b4-h32-n32k-d128-bf16-causal", 4, 32, 32768, 32768, 128, 128, "bf16", True, 0.5, False, 6,
                 lengths=(8192, 16384, 4096, 32768)),
    ]
}


def generate(w: Workload, device="cpu"):
    """Return (q1, k1, q2, k2) for workload ``w`` on ``device`` (K with
    ``kv_heads`` heads when set; ragged workloads are drawn at the padded size)."""
    dev = torch.device(device)
    gt = torch.Generator(device=dev).manual_seed(w.seed)
    gn = torch.Generator(device=dev).manual_seed(100 + w.seed)
    f32 = torch.float32

    def randn(shape, gen):
        return torch.randn(shape, generator=gen, device=dev, dtype=f32)

    shp = lambda n, d, h=w.H: (w.B, h, n, d)  # noqa: E731
    kv = w.kv_heads or w.H
    q1 = randn(shp(w.n_q, w.d1), gt)
    k1 = randn(shp(w.n_k, w.d1, kv), gt)
    if w.independent:
        q2 = randn(shp(w.n_q, w.d2), gn)
        k2 = randn(shp(w.n_k, w.d2, kv), gn)
    else:
        assert w.d1 == w.d2
        q2 = q1 + w.noise * randn(shp(w.n_q, w.d2), gn)
        k2 = k1 + w.noise * randn(shp(w.n_k, w.d2, kv), gn)
    dt = w.torch_dtype
    return (q1.to(dt).contiguous(), k1.to(dt).contiguous(),
            q2.to(dt).contiguous(), k2.to(dt).contiguous())


def upstream_grad(w: Workload, device="cpu", kind: str = "mean", seed: int = 0):
    """Per-row upstream gradient g of shape [B, H, n_q] (fp32).

    kind="mean": g = 1/n_q, the gradient of the mean row KL.
    kind="random": seeded N(0,1)/n_q values, so per-row scaling errors show.
    """
    dev = torch.device(device)
    if kind == "mean":
        return torch.full((w.B, w.H, w.n_q), 1.0 / w.n_q, device=dev, dtype=torch.float32)
    gen = torch.Generator(device=dev).manual_seed(1000 + 17 * w.seed + seed)
    return torch.randn((w.B, w.H, w.n_q), generator=gen, device=dev,
                       dtype=torch.float32) / w.n_q


def small(w: Workload, H: int, n_q: int, n_k: int | None = None) -> Workload:
    """Same recipe, smaller shape (for tests the oracle finishes in seconds)."""
    return w.with_(H=H, n_q=n_q, n_k=n_q if n_k is None else n_k,
                   name=f"{w.name}@H{H}-q{n_q}-k{n_q if n_k is None else n_k}")
