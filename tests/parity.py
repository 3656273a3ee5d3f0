"""Helpers for GPU-vs-oracle parity checks (imported by the gpu tests and smoke()).

Tolerances:
* KL per row: |dKL| <= 1e-4 + 1e-3 |KL| for fp32 inputs, 1e-3 + 1e-2 |KL| for bf16.
* LSE per row: |dLSE| <= 1e-4 (1 + |LSE|) (fp32 accumulation of the same
  inputs; derived from fp32 rounding over up to 2^19 keys, with margin).
* dQ, dK: relative L2 error <= 1e-2, per head and over everything compared.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle


def kl_tol(dtype: torch.dtype):
    return (1e-4, 1e-3) if dtype == torch.float32 else (1e-3, 1e-2)


def to_np(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def check_forward_rows(name, kl, lse1, lse2, ref, dtype):
    """kl/lse*: GPU values (numpy) for the rows ref was computed on."""
    rkl, rl1, rl2 = ref
    a, r = kl_tol(dtype)
    err = np.abs(kl - rkl)
    bad = err > a + r * np.abs(rkl)
    assert not bad.any(), (f"{name}: KL mismatch in {bad.sum()} rows, worst |d|={err.max():.3e} "
                           f"at KL={rkl[np.argmax(err)]:.4e}")
    for lab, g, o in (("LSE1", lse1, rl1), ("LSE2", lse2, rl2)):
        e = np.abs(g - o)
        assert (e <= 1e-4 * (1 + np.abs(o))).all(), f"{name}: {lab} worst |d|={e.max():.3e}"
    return float(err.max())


def rel_l2(a, b):
    den = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / den) if den > 0 else float(np.linalg.norm(a))


def check_grad(name, got, ref, tol=1e-2):
    e = rel_l2(got, ref)
    assert e <= tol, f"{name}: relative L2 error {e:.3e} > {tol}"
    return e


def head_inputs(q1, k1, q2, k2, b, h):
    return [to_np(t[b, h]) for t in (q1, k1, q2, k2)]
