"""Seeded random small shapes, every row against the fp64 oracle.

Each case draws B, H, N_Q, N_K, the two head dims, the dtype and the mask, so
ragged tails, tiny and tall/wide ranges, mixed head dims and the decode path
(bf16, N_Q <= 32) all come up; the forward runs with the library's split
plan, one split and three splits, the backward in both settings and both
modes (the same checks as the fixed small shapes).
"""
import numpy as np
import pytest

import workloads
from test_gpu_parity import run_full

pytestmark = pytest.mark.gpu


def _case(seed):
    r = np.random.default_rng(5000 + seed)
    dt = "bf16" if r.random() < 0.75 else "f32"
    d1, d2 = (int(x) for x in r.choice([64, 128], size=2))
    n_q = int(r.choice([int(r.integers(1, 33)), int(r.integers(33, 400))]))
    n_k = int(r.integers(1, 500))
    causal = bool(r.random() < 0.5)
    if causal and n_q > n_k:
        n_q, n_k = n_k, n_q
    B, H = int(r.integers(1, 3)), int(r.integers(1, 3))
    name = f"rand{seed}-{dt}-d{d1}x{d2}-{'c' if causal else 'nc'}-B{B}H{H}-q{n_q}-k{n_k}"
    return workloads.Workload(name, B, H, n_q, n_k, d1, d2, dt, causal, 0.5, d1 != d2, 40 + seed)


CASES = [_case(s) for s in range(48)]


@pytest.mark.parametrize("w", CASES, ids=[w.name for w in CASES])
def test_random_shape(w, cuda_device):
    print(w.name, flush=True)
    run_full(w, cuda_device, splits=(0, 1, 3))
