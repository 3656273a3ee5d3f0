"""Seeded random ragged batches with grouped key heads, every row of every
sequence against the fp64 oracle (the checks of test_gpu_ragged: padded
rows 0, the library on the trimmed tensors, both settings in every mode and
the joint backward).

Each case draws the batch size, the query and key-head counts, the dtype,
both head dims, the mask, the padded sizes and one query and key length per
sequence, empty and decode-shaped (at most 32 query rows) ones included.
"""
import numpy as np
import pytest

from test_gpu_ragged import test_ragged_batch as check_ragged

pytestmark = pytest.mark.gpu


def _case(seed):
    r = np.random.default_rng(7000 + seed)
    dt = "bf16" if r.random() < 0.75 else "f32"
    d1, d2 = (int(x) for x in r.choice([64, 128], size=2))
    causal = bool(r.random() < 0.5)
    H = int(r.choice([2, 4, 8]))
    divisors = [k for k in (1, 2, 4, 8) if H % k == 0]
    kv1, kv2 = int(r.choice(divisors)), int(r.choice(divisors))
    B = int(r.integers(1, 5))
    n_k = int(r.integers(8, 400))
    n_q = int(r.integers(1, n_k + 1)) if causal else int(r.integers(1, 300))
    q_len, k_len = [], []
    for _ in range(B):
        k = int(r.integers(1, n_k + 1))
        q = int(r.choice([0, int(r.integers(1, 33)), int(r.integers(1, n_q + 1))]))
        q = min(q, n_q, k if causal else n_q)
        q_len.append(q)
        k_len.append(k)
    name = f"rr{seed}-{dt}-d{d1}x{d2}-{'c' if causal else 'nc'}-H{H}kv{kv1}x{kv2}-B{B}-q{n_q}-k{n_k}"
    return (name, dt, d1, d2, causal, H, kv1, kv2, n_q, n_k, q_len, k_len)


CASES = [_case(s) for s in range(16)]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_random_ragged(case, cuda_device):
    check_ragged(case, cuda_device)
