"""GPU parity of the joint backward (gradients to both models in one pass)
against the fp64 oracle's two settings.

The joint result must equal setting 2 (dQ1, dK1) and setting 1 (dQ2, dK2)
of the definition: every element on small shapes (several key and query
tiles, ragged tails, masks, mixed head dims), sampled rows and the causal dK
tail at the 8K, 32-head workload, and exact zeros for identical models.  The
autograd wrapper takes this path when both sides are trainable (its weighted
loss test in test_gpu_autograd.py).
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from attention_kl_divergence_amd import streamkl as sk
from parity import check_grad, head_inputs, to_np

pytestmark = pytest.mark.gpu

CASES = [
    # name, dtype, d1, d2, causal, B, H, n_q, n_k
    ("bf16-d128-c", "bf16", 128, 128, True, 1, 2, 300, 300),
    ("bf16-d128-nc-rect", "bf16", 128, 128, False, 1, 2, 257, 517),
    ("bf16-d128x64-c", "bf16", 128, 64, True, 1, 2, 260, 333),
    ("bf16-d64x128-nc-tall", "bf16", 64, 128, False, 2, 1, 400, 130),
    ("bf16-d64-c", "bf16", 64, 64, True, 1, 2, 190, 190),
    ("bf16-q16-k2000", "bf16", 128, 128, False, 1, 2, 16, 2000),
    ("f32-d64x128-c", "f32", 64, 128, True, 1, 2, 100, 150),
]
MODES = [sk.BWD_AUTO, sk.BWD_SEPARATE, sk.BWD_FUSED]


def _say(msg):
    print(msg, flush=True)


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_joint_small_full_parity(case, cuda_device):
    name, dt, d1, d2, causal, B, H, n_q, n_k = case
    w = workloads.Workload(name, B, H, n_q, n_k, d1, d2, dt, causal, 0.5, d1 != d2, 11)
    q1, k1, q2, k2 = workloads.generate(w, cuda_device)
    g = workloads.upstream_grad(w, cuda_device, "random")
    kl, l1, l2 = sk.streamkl_fwd(q1, k1, q2, k2, causal)
    outs = {}
    for m in MODES:
        _say(f"joint {name} mode {m}")
        outs[m] = [to_np(t) for t in sk.streamkl_bwd_joint(q1, k1, q2, k2, causal, kl, l1, l2, g, bwd_mode=m)]
        torch.cuda.synchronize()
    # the single-output modes write exactly their pair
    dq1, dk1, dq2, dk2 = sk.streamkl_bwd_joint(q1, k1, q2, k2, causal, kl, l1, l2, g, bwd_mode=sk.BWD_DK_ONLY)
    assert dq1 is None and dq2 is None
    np.testing.assert_array_equal(to_np(dk1), outs[sk.BWD_SEPARATE][1])
    np.testing.assert_array_equal(to_np(dk2), outs[sk.BWD_SEPARATE][3])
    dq1, dk1, dq2, dk2 = sk.streamkl_bwd_joint(q1, k1, q2, k2, causal, kl, l1, l2, g, bwd_mode=sk.BWD_DQ_ONLY)
    assert dk1 is None and dk2 is None
    np.testing.assert_array_equal(to_np(dq1), outs[sk.BWD_SEPARATE][0])
    np.testing.assert_array_equal(to_np(dq2), outs[sk.BWD_SEPARATE][2])
    gn = to_np(g)
    for b in range(B):
        for h in range(H):
            hi = head_inputs(q1, k1, q2, k2, b, h)
            r2 = oracle.head_backward(2, *hi, causal, gn[b, h])
            r1 = oracle.head_backward(1, *hi, causal, gn[b, h])
            for m, (a1, a2, a3, a4) in outs.items():
                tag = f"{name} b{b}h{h} m{m}"
                check_grad(tag + " dQ1", a1[b, h], r2[0])
                check_grad(tag + " dK1", a2[b, h], r2[1])
                check_grad(tag + " dQ2", a3[b, h], r1[0])
                check_grad(tag + " dK2", a4[b, h], r1[1])


def test_joint_identical_models_exact_zero(cuda_device):
    w = workloads.Workload("same", 1, 2, 200, 260, 128, 128, "bf16", True, 0.0, False, 5)
    q1, k1, _, _ = workloads.generate(w, cuda_device)
    g = workloads.upstream_grad(w, cuda_device, "random")
    kl, l1, l2 = sk.streamkl_fwd(q1, k1, q1, k1, True)
    assert (kl == 0).all()
    for t in sk.streamkl_bwd_joint(q1, k1, q1, k1, True, kl, l1, l2, g):
        assert (t == 0).all()


def test_joint_8k_causal_sampled(cuda_device):
    """The 32-head, 8K causal bf16 workload, both models trained in one pass:
    sampled query rows (dQ1, dQ2) and the last 2048 keys (dK1, dK2) against
    the oracle on three heads."""
    w = workloads.WORKLOADS["h32-n8k-d128-bf16-causal"]
    q1, k1, q2, k2 = workloads.generate(w, cuda_device)
    g = workloads.upstream_grad(w, cuda_device, "random")
    kl, l1, l2 = sk.streamkl_fwd(q1, k1, q2, k2, True)
    assert sk.bwd_plan(sk.shape_of(q1, k1, q2, k2), True, 1) == sk.BWD_SEPARATE
    _say("joint 8k")
    dq1, dk1, dq2, dk2 = sk.streamkl_bwd_joint(q1, k1, q2, k2, True, kl, l1, l2, g)
    torch.cuda.synchronize()
    rng = np.random.default_rng(3)
    rows = np.unique(np.concatenate([[0, 1, w.n_q - 1], rng.choice(w.n_q, 125, replace=False)]))
    keys = np.arange(w.n_k - 2048, w.n_k)
    for h in (0, 17, 31):
        hi = head_inputs(q1, k1, q2, k2, 0, h)
        gh = to_np(g[0, h])
        _say(f"oracle head {h}")
        r2q, _ = oracle.head_backward(2, *hi, True, gh, rows=rows, block=256)
        r1q, _ = oracle.head_backward(1, *hi, True, gh, rows=rows, block=256)
        check_grad(f"8k h{h} dQ1", to_np(dq1[0, h])[rows], r2q)
        check_grad(f"8k h{h} dQ2", to_np(dq2[0, h])[rows], r1q)
        r2k = oracle.head_backward_dk_rows(2, *hi, True, gh, key_rows=keys, block=256)
        r1k = oracle.head_backward_dk_rows(1, *hi, True, gh, key_rows=keys, block=256)
        check_grad(f"8k h{h} dK1 tail", to_np(dk1[0, h])[keys], r2k)
        check_grad(f"8k h{h} dK2 tail", to_np(dk2[0, h])[keys], r1k)
