"""The autograd wrapper attention_kl against the fp64 oracle.

KL(P1 || P2) depends on (Q2, K2) only through P2 and on (Q1, K1) only through
P1, so the gradients the wrapper returns (setting 1 for the student side,
setting 2 for the teacher side) are the true gradients of the loss; they are
compared with the oracle's, cast to the input dtype as the wrapper casts them.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from attention_kl_divergence_amd import streamkl as sk
from parity import check_grad, head_inputs, kl_tol, to_np

pytestmark = pytest.mark.gpu

CASES = [
    # name, dtype, d1, d2, causal, H, n_q, n_k, scale1, scale2
    ("bf16-d128-c", "bf16", 128, 128, True, 2, 190, 190, 0.0, 0.0),
    ("bf16-d128x64-nc-scaled", "bf16", 128, 64, False, 2, 130, 257, 0.05, 0.2),
    ("f32-d64-c", "f32", 64, 64, True, 1, 150, 150, 0.0, 0.0),
]


def _inputs(case, dev):
    name, dt, d1, d2, causal, H, n_q, n_k, s1, s2 = case
    w = workloads.Workload(name, 1, H, n_q, n_k, d1, d2, dt, causal, 0.5, d1 != d2, 11)
    return w, workloads.generate(w, dev)


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_weighted_loss_all_inputs(case, cuda_device):
    """loss = sum_i w_i KL_i with gradients to all four inputs."""
    w, (q1, k1, q2, k2) = _inputs(case, cuda_device)
    s1, s2 = case[8], case[9]
    wt = workloads.upstream_grad(w, cuda_device, "random")
    leaves = [t.clone().requires_grad_(True) for t in (q1, k1, q2, k2)]
    print(f"autograd {w.name}", flush=True)
    kl = sk.attention_kl(*leaves, causal=w.causal, scale1=s1, scale2=s2)
    (kl.float() * wt).sum().backward()
    torch.cuda.synchronize()
    for t, leaf in zip((q1, k1, q2, k2), leaves):
        assert leaf.grad is not None and leaf.grad.dtype == t.dtype and leaf.grad.shape == t.shape
    sc = dict(scale1=s1 or None, scale2=s2 or None)
    gn = to_np(wt)
    for h in range(w.H):
        hi = head_inputs(q1, k1, q2, k2, 0, h)
        ref = oracle.head_forward(*hi, w.causal, **sc)
        rkl = ref[0]
        a, r = kl_tol(w.torch_dtype)
        err = np.abs(to_np(kl[0, h]) - rkl)
        assert (err <= a + r * np.abs(rkl)).all(), f"{w.name} h{h}: KL worst |d|={err.max():.3e}"
        dq2, dk2 = oracle.head_backward(1, *hi, w.causal, gn[0, h], **sc)
        dq1, dk1 = oracle.head_backward(2, *hi, w.causal, gn[0, h], **sc)
        for lab, leaf, rv in (("dQ1", leaves[0], dq1), ("dK1", leaves[1], dk1),
                              ("dQ2", leaves[2], dq2), ("dK2", leaves[3], dk2)):
            check_grad(f"{w.name} h{h} {lab}", to_np(leaf.grad[0, h]), rv)


def test_student_only_mean_loss(cuda_device):
    """Only (Q2, K2) require grad and the loss is the mean KL: the upstream
    gradient arrives as an expanded (stride-0) tensor, and the teacher side
    gets no gradient."""
    case = CASES[0]
    w, (q1, k1, q2, k2) = _inputs(case, cuda_device)
    q2l, k2l = q2.clone().requires_grad_(True), k2.clone().requires_grad_(True)
    print(f"autograd student-only {w.name}", flush=True)
    kl = sk.attention_kl(q1, k1, q2l, k2l, causal=w.causal)
    kl.mean().backward()
    torch.cuda.synchronize()
    assert q1.grad is None and k1.grad is None
    g = np.full(w.n_q, 1.0 / (w.H * w.n_q))
    for h in range(w.H):
        hi = head_inputs(q1, k1, q2, k2, 0, h)
        dq2, dk2 = oracle.head_backward(1, *hi, w.causal, g)
        check_grad(f"{w.name} h{h} dQ2", to_np(q2l.grad[0, h]), dq2)
        check_grad(f"{w.name} h{h} dK2", to_np(k2l.grad[0, h]), dk2)


@pytest.mark.parametrize("ragged", [False, True], ids=["dense", "ragged"])
def test_fused_loss_autograd_matches_unfused(ragged, cuda_device):
    """attention_kl_loss (the loss formed in the forward's epilogue) against
    attention_kl followed by the same reduction in PyTorch: the loss agrees
    to fp32 rounding, and the input gradients are bitwise equal (both feed
    the same d loss / d KL_i to the same deterministic kernels).  Weighted
    with a gradient to the weights, and the mean over the rows (ragged:
    each element's rows only)."""
    B, H, n_q, n_k = 3, 2, 200, 260
    w = workloads.Workload("loss-autograd", B, H, n_q, n_k, 128, 128, "bf16", True, 0.5, False, 21)
    q1, k1, q2, k2 = workloads.generate(w, cuda_device)
    lens = dict(q_len=[200, 0, 77], k_len=[260, 5, 100]) if ragged else {}
    valid = torch.zeros((B, H, n_q), device=cuda_device)
    for b, n in enumerate(lens.get("q_len", [n_q] * B)):
        valid[b, :, :n] = 1.0
    rows = valid.sum().item()
    print(f"fused loss autograd ragged={ragged}", flush=True)
    for weighted in (True, False):
        wt = torch.rand((B, H, n_q), device=cuda_device) if weighted else None
        fused = [t.clone().requires_grad_(True) for t in (q1, k1, q2, k2)]
        plain = [t.clone().requires_grad_(True) for t in (q1, k1, q2, k2)]
        wf = wt.clone().requires_grad_(True) if weighted else None
        wp = wt.clone().requires_grad_(True) if weighted else None
        loss = sk.attention_kl_loss(*fused, causal=True, weights=wf, bwd_mode=sk.BWD_SEPARATE, **lens)
        kl = sk.attention_kl(*plain, causal=True, bwd_mode=sk.BWD_SEPARATE, **lens)
        ref = (kl * wp).sum() if weighted else (kl * valid).sum() / rows
        loss.backward()
        ref.backward()
        torch.cuda.synchronize()
        assert loss.dim() == 0
        assert abs(loss.item() - ref.item()) <= 1e-5 * abs(ref.item()) + 1e-7, (loss.item(), ref.item())
        for i, (a, b) in enumerate(zip(fused, plain)):
            assert torch.equal(a.grad, b.grad), f"weighted={weighted} input {i}: gradients differ"
        if weighted:
            assert torch.equal(wf.grad, wp.grad)
