"""Packed batches: sequences one after another in every head ([H, N, d]
tensors, per-sequence row offsets), against the same batch padded.

The library plans each sequence from its own lengths in either layout and
runs the same kernels over it, so every sequence's outputs must agree
bitwise between the layouts, except the sums formed by atomics (dQ of the
fused and decode backward, dK of shared key heads), which agree to fp32
rounding.  The padded layout is itself checked against the oracle
elsewhere; one sequence here is also checked against the oracle directly.
"""
import numpy as np
import pytest
import torch

import oracle
import test_gpu_random_ragged as random_ragged
import workloads
from attention_kl_divergence_amd import streamkl as sk
from parity import check_forward_rows, check_grad, to_np

pytestmark = pytest.mark.gpu

CASES = [
    # name, dtype, d1, d2, causal, H, kv1, kv2, lengths kind, B, seed
    ("bf16-c-prefill-b70", "bf16", 128, 128, True, 4, 4, 4, "prefill", 70, 1),
    ("bf16-nc-decode-gqa-b66", "bf16", 128, 64, False, 8, 2, 4, "decode", 66, 2),
    ("f32-c-d64-b20", "f32", 64, 64, True, 2, 2, 2, "prefill", 20, 3),
    ("bf16-nc-mixed-split-b6", "bf16", 128, 128, False, 2, 2, 2, "mixed", 6, 4),
]


def _lengths(kind, B, causal, seed):
    r = np.random.default_rng(300 + seed)
    if kind == "mixed":  # short ranges that split on their own, decode-shaped ones, an empty one
        return [64, 16, 100, 0, 9, 40], [2000, 3000, 4000, 10, 2500, 2100]
    q_len, k_len = [], []
    for i in range(B):
        if kind == "decode":
            k = int(r.integers(33, 3000))
            q = 0 if i % 13 == 12 else int(r.integers(1, 33))
        else:
            k = int(r.integers(1, 700))
            q = 0 if i % 9 == 8 else (k if causal else int(r.integers(1, 700)))
        q_len.append(q)
        k_len.append(k)
    return q_len, k_len


def _pack(x, lens):
    """[B, heads, N, d] (or [B, heads, N]) padded -> [heads, sum(lens), ...] packed."""
    return torch.cat([x[b, :, :n] for b, n in enumerate(lens)], dim=1).contiguous()


def _inputs(case, dev):
    name, dt, d1, d2, causal, H, kv1, kv2, kind, B, seed = case
    q_len, k_len = _lengths(kind, B, causal, seed)
    B = len(q_len)
    w = workloads.Workload(name, B, H, max(q_len), max(k_len), d1, d2, dt, causal, 0.0, True, 80 + seed)
    q1, _, q2, _ = workloads.generate(w, dev)
    gen = torch.Generator(device=dev).manual_seed(180 + seed)
    k1 = torch.randn((B, kv1, w.n_k, d1), generator=gen, device=dev).to(w.torch_dtype)
    k2 = torch.randn((B, kv2, w.n_k, d2), generator=gen, device=dev).to(w.torch_dtype)
    g = workloads.upstream_grad(w, dev, "random")
    return w, (q1, k1, q2, k2, g), q_len, k_len


def _offsets(lens):
    return [0] + list(np.cumsum(lens).astype(int))


def _same(a, b, exact, what):
    if exact:
        assert torch.equal(a, b), what
    else:
        torch.testing.assert_close(a, b, rtol=1e-5, atol=1e-6 * b.abs().max().item(), msg=what)


def _check_layouts(w, q1, k1, q2, k2, g, q_len, k_len, dev, oracle_rows=True):
    """Every entry point on the padded batch and on the same sequences packed:
    each sequence's outputs equal across the layouts (bitwise except sums
    formed by atomics); the longest sequence against the oracle."""
    H, causal = w.H, w.causal
    g1, g2 = H // k1.shape[1], H // k2.shape[1]
    pad = dict(q_len=q_len, k_len=k_len)
    pk = dict(q_off=_offsets(q_len), k_off=_offsets(k_len))
    P = [_pack(q1, q_len), _pack(k1, k_len), _pack(q2, q_len), _pack(k2, k_len)]
    gp = _pack(g, q_len)
    print(f"packed {w.name}", flush=True)

    fwd_a = sk.streamkl_fwd(q1, k1, q2, k2, causal, **pad)
    fwd_b = sk.streamkl_fwd(*P, causal, **pk)
    weights = torch.rand((w.B, H, w.n_q), device=dev)
    loss_a = sk.streamkl_fwd_loss(q1, k1, q2, k2, causal, weights, **pad)[3]
    loss_b = sk.streamkl_fwd_loss(*P, causal, _pack(weights, q_len), **pk)[3]
    modes = (sk.BWD_AUTO, sk.BWD_SEPARATE, sk.BWD_FUSED)
    bwd_a = {(s, m): sk.streamkl_bwd(s, q1, k1, q2, k2, causal, *fwd_a, g, bwd_mode=m, **pad)
             for s in (1, 2) for m in modes}
    bwd_b = {(s, m): sk.streamkl_bwd(s, *P, causal, *fwd_b, gp, bwd_mode=m, **pk) for s in (1, 2) for m in modes}
    joint_a = sk.streamkl_bwd_joint(q1, k1, q2, k2, causal, *fwd_a, g, **pad)
    joint_b = sk.streamkl_bwd_joint(*P, causal, *fwd_b, gp, **pk)
    torch.cuda.synchronize()

    for a, b, n in zip(fwd_a, fwd_b, ("KL", "LSE1", "LSE2")):
        assert b.shape == (H, sum(q_len))
        _same(b, _pack(a, q_len), True, f"{w.name} {n}")
    # the loss sums the same per-workgroup partials in a different order of launches
    assert abs(loss_b.item() - loss_a.item()) <= 1e-5 * abs(loss_a.item()) + 1e-7
    for (s, m), (dqa, dka) in bwd_a.items():
        dqb, dkb = bwd_b[(s, m)]
        shared = (g2 if s == 1 else g1) > 1
        # dQ by atomics: the fused mode, and the automatic mode where it picks
        # the fused or decode backward for a sequence
        _same(dqb, _pack(dqa, q_len), m == sk.BWD_SEPARATE, f"{w.name} s{s} m{m} dQ")
        _same(dkb, _pack(dka, k_len), not shared, f"{w.name} s{s} m{m} dK")
    # the joint kernels (a separate plan) or one automatic pass per setting
    joint_sep = sk.bwd_plan(sk.packed_shape_of(*P, **pk), causal, 1) == sk.BWD_SEPARATE
    for i, (a, b) in enumerate(zip(joint_a, joint_b)):
        lens = q_len if i % 2 == 0 else k_len
        exact = (i % 2 == 0 and joint_sep) or (i % 2 == 1 and (g1 if i == 1 else g2) == 1)
        _same(b, _pack(a, lens), exact, f"{w.name} joint output {i}")
    if not oracle_rows:
        return

    # one sequence straight against the oracle, from the packed outputs
    b = int(np.argmax(q_len))
    qo, ko = pk["q_off"][b], pk["k_off"][b]
    nq, nk = q_len[b], k_len[b]
    kl_n, l1n, l2n, gn = (to_np(t) for t in (*fwd_b, gp))
    dq, dk = (to_np(t) for t in bwd_b[(1, sk.BWD_SEPARATE)])
    ref_dk = np.zeros((k2.shape[1], nk, w.d2))
    for h in range(H):
        hi = [to_np(P[0][h, qo:qo + nq]), to_np(P[1][h // g1, ko:ko + nk]), to_np(P[2][h, qo:qo + nq]),
              to_np(P[3][h // g2, ko:ko + nk])]
        ref = oracle.head_forward(*hi, causal)
        check_forward_rows(f"{w.name} packed b{b}h{h}", kl_n[h, qo:qo + nq], l1n[h, qo:qo + nq], l2n[h, qo:qo + nq],
                           ref, w.torch_dtype)
        rdq, rdk = oracle.head_backward(1, *hi, causal, gn[h, qo:qo + nq])
        check_grad(f"{w.name} packed b{b}h{h} dQ", dq[h, qo:qo + nq], rdq)
        ref_dk[h // g2] += rdk
    for kh in range(ref_dk.shape[0]):
        check_grad(f"{w.name} packed b{b} kh{kh} dK", dk[kh, ko:ko + nk], ref_dk[kh])


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_packed_matches_padded(case, cuda_device):
    w, (q1, k1, q2, k2, g), q_len, k_len = _inputs(case, cuda_device)
    _check_layouts(w, q1, k1, q2, k2, g, q_len, k_len, cuda_device)


RANDOM = [c for c in random_ragged.CASES if sum(c[10]) > 0]


@pytest.mark.parametrize("case", RANDOM, ids=[c[0] for c in RANDOM])
def test_random_batches_packed(case, cuda_device):
    """The seeded random ragged batches (dtypes, head dims, masks, grouped
    keys, empty and decode-shaped sequences) packed against padded."""
    name, dt, d1, d2, causal, H, kv1, kv2, n_q, n_k, q_len, k_len = case
    B = len(q_len)
    w = workloads.Workload(name, B, H, n_q, n_k, d1, d2, dt, causal, 0.0, True, 31)
    q1, _, q2, _ = workloads.generate(w, cuda_device)
    gen = torch.Generator(device=cuda_device).manual_seed(91)
    k1 = torch.randn((B, kv1, n_k, d1), generator=gen, device=cuda_device).to(w.torch_dtype)
    k2 = torch.randn((B, kv2, n_k, d2), generator=gen, device=cuda_device).to(w.torch_dtype)
    g = workloads.upstream_grad(w, cuda_device, "random")
    _check_layouts(w, q1, k1, q2, k2, g, q_len, k_len, cuda_device, oracle_rows=False)


def test_packed_autograd_loss(cuda_device):
    """attention_kl_loss on a packed batch: the loss and the gradients (in
    the packed layout) equal those of the same batch padded."""
    case = CASES[0]
    w, (q1, k1, q2, k2, _), q_len, k_len = _inputs(case, cuda_device)
    pad_leaves = [t.clone().requires_grad_(True) for t in (q1, k1, q2, k2)]
    pk_leaves = [_pack(t, n).requires_grad_(True) for t, n in zip((q1, k1, q2, k2), (q_len, k_len, q_len, k_len))]
    print("packed autograd", flush=True)
    loss_a = sk.attention_kl_loss(*pad_leaves, causal=True, bwd_mode=sk.BWD_SEPARATE, q_len=q_len, k_len=k_len)
    loss_b = sk.attention_kl_loss(*pk_leaves, causal=True, bwd_mode=sk.BWD_SEPARATE, q_off=_offsets(q_len),
                                  k_off=_offsets(k_len))
    loss_a.backward()
    loss_b.backward()
    torch.cuda.synchronize()
    assert abs(loss_b.item() - loss_a.item()) <= 1e-5 * abs(loss_a.item())
    for a, b, n in zip(pad_leaves, pk_leaves, (q_len, k_len, q_len, k_len)):
        assert torch.equal(b.grad, _pack(a.grad, n))


def test_packed_ragged_workload_full_size(cuda_device):
    """The ragged benchmark workload (causal sequences of 8K, 16K, 4K and 32K
    rows, 32 heads) packed, as the benchmark's packed line runs it: sampled
    rows of every sequence on two heads, forward and dQ, against the oracle;
    the packed outputs equal the padded call's on every sequence's rows."""
    w = workloads.WORKLOADS["ragged-b4-h32-n32k-d128-bf16-causal"]
    q1, k1, q2, k2 = workloads.generate(w, cuda_device)
    L = list(w.lengths)
    g = workloads.upstream_grad(w, cuda_device, "random")
    off = _offsets(L)
    P = [_pack(t, L) for t in (q1, k1, q2, k2)]
    gp = _pack(g, L)
    print("packed ragged workload", flush=True)
    kl, l1, l2 = sk.streamkl_fwd(*P, True, q_off=off, k_off=off)
    dq, _ = sk.streamkl_bwd(1, *P, True, kl, l1, l2, gp, bwd_mode=sk.BWD_DQ_ONLY, q_off=off, k_off=off)
    kla, l1a, l2a = sk.streamkl_fwd(q1, k1, q2, k2, True, q_len=L, k_len=L)
    torch.cuda.synchronize()
    assert torch.equal(kl, _pack(kla, L)) and torch.equal(l1, _pack(l1a, L)) and torch.equal(l2, _pack(l2a, L))
    rng = np.random.default_rng(8)
    gn = to_np(gp)
    for b, n in enumerate(L):
        o = off[b]
        rows = np.unique(np.concatenate([[0, n - 1], rng.choice(n, 24, replace=False)]))
        for h in (0, 31):
            print(f"oracle sequence {b} head {h}", flush=True)
            hi = [to_np(t[h, o:o + n]) for t in P]
            ref = oracle.head_forward(*hi, True, rows=rows, block=64)
            check_forward_rows(f"packed ragged b{b}h{h}", to_np(kl[h, o:o + n])[rows], to_np(l1[h, o:o + n])[rows],
                               to_np(l2[h, o:o + n])[rows], ref, w.torch_dtype)
            rdq, _ = oracle.head_backward(1, *hi, True, gn[h, o:o + n], rows=rows, block=64, want_dk=False)
            check_grad(f"packed ragged b{b}h{h} dQ rows", to_np(dq[h, o:o + n])[rows], rdq)
