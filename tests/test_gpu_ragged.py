"""GPU parity for ragged batches: batch element b uses its first q_len[b]
query rows and k_len[b] key rows of padded tensors.

Each element is compared with the fp64 oracle on its trimmed tensors and
with the library's own call on those trimmed tensors (the same arithmetic:
the forward and the separate-mode gradients are bitwise equal, except dK of
a shared key head, summed by atomics in no fixed order); padded rows
of every output are exactly 0.  The elements mix long ranges, decode-shaped
ones (at most 32 query rows, which take the decode kernels) and empty ones.
"""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import workloads
from attention_kl_divergence_amd import streamkl as sk
from parity import check_forward_rows, check_grad, to_np

pytestmark = pytest.mark.gpu

CASES = [
    # name, dtype, d1, d2, causal, H, kv1, kv2, n_q, n_k, q_len, k_len
    ("bf16-nc", "bf16", 128, 128, False, 2, 2, 2, 200, 300, [200, 17, 0, 90], [300, 150, 40, 1]),
    ("bf16-c-d128x64", "bf16", 128, 64, True, 2, 2, 2, 160, 260, [160, 31, 5, 0], [260, 31, 200, 0]),
    ("f32-c-gqa", "f32", 64, 64, True, 4, 2, 1, 96, 130, [96, 40, 1], [130, 40, 77]),
    ("bf16-nc-gqa-joint", "bf16", 64, 128, False, 4, 1, 2, 120, 150, [120, 9, 64], [150, 150, 33]),
]


def _inputs(case, dev):
    name, dt, d1, d2, causal, H, kv1, kv2, n_q, n_k, ql, kl_ = case
    B = len(ql)
    w = workloads.Workload(name, B, H, n_q, n_k, d1, d2, dt, causal, 0.0, True, 31)
    q1, _, q2, _ = workloads.generate(w, dev)
    gen = torch.Generator(device=dev).manual_seed(91)
    k1 = torch.randn((B, kv1, n_k, d1), generator=gen, device=dev).to(w.torch_dtype)
    k2 = torch.randn((B, kv2, n_k, d2), generator=gen, device=dev).to(w.torch_dtype)
    return w, q1, k1, q2, k2, ql, kl_


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_ragged_batch(case, cuda_device):
    w, q1, k1, q2, k2, ql, kln = _inputs(case, cuda_device)
    B, H = w.B, w.H
    g1, g2 = H // k1.shape[1], H // k2.shape[1]
    lens = dict(q_len=ql, k_len=kln)
    g = workloads.upstream_grad(w, cuda_device, "random")
    print(f"ragged {w.name}", flush=True)
    kl, l1, l2 = sk.streamkl_fwd(q1, k1, q2, k2, w.causal, **lens)
    grads = {}
    for s in (1, 2):
        for m in (sk.BWD_AUTO, sk.BWD_FUSED, sk.BWD_SEPARATE):
            grads[(s, m)] = [to_np(t) for t in sk.streamkl_bwd(s, q1, k1, q2, k2, w.causal, kl, l1, l2, g,
                                                                 bwd_mode=m, **lens)]
    joint = [to_np(t) for t in sk.streamkl_bwd_joint(q1, k1, q2, k2, w.causal, kl, l1, l2, g, **lens)]
    torch.cuda.synchronize()
    kln_, l1n, l2n, gn = to_np(kl), to_np(l1), to_np(l2), to_np(g)
    for b in range(B):
        nq, nk = ql[b], kln[b]
        # padded rows are zero
        assert (kln_[b, :, nq:] == 0).all() and (l1n[b, :, nq:] == 0).all() and (l2n[b, :, nq:] == 0).all()
        outs = {s: [grads[(s, m)] for m in (sk.BWD_AUTO, sk.BWD_FUSED, sk.BWD_SEPARATE)] for s in (1, 2)}
        outs[1].append(joint[2:])
        outs[2].append(joint[:2])
        for s in (1, 2):
            for dq, dk in outs[s]:
                assert (dq[b, :, nq:] == 0).all() and (dk[b, :, nk:] == 0).all()
                if nq == 0:
                    assert (dq[b] == 0).all() and (dk[b] == 0).all()
        if nq == 0:
            continue
        # the library on the trimmed element: the same arithmetic
        t = [x[b:b + 1, :, :n].contiguous() for x, n in ((q1, nq), (k1, nk), (q2, nq), (k2, nk))]
        gt = g[b:b + 1, :, :nq].contiguous()
        rkl, rl1, rl2 = sk.streamkl_fwd(*t, w.causal)
        assert torch.equal(kl[b:b + 1, :, :nq], rkl) and torch.equal(l1[b:b + 1, :, :nq], rl1)
        for s in (1, 2):
            rdq, rdk = sk.streamkl_bwd(s, *t, w.causal, rkl, rl1, rl2, gt, bwd_mode=sk.BWD_SEPARATE)
            dq, dk = grads[(s, sk.BWD_SEPARATE)]
            np.testing.assert_array_equal(dq[b:b + 1, :, :nq], to_np(rdq))
            if (g2 if s == 1 else g1) == 1:
                np.testing.assert_array_equal(dk[b:b + 1, :, :nk], to_np(rdk))
            else:  # a shared key head sums its query heads with atomics, in no fixed order
                np.testing.assert_allclose(dk[b:b + 1, :, :nk], to_np(rdk), rtol=1e-5,
                                           atol=1e-6 * np.abs(to_np(rdk)).max())
        # the oracle, per head on the trimmed tensors; dK summed per key head
        ref_dk = {1: np.zeros((k2.shape[1], nk, w.d2)), 2: np.zeros((k1.shape[1], nk, w.d1))}
        ref_dq = {}
        for h in range(H):
            hi = [to_np(q1[b, h, :nq]), to_np(k1[b, h // g1, :nk]), to_np(q2[b, h, :nq]), to_np(k2[b, h // g2, :nk])]
            ref = oracle.head_forward(*hi, w.causal)
            check_forward_rows(f"{w.name} b{b}h{h}", kln_[b, h, :nq], l1n[b, h, :nq], l2n[b, h, :nq], ref,
                               w.torch_dtype)
            for s in (1, 2):
                dq, dk = oracle.head_backward(s, *hi, w.causal, gn[b, h, :nq])
                ref_dq[(s, h)] = dq
                ref_dk[s][h // (g2 if s == 1 else g1)] += dk
        for s in (1, 2):
            for i, (dq, dk) in enumerate(outs[s]):
                for h in range(H):
                    check_grad(f"{w.name} b{b} s{s} out{i} h{h} dQ", dq[b, h, :nq], ref_dq[(s, h)])
                for kh in range(ref_dk[s].shape[0]):
                    check_grad(f"{w.name} b{b} s{s} out{i} kh{kh} dK", dk[b, kh, :nk], ref_dk[s][kh])


def test_ragged_workload_full_size(cuda_device):
    """The ragged benchmark workload (four causal sequences of 8K, 16K, 4K and
    32K rows padded to 32K, 32 heads) in the configuration the benchmark
    times: sampled rows of every sequence on two heads, forward and dQ,
    against the oracle on the trimmed tensors; padded rows are 0."""
    w = workloads.WORKLOADS["ragged-b4-h32-n32k-d128-bf16-causal"]
    q1, k1, q2, k2 = workloads.generate(w, cuda_device)
    L = list(w.lengths)
    g = workloads.upstream_grad(w, cuda_device, "random")
    print("ragged workload forward", flush=True)
    kl, l1, l2 = sk.streamkl_fwd(q1, k1, q2, k2, True, q_len=L, k_len=L)
    dq, dk = sk.streamkl_bwd(1, q1, k1, q2, k2, True, kl, l1, l2, g, q_len=L, k_len=L)
    torch.cuda.synchronize()
    rng = np.random.default_rng(7)
    gn = to_np(g)
    for b, n in enumerate(L):
        assert (kl[b, :, n:] == 0).all() and (dq[b, :, n:] == 0).all() and (dk[b, :, n:] == 0).all()
        rows = np.unique(np.concatenate([[0, n - 1], rng.choice(n, 30, replace=False)]))
        for h in (0, 31):
            print(f"oracle sequence {b} head {h}", flush=True)
            hi = [to_np(t[b, h, :n]) for t in (q1, k1, q2, k2)]
            ref = oracle.head_forward(*hi, True, rows=rows, block=64)
            check_forward_rows(f"ragged b{b}h{h}", to_np(kl[b, h])[rows], to_np(l1[b, h])[rows],
                               to_np(l2[b, h])[rows], ref, w.torch_dtype)
            rdq, _ = oracle.head_backward(1, *hi, True, gn[b, h, :n], rows=rows, block=64)
            check_grad(f"ragged b{b}h{h} dQ rows", to_np(dq[b, h])[rows], rdq)


def test_ragged_batch_of_empty_elements(cuda_device):
    """Every element empty: every entry point succeeds without a workspace,
    writes zeros to every output (over earlier contents), and the fused loss
    is 0."""
    w = workloads.Workload("ragged-empty", 3, 2, 40, 60, 128, 128, "bf16", False, 0.0, False, 8)
    q1, k1, q2, k2 = workloads.generate(w, cuda_device)
    lens = dict(q_len=[0, 0, 0], k_len=[5, 0, 60])
    g = workloads.upstream_grad(w, cuda_device, "random")
    print("ragged empty", flush=True)
    f32 = dict(device=cuda_device, dtype=torch.float32)
    out = tuple(torch.full((3, 2, 40), 7.0, **f32) for _ in range(3))
    kl, l1, l2 = sk.streamkl_fwd(q1, k1, q2, k2, False, out=out, **lens)
    for t in (kl, l1, l2):
        assert (t == 0).all()
    kl2, _, _, loss = sk.streamkl_fwd_loss(q1, k1, q2, k2, False, **lens)
    wt = torch.rand((3, 2, 40), **f32)
    _, _, _, loss_w = sk.streamkl_fwd_loss(q1, k1, q2, k2, False, wt, **lens)
    torch.cuda.synchronize()
    assert (kl2 == 0).all() and loss.item() == 0.0 and loss_w.item() == 0.0
    for s in (1, 2):
        for m in (sk.BWD_AUTO, sk.BWD_FUSED, sk.BWD_SEPARATE):
            dq, dk = sk.streamkl_bwd(s, q1, k1, q2, k2, False, kl, l1, l2, g, bwd_mode=m, **lens)
            assert (dq == 0).all() and (dk == 0).all()
    for t in sk.streamkl_bwd_joint(q1, k1, q2, k2, False, kl, l1, l2, g, **lens):
        assert (t == 0).all()


def test_ragged_split_elements_and_workspace_fallback(cuda_device):
    """Elements that take a key split of their own: short query ranges
    (40-100 rows) against 2000-4000 keys in a batch too small to fill the
    chip unsplit (bf16: the 4-wave split-K kernel and its merge, one element
    after another), beside decode-shaped ones (grouped split-K).  Each
    element equals its own call bitwise.  Then a batch of decode-shaped
    requests given a workspace too small for their grouped partials but
    large enough for each request's own: each request then runs on its own
    plan and equals its own call bitwise."""
    q_len, k_len = [64, 16, 100, 0, 9, 40], [2000, 3000, 4000, 10, 2500, 2100]
    B, H = len(q_len), 2
    w = workloads.Workload("ragged-split", B, H, max(q_len), max(k_len), 128, 128, "bf16", False, 0.0, False, 12)
    q1, k1, q2, k2 = workloads.generate(w, cuda_device)
    print("ragged split elements", flush=True)
    kl, l1, l2 = sk.streamkl_fwd(q1, k1, q2, k2, False, q_len=q_len, k_len=k_len)
    for b, (nq, nk) in enumerate(zip(q_len, k_len)):
        if nq == 0:
            continue
        t = [x[b:b + 1, :, :n].contiguous() for x, n in ((q1, nq), (k1, nk), (q2, nq), (k2, nk))]
        if nq > 32:  # its own plan, as in the batch
            assert sk.fwd_plan(sk.shape_of(*t), False) > 1, "the case should split"
            rkl, rl1, rl2 = sk.streamkl_fwd(*t, False)
        else:  # the grouped decode plan: about 64 blocks of 32 keys per split, whole groups of 4
            blocks = -(-nk // 32)
            ns = min((-(-blocks // 64) + 3) // 4 * 4, max(1, blocks // 8), 4096)
            rkl, rl1, rl2 = sk.streamkl_fwd(*t, False, num_splits=ns)
        assert torch.equal(kl[b:b + 1, :, :nq], rkl), f"b{b}: KL differs from the element alone"
        assert torch.equal(l1[b:b + 1, :, :nq], rl1) and torch.equal(l2[b:b + 1, :, :nq], rl2)

    k_len = [2500, 2700, 3000, 2600, 2900, 2800]
    q_len = [16] * 6
    w = workloads.Workload("ragged-fallback", 6, H, 16, max(k_len), 128, 128, "bf16", False, 0.0, False, 13)
    q1, k1, q2, k2 = workloads.generate(w, cuda_device)
    shp = sk.shape_of(q1, k1, q2, k2).set_lengths(q_len, k_len)
    own = [sk.fwd_workspace_bytes(sk.make_shape(1, H, 16, nk, 128, 128, sk.BF16), False) for nk in k_len]
    need = sk.fwd_workspace_bytes(shp, False)
    assert need > max(own) + 256, (need, own)
    # through the C ABI: the binding would replace a workspace that is too small
    ws = torch.empty(need - 256, dtype=torch.uint8, device=cuda_device)
    ln = sk.Launch(0, 0, ws.data_ptr(), need - 256)
    kl, l1, l2 = (torch.full((6, H, 16), 7.0, device=cuda_device, dtype=torch.float32) for _ in range(3))
    st = sk.library().streamkl_fwd(q1.data_ptr(), k1.data_ptr(), q2.data_ptr(), k2.data_ptr(), 0, 0.0, 0.0,
                                   kl.data_ptr(), l1.data_ptr(), l2.data_ptr(), ctypes.byref(shp), ctypes.byref(ln),
                                   sk._stream(cuda_device))
    assert st == 0, st
    for b, nk in enumerate(k_len):
        t = [x[b:b + 1, :, :n].contiguous() for x, n in ((q1, 16), (k1, nk), (q2, 16), (k2, nk))]
        rkl, rl1, rl2 = sk.streamkl_fwd(*t, False)
        assert torch.equal(kl[b:b + 1], rkl), f"fallback b{b}: KL differs from the request alone"
        assert torch.equal(l1[b:b + 1], rl1) and torch.equal(l2[b:b + 1], rl2)
