"""Ragged batches of many short sequences: grouped launches.

Where the elements of a ragged batch together fill the chip, the library
runs them unsplit in a few launches per kernel, each over a table of at most
64 elements, instead of one launch (or several) per element.  Each case has
more than 64 sequences, so every kernel runs several tables, and mixes
decode-shaped sequences (at most 32 query rows, which keep their own decode
kernels in the automatic backward), short and long ones and empty ones.

Every sequence must match the library's own call on its trimmed tensors with
the same kernels (the forward unsplit; the backward in separate mode; the
joint backward with its joint kernels): bitwise, except dK of a shared key
head, summed by atomics in no fixed order.  Padded rows are 0, the fused loss
agrees with the per-row KL it sums, and sampled sequences and heads are
checked against the fp64 oracle.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from attention_kl_divergence_amd import streamkl as sk
from parity import check_forward_rows, check_grad, to_np

pytestmark = pytest.mark.gpu

CASES = [
    # name, dtype, d1, d2, causal, H, kv1, kv2, B, seed
    ("bf16-c-d128-b80", "bf16", 128, 128, True, 8, 8, 8, 80, 1),
    ("bf16-nc-d128x64-gqa-b72", "bf16", 128, 64, False, 8, 2, 4, 72, 2),
    ("f32-c-d64-b70", "f32", 64, 64, True, 8, 8, 8, 70, 3),
]


def _lengths(B, causal, seed):
    r = np.random.default_rng(500 + seed)
    q_len, k_len = [], []
    for i in range(B):
        kind = i % 10
        k = int(r.integers(1, 33)) if kind == 0 else int(r.integers(40, 700))
        q = 0 if kind == 9 else (k if causal else int(r.integers(1, 700)))
        if kind == 1 and not causal:
            q = int(r.integers(1, 33))  # decode-shaped against a longer key range
        q_len.append(q)
        k_len.append(k)
    return q_len, k_len


def _decode_splits(q_len, k_len, dtype):
    """The key splits the library plans for the decode-shaped (bf16, at most
    32 query rows) sequences of a ragged batch that it groups: about 64
    blocks of 32 keys per split, in multiples of 4, at least 8 blocks per
    split (1: unsplit).  An element's own call with this split count runs the
    same arithmetic."""
    out = []
    for q, k in zip(q_len, k_len):
        b = -(-k // 32)
        dec = dtype == "bf16" and 0 < q <= 32
        out.append(min((-(-b // 64) + 3) // 4 * 4, max(1, b // 8), 4096) if dec else None)
    return out


def _inputs(case, dev):
    name, dt, d1, d2, causal, H, kv1, kv2, B, seed = case
    ql, kln = _lengths(B, causal, seed)
    n_q, n_k = max(ql), max(kln)
    w = workloads.Workload(name, B, H, n_q, n_k, d1, d2, dt, causal, 0.0, True, 40 + seed)
    q1, _, q2, _ = workloads.generate(w, dev)
    gen = torch.Generator(device=dev).manual_seed(77 + seed)
    k1 = torch.randn((B, kv1, n_k, d1), generator=gen, device=dev).to(w.torch_dtype)
    k2 = torch.randn((B, kv2, n_k, d2), generator=gen, device=dev).to(w.torch_dtype)
    return w, q1, k1, q2, k2, ql, kln


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_many_short_sequences(case, cuda_device):
    w, q1, k1, q2, k2, ql, kln = _inputs(case, cuda_device)
    B, H = w.B, w.H
    g1, g2 = H // k1.shape[1], H // k2.shape[1]
    lens = dict(q_len=ql, k_len=kln)
    # the grouped plan needs the unsplit workgroups to fill the chip
    assert sum(H * -(-q // 128) for q in ql if q > 32) >= 2 * 256
    g = workloads.upstream_grad(w, cuda_device, "random")
    weights = torch.rand((B, H, w.n_q), device=cuda_device)
    print(f"ragged many {w.name}", flush=True)
    kl, l1, l2 = sk.streamkl_fwd(q1, k1, q2, k2, w.causal, **lens)
    lkl, _, _, loss = sk.streamkl_fwd_loss(q1, k1, q2, k2, w.causal, weights, **lens)
    modes = (sk.BWD_AUTO, sk.BWD_SEPARATE)
    grads = {(s, m): sk.streamkl_bwd(s, q1, k1, q2, k2, w.causal, kl, l1, l2, g, bwd_mode=m, **lens)
             for s in (1, 2) for m in modes}
    joint = sk.streamkl_bwd_joint(q1, k1, q2, k2, w.causal, kl, l1, l2, g, bwd_mode=sk.BWD_SEPARATE, **lens)
    torch.cuda.synchronize()
    assert torch.equal(lkl, kl)
    ref_loss = sum((weights[b, :, :n].double() * kl[b, :, :n].double()).sum() for b, n in enumerate(ql))
    assert abs(loss.item() - ref_loss.item()) <= 1e-5 * abs(ref_loss.item()) + 1e-6

    dsplits = _decode_splits(ql, kln, w.dtype)
    for b in range(B):
        nq, nk = ql[b], kln[b]
        assert (kl[b, :, nq:] == 0).all() and (l1[b, :, nq:] == 0).all() and (l2[b, :, nq:] == 0).all()
        for dq, dk in list(grads.values()) + [joint[:2], joint[2:]]:
            assert (dq[b, :, nq:] == 0).all() and (dk[b, :, nk:] == 0).all()
            if nq == 0:
                assert (dq[b] == 0).all() and (dk[b] == 0).all()
        if nq == 0:
            continue
        t = [x[b:b + 1, :, :n].contiguous() for x, n in ((q1, nq), (k1, nk), (q2, nq), (k2, nk))]
        gt = g[b:b + 1, :, :nq].contiguous()
        # decode-shaped bf16 sequences take the batch's split plan; the rest run unsplit
        rkl, rl1, rl2 = sk.streamkl_fwd(*t, w.causal, num_splits=dsplits[b] or 1)
        assert torch.equal(kl[b:b + 1, :, :nq], rkl), f"{w.name} b{b}: KL differs from the element alone"
        assert torch.equal(l1[b:b + 1, :, :nq], rl1) and torch.equal(l2[b:b + 1, :, :nq], rl2)
        rj = sk.streamkl_bwd_joint(*t, w.causal, rkl, rl1, rl2, gt, bwd_mode=sk.BWD_SEPARATE)
        for s in (1, 2):
            shared = (g2 if s == 1 else g1) > 1
            rdq, rdk = sk.streamkl_bwd(s, *t, w.causal, rkl, rl1, rl2, gt, bwd_mode=sk.BWD_SEPARATE)
            jdq, jdk = rj[2:] if s == 1 else rj[:2]
            sep = grads[(s, sk.BWD_SEPARATE)]
            pairs = [(sep, (rdq, rdk)), ((joint[2:] if s == 1 else joint[:2]), (jdq, jdk))]
            for (dq, dk), (edq, edk) in pairs:
                assert torch.equal(dq[b:b + 1, :, :nq], edq), f"{w.name} b{b} s{s}: dQ differs from the element alone"
                if not shared:
                    assert torch.equal(dk[b:b + 1, :, :nk], edk), f"{w.name} b{b} s{s}: dK differs"
                else:
                    torch.testing.assert_close(dk[b:b + 1, :, :nk], edk, rtol=1e-5,
                                               atol=1e-6 * edk.abs().max().item())
    torch.cuda.synchronize()

    # the oracle on a few sequences: a decode-shaped one, a short and the
    # longest; the automatic backward (grouped separate kernels, or the
    # decode backward of a decode-shaped sequence) against it
    kl_n, l1n, l2n, gn = to_np(kl), to_np(l1), to_np(l2), to_np(g)
    picks = {0, 3, int(np.argmax(ql))}
    auto = {s: [to_np(t) for t in grads[(s, sk.BWD_AUTO)]] for s in (1, 2)}
    for b in sorted(picks):
        nq, nk = ql[b], kln[b]
        if nq == 0:
            continue
        ref_dk = {1: np.zeros((k2.shape[1], nk, w.d2)), 2: np.zeros((k1.shape[1], nk, w.d1))}
        ref_dq = {}
        for h in range(H):
            hi = [to_np(q1[b, h, :nq]), to_np(k1[b, h // g1, :nk]), to_np(q2[b, h, :nq]), to_np(k2[b, h // g2, :nk])]
            ref = oracle.head_forward(*hi, w.causal)
            check_forward_rows(f"{w.name} b{b}h{h}", kl_n[b, h, :nq], l1n[b, h, :nq], l2n[b, h, :nq], ref,
                               w.torch_dtype)
            for s in (1, 2):
                dq, dk = oracle.head_backward(s, *hi, w.causal, gn[b, h, :nq])
                ref_dq[(s, h)] = dq
                ref_dk[s][h // (g2 if s == 1 else g1)] += dk
        for s in (1, 2):
            dq, dk = auto[s]
            for h in range(H):
                check_grad(f"{w.name} b{b} s{s} auto h{h} dQ", dq[b, h, :nq], ref_dq[(s, h)])
            for kh in range(ref_dk[s].shape[0]):
                check_grad(f"{w.name} b{b} s{s} auto kh{kh} dK", dk[b, kh, :nk], ref_dk[s][kh])


DEC_CASES = [
    # name, d1, d2, causal, H, kv1, kv2, B, seed
    ("dec-bf16-nc-d128-b70", 128, 128, False, 8, 8, 8, 70, 4),
    ("dec-bf16-c-d128x64-gqa-b66", 128, 64, True, 8, 4, 2, 66, 5),
]


@pytest.mark.parametrize("case", DEC_CASES, ids=[c[0] for c in DEC_CASES])
def test_many_decode_sequences(case, cuda_device):
    """Batches of decode-shaped sequences (at most 32 query rows against key
    ranges of up to 3000 rows): the forward runs them in grouped split-K
    launches (the split partials of up to 64 sequences side by side, one
    merge launch), bitwise equal per sequence to its own call with the same
    split count; the automatic backward runs the decode backward over all of
    them in grouped launches.  Per sequence, dK equals
    the sequence's own call on its trimmed tensors bitwise (a key tile's dK is
    formed by one workgroup whatever the split count), except for shared key
    heads (atomics); dQ, added by atomics over a different split, agrees to
    fp32 rounding.  Sampled sequences are checked against the oracle."""
    name, d1, d2, causal, H, kv1, kv2, B, seed = case
    r = np.random.default_rng(900 + seed)
    q_len, k_len = [], []
    for i in range(B):
        k = int(r.integers(33, 3000))
        q = 0 if i % 11 == 10 else int(r.integers(1, 33))
        q_len.append(q)
        k_len.append(k)
    n_q, n_k = max(q_len), max(k_len)
    w = workloads.Workload(name, B, H, n_q, n_k, d1, d2, "bf16", causal, 0.0, True, 60 + seed)
    q1, _, q2, _ = workloads.generate(w, cuda_device)
    gen = torch.Generator(device=cuda_device).manual_seed(177 + seed)
    k1 = torch.randn((B, kv1, n_k, d1), generator=gen, device=cuda_device).to(torch.bfloat16)
    k2 = torch.randn((B, kv2, n_k, d2), generator=gen, device=cuda_device).to(torch.bfloat16)
    g1, g2 = H // kv1, H // kv2
    g = workloads.upstream_grad(w, cuda_device, "random")
    lens = dict(q_len=q_len, k_len=k_len)
    print(f"ragged decode {name}", flush=True)
    kl, l1, l2 = sk.streamkl_fwd(q1, k1, q2, k2, causal, **lens)
    weights = torch.rand((B, H, n_q), device=cuda_device)
    lkl, _, _, loss = sk.streamkl_fwd_loss(q1, k1, q2, k2, causal, weights, **lens)
    grads = {s: sk.streamkl_bwd(s, q1, k1, q2, k2, causal, kl, l1, l2, g, **lens) for s in (1, 2)}
    torch.cuda.synchronize()
    assert torch.equal(lkl, kl)
    ref_loss = sum((weights[b, :, :n].double() * kl[b, :, :n].double()).sum() for b, n in enumerate(q_len))
    assert abs(loss.item() - ref_loss.item()) <= 1e-5 * abs(ref_loss.item()) + 1e-6
    dsplits = _decode_splits(q_len, k_len, "bf16")
    for b in range(B):
        nq, nk = q_len[b], k_len[b]
        for s in (1, 2):
            dq, dk = grads[s]
            assert (dq[b, :, nq:] == 0).all() and (dk[b, :, nk:] == 0).all()
            if nq == 0:
                assert (dq[b] == 0).all() and (dk[b] == 0).all()
        if nq == 0:
            continue
        t = [x[b:b + 1, :, :n].contiguous() for x, n in ((q1, nq), (k1, nk), (q2, nq), (k2, nk))]
        gt = g[b:b + 1, :, :nq].contiguous()
        rkl, rl1, rl2 = sk.streamkl_fwd(*t, causal, num_splits=dsplits[b])
        assert torch.equal(kl[b:b + 1, :, :nq], rkl), f"{name} b{b}: KL differs from the element alone"
        assert torch.equal(l1[b:b + 1, :, :nq], rl1) and torch.equal(l2[b:b + 1, :, :nq], rl2)
        for s in (1, 2):
            rdq, rdk = sk.streamkl_bwd(s, *t, causal, rkl, rl1, rl2, gt)
            dq, dk = grads[s]
            edq = dq[b:b + 1, :, :nq]
            err = ((edq - rdq).norm() / rdq.norm().clamp_min(1e-30)).item()
            assert err <= 1e-5, f"{name} b{b} s{s}: dQ relative L2 {err:.3e} against the element alone"
            if (g2 if s == 1 else g1) == 1:
                assert torch.equal(dk[b:b + 1, :, :nk], rdk), f"{name} b{b} s{s}: dK differs from the element alone"
            else:
                torch.testing.assert_close(dk[b:b + 1, :, :nk], rdk, rtol=1e-5, atol=1e-6 * rdk.abs().max().item())
    torch.cuda.synchronize()
    kl_n, l1n, l2n, gn = to_np(kl), to_np(l1), to_np(l2), to_np(g)
    auto = {s: [to_np(t) for t in grads[s]] for s in (1, 2)}
    for b in (0, int(np.argmax(k_len))):
        nq, nk = q_len[b], k_len[b]
        if nq == 0:
            continue
        ref_dk = {1: np.zeros((kv2, nk, d2)), 2: np.zeros((kv1, nk, d1))}
        ref_dq = {}
        for h in range(H):
            hi = [to_np(q1[b, h, :nq]), to_np(k1[b, h // g1, :nk]), to_np(q2[b, h, :nq]), to_np(k2[b, h // g2, :nk])]
            ref = oracle.head_forward(*hi, causal)
            check_forward_rows(f"{name} b{b}h{h}", kl_n[b, h, :nq], l1n[b, h, :nq], l2n[b, h, :nq], ref,
                               torch.bfloat16)
            for s in (1, 2):
                rdq, rdk = oracle.head_backward(s, *hi, causal, gn[b, h, :nq])
                ref_dq[(s, h)] = rdq
                ref_dk[s][h // (g2 if s == 1 else g1)] += rdk
        for s in (1, 2):
            dq, dk = auto[s]
            for h in range(H):
                check_grad(f"{name} b{b} s{s} h{h} dQ", dq[b, h, :nq], ref_dq[(s, h)])
            for kh in range(ref_dk[s].shape[0]):
                check_grad(f"{name} b{b} s{s} kh{kh} dK", dk[b, kh, :nk], ref_dk[s][kh])
