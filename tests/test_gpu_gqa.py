"""GPU parity with grouped key heads: K_t holds kv_heads_t heads and query
head h reads key head h / (H / kv_heads_t); dK_t of a key head is the sum over
the query heads that share it.

Checked against the fp64 oracle per query head (each with its own key head)
and against the library's own ungrouped path on K repeated per query head:
the forward and dQ are then the same arithmetic (bitwise equal), and the
grouped dK equals the per-group sum of the ungrouped dK.
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
    # name, dtype, d1, d2, causal, H, kv1, kv2, n_q, n_k
    ("bf16-c-g4g2", "bf16", 128, 128, True, 8, 2, 4, 200, 260),
    ("bf16-nc-d128x64-g8g1", "bf16", 128, 64, False, 8, 1, 8, 130, 300),
    ("f32-c-g2g4", "f32", 64, 128, True, 8, 4, 2, 90, 90),
    ("bf16-dec-q16-g4g4", "bf16", 128, 128, False, 8, 2, 2, 16, 3000),
    ("bf16-dec-q5-c-g2g8", "bf16", 64, 128, True, 8, 4, 1, 5, 700),
]


def _inputs(case, dev):
    name, dt, d1, d2, causal, H, kv1, kv2, n_q, n_k = case
    w = workloads.Workload(name, 1, H, n_q, n_k, d1, d2, dt, causal, 0.0, True, 21)
    q1, _, q2, _ = workloads.generate(w, dev)
    gen = torch.Generator(device=dev).manual_seed(77)
    k1 = torch.randn((1, kv1, n_k, d1), generator=gen, device=dev).to(w.torch_dtype)
    k2 = torch.randn((1, kv2, n_k, d2), generator=gen, device=dev).to(w.torch_dtype)
    return w, q1, k1, q2, k2


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_grouped_key_heads(case, cuda_device):
    w, q1, k1, q2, k2 = _inputs(case, cuda_device)
    H, kv1, kv2 = w.H, k1.shape[1], k2.shape[1]
    g1, g2 = H // kv1, H // kv2
    shp = sk.shape_of(q1, k1, q2, k2)
    assert (shp.kv_heads1, shp.kv_heads2) == ((kv1 if kv1 < H else 0), (kv2 if kv2 < H else 0))
    g = workloads.upstream_grad(w, cuda_device, "random")
    print(f"gqa {w.name}", flush=True)
    kl, l1, l2 = sk.streamkl_fwd(q1, k1, q2, k2, w.causal)
    grads = {}
    for s in (1, 2):
        for m in (sk.BWD_FUSED, sk.BWD_SEPARATE):
            grads[(s, m)] = [to_np(t) for t in sk.streamkl_bwd(s, q1, k1, q2, k2, w.causal, kl, l1, l2, g, bwd_mode=m)]
    joint = [to_np(t) for t in sk.streamkl_bwd_joint(q1, k1, q2, k2, w.causal, kl, l1, l2, g)]
    torch.cuda.synchronize()

    # the ungrouped path on K repeated per query head
    k1r = k1.repeat_interleave(g1, dim=1).contiguous()
    k2r = k2.repeat_interleave(g2, dim=1).contiguous()
    rkl, rl1, rl2 = sk.streamkl_fwd(q1, k1r, q2, k2r, w.causal)
    assert torch.equal(kl, rkl) and torch.equal(l1, rl1) and torch.equal(l2, rl2)
    for s in (1, 2):
        gs = g2 if s == 1 else g1
        rdq, rdk = sk.streamkl_bwd(s, q1, k1r, q2, k2r, w.causal, kl, l1, l2, g, bwd_mode=sk.BWD_SEPARATE)
        dq, dk = grads[(s, sk.BWD_SEPARATE)]
        np.testing.assert_array_equal(dq, to_np(rdq))
        rsum = to_np(rdk).reshape(1, H // gs, gs, w.n_k, -1).sum(axis=2)
        np.testing.assert_allclose(dk, rsum, rtol=1e-5, atol=1e-6 * np.abs(rsum).max())

    # the oracle, per query head with its key head; dK summed per key head
    gn = to_np(g)
    ref_dk = {1: np.zeros((kv2, w.n_k, w.d2)), 2: np.zeros((kv1, w.n_k, w.d1))}
    ref_dq = {}
    for h in range(H):
        hi = [to_np(q1[0, h]), to_np(k1[0, h // g1]), to_np(q2[0, h]), to_np(k2[0, h // g2])]
        ref = oracle.head_forward(*hi, w.causal)
        check_forward_rows(f"{w.name} h{h}", to_np(kl[0, h]), to_np(l1[0, h]), to_np(l2[0, h]), ref, w.torch_dtype)
        for s in (1, 2):
            dq, dk = oracle.head_backward(s, *hi, w.causal, gn[0, h])
            ref_dq[(s, h)] = dq
            ref_dk[s][h // (g2 if s == 1 else g1)] += dk
    for s in (1, 2):
        outs = [grads[(s, m)] for m in (sk.BWD_FUSED, sk.BWD_SEPARATE)]
        outs.append(joint[2:] if s == 1 else joint[:2])
        for i, (dq, dk) in enumerate(outs):
            for h in range(H):
                check_grad(f"{w.name} s{s} out{i} h{h} dQ", dq[0, h], ref_dq[(s, h)])
            for kh in range(ref_dk[s].shape[0]):
                check_grad(f"{w.name} s{s} out{i} key head {kh} dK", dk[0, kh], ref_dk[s][kh])


def test_grouped_key_heads_64k_workload(cuda_device):
    """The 64K causal workload with 32 query heads on 8 key heads, in the
    configuration the benchmark times: sampled query rows (forward, dQ) of
    two query heads, and the last 1024 keys' dK of two key heads summed over
    their four query heads, against the oracle."""
    w = workloads.WORKLOADS["h32-kv8-n64k-d128-bf16-causal"]
    q1, k1, q2, k2 = workloads.generate(w, cuda_device)
    G = w.H // w.kv_heads
    g = workloads.upstream_grad(w, cuda_device, "random")
    print("gqa 64k forward", flush=True)
    kl, l1, l2 = sk.streamkl_fwd(q1, k1, q2, k2, True)
    print("gqa 64k backward", flush=True)
    dq, dk = sk.streamkl_bwd(1, q1, k1, q2, k2, True, kl, l1, l2, g)
    torch.cuda.synchronize()
    rng = np.random.default_rng(5)
    rows = np.unique(np.concatenate([[0, 1, w.n_q - 1], rng.choice(w.n_q, 61, replace=False)]))
    keys = np.arange(w.n_k - 1024, w.n_k)
    gn = to_np(g)
    hin = lambda h: [to_np(q1[0, h]), to_np(k1[0, h // G]), to_np(q2[0, h]), to_np(k2[0, h // G])]  # noqa: E731
    for h in (0, 31):
        print(f"oracle head {h}", flush=True)
        ref = oracle.head_forward(*hin(h), True, rows=rows, block=64)
        check_forward_rows(f"64k gqa h{h}", to_np(kl[0, h])[rows], to_np(l1[0, h])[rows], to_np(l2[0, h])[rows],
                           ref, w.torch_dtype)
        rdq, _ = oracle.head_backward(1, *hin(h), True, gn[0, h], rows=rows, block=64)
        check_grad(f"64k gqa h{h} dQ rows", to_np(dq[0, h])[rows], rdq)
    for kh in (0, w.kv_heads - 1):
        print(f"oracle key head {kh}", flush=True)
        rdk = sum(oracle.head_backward_dk_rows(1, *hin(h), True, gn[0, h], key_rows=keys, block=128)
                  for h in range(kh * G, (kh + 1) * G))
        check_grad(f"64k gqa key head {kh} dK tail", to_np(dk[0, kh])[keys], rdk)
