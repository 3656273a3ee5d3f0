"""The library's calls under HIP graph capture.

Every entry point only enqueues kernels on the caller's stream (no host
synchronisation, no device allocation, no memset nodes: buffers that must
start at zero are cleared by a fill kernel), so a training step can be
captured once and replayed.  Each test captures a step, then replays it
three times; before each replay the inputs are rewritten in place by eager
work on the same stream, and after it the replay's outputs are compared with
an eager run of the same step on the same inputs.  The forward, the fused
loss and the separate-mode backward are deterministic, so they must match
bit for bit; the fused-mode backward adds dQ with atomics in no fixed order
and is compared at fp32 rounding.
"""
import pytest
import torch

import workloads
from attention_kl_divergence_amd import streamkl as sk

pytestmark = pytest.mark.gpu


def _capture(step):
    """Warm up on a side stream, then capture step() into a graph."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        outs = step()
    return graph, outs


def _replays(w, step, inputs, exact, rtol=0.0):
    graph, outs = _capture(step)
    gen = torch.Generator(device=inputs[0].device)
    for r in range(3):
        gen.manual_seed(1000 + r)
        for t in inputs:  # new inputs, written in place by eager work
            t.copy_(torch.randn(t.shape, generator=gen, device=t.device).to(t.dtype))
        graph.replay()
        torch.cuda.synchronize()
        got = [o.clone() for o in outs]
        ref = step()
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(got, ref)):
            assert torch.isfinite(a).all(), f"{w.name} replay {r} output {i} not finite"
            if exact[i]:
                assert torch.equal(a, b), f"{w.name} replay {r} output {i} differs from the eager run"
            else:
                err = ((a - b).norm() / b.norm().clamp_min(1e-30)).item()
                assert err <= rtol, f"{w.name} replay {r} output {i}: relative L2 {err:.3e}"
    del graph


@pytest.mark.parametrize("mode", [sk.BWD_SEPARATE, sk.BWD_FUSED])
def test_captured_step_matches_eager(mode, cuda_device):
    w = workloads.Workload("graph-step", 1, 4, 700, 700, 128, 128, "bf16", True, 0.5, False, 3)
    print(w.name, mode, flush=True)
    q1, k1, q2, k2 = workloads.generate(w, cuda_device)
    g = workloads.upstream_grad(w, cuda_device, "random")
    weights = torch.rand((w.B, w.H, w.n_q), device=cuda_device)

    def step():
        kl, l1, l2, loss = sk.streamkl_fwd_loss(q1, k1, q2, k2, True, weights)
        dq, dk = sk.streamkl_bwd(1, q1, k1, q2, k2, True, kl, l1, l2, g, bwd_mode=mode)
        return kl, l1, l2, loss, dq, dk

    fused = mode == sk.BWD_FUSED
    _replays(w, step, (q1, k1, q2, k2, g), exact=(True, True, True, True, not fused, True), rtol=1e-5)


def test_captured_decode_split_forward_and_backward(cuda_device):
    # 16 query rows against 3000 keys: the split-K forward (workspace from the
    # binding, merge kernel) and the decode backward
    w = workloads.Workload("graph-decode", 1, 8, 16, 3000, 128, 128, "bf16", False, 0.5, False, 4)
    print(w.name, flush=True)
    q1, k1, q2, k2 = workloads.generate(w, cuda_device)
    g = workloads.upstream_grad(w, cuda_device, "random")

    def step():
        kl, l1, l2 = sk.streamkl_fwd(q1, k1, q2, k2, False, num_splits=4)
        dq, dk = sk.streamkl_bwd(1, q1, k1, q2, k2, False, kl, l1, l2, g)
        return kl, l1, l2, dq, dk

    # the decode backward adds its per-wave dQ partials with atomics
    _replays(w, step, (q1, k1, q2, k2, g), exact=(True, True, True, False, True), rtol=1e-5)


def test_captured_grouped_heads_backward(cuda_device):
    # dK of shared key heads is summed with atomics into an output the library
    # clears first with a fill kernel (no memset node in the graph)
    w = workloads.Workload("graph-gqa", 1, 8, 300, 300, 128, 128, "bf16", True, 0.0, True, 5)
    print(w.name, flush=True)
    q1, _, q2, _ = workloads.generate(w, cuda_device)
    gen = torch.Generator(device=cuda_device).manual_seed(9)
    k1 = torch.randn((1, 2, w.n_k, 128), generator=gen, device=cuda_device).to(torch.bfloat16)
    k2 = torch.randn((1, 4, w.n_k, 128), generator=gen, device=cuda_device).to(torch.bfloat16)
    g = workloads.upstream_grad(w, cuda_device, "random")

    def step():
        kl, l1, l2 = sk.streamkl_fwd(q1, k1, q2, k2, True)
        dq, dk = sk.streamkl_bwd(1, q1, k1, q2, k2, True, kl, l1, l2, g, bwd_mode=sk.BWD_SEPARATE)
        return kl, dq, dk

    _replays(w, step, (q1, k1, q2, k2, g), exact=(True, True, False), rtol=1e-5)


def test_captured_ragged_grouped_step(cuda_device):
    # 70 short sequences: the forward and both backward settings run as
    # grouped launches over tables of up to 64 elements, and the padded rows
    # are cleared by the span-fill kernel
    import numpy as np
    r = np.random.default_rng(12)
    lens = [0 if i % 9 == 8 else int(r.integers(40, 600)) for i in range(70)]
    n = max(lens)
    w = workloads.Workload("graph-ragged", len(lens), 8, n, n, 128, 128, "bf16", True, 0.5, False, 6)
    print(w.name, flush=True)
    q1, k1, q2, k2 = workloads.generate(w, cuda_device)
    g = workloads.upstream_grad(w, cuda_device, "random")
    weights = torch.rand((w.B, w.H, w.n_q), device=cuda_device)
    lk = dict(q_len=lens, k_len=lens)

    def step():
        kl, l1, l2, loss = sk.streamkl_fwd_loss(q1, k1, q2, k2, True, weights, **lk)
        dq, dk = sk.streamkl_bwd(1, q1, k1, q2, k2, True, kl, l1, l2, g, bwd_mode=sk.BWD_SEPARATE, **lk)
        dq1, dk1, dq2, dk2 = sk.streamkl_bwd_joint(q1, k1, q2, k2, True, kl, l1, l2, g, **lk)
        return kl, l1, l2, loss, dq, dk, dq1, dk1, dq2, dk2

    _replays(w, step, (q1, k1, q2, k2, g), exact=(True,) * 10)


def test_captured_ragged_decode_step(cuda_device):
    # 40 decode-shaped requests (1-32 query rows, 300-5000 keys): grouped
    # split-K forward with its merge and the grouped decode backward
    import numpy as np
    r = np.random.default_rng(13)
    q_len = [int(r.integers(1, 33)) for _ in range(40)]
    k_len = [int(r.integers(300, 5000)) for _ in range(40)]
    w = workloads.Workload("graph-ragged-decode", 40, 8, max(q_len), max(k_len), 128, 128, "bf16", False, 0.5,
                           False, 7)
    print(w.name, flush=True)
    q1, k1, q2, k2 = workloads.generate(w, cuda_device)
    g = workloads.upstream_grad(w, cuda_device, "random")
    lk = dict(q_len=q_len, k_len=k_len)

    def step():
        kl, l1, l2 = sk.streamkl_fwd(q1, k1, q2, k2, False, **lk)
        dq, dk = sk.streamkl_bwd(1, q1, k1, q2, k2, False, kl, l1, l2, g, **lk)
        return kl, l1, l2, dq, dk

    # the decode backward adds its dQ partials with atomics
    _replays(w, step, (q1, k1, q2, k2, g), exact=(True, True, True, False, True), rtol=1e-5)


def test_captured_packed_step(cuda_device):
    # a packed batch (sequences one after another, row offsets): 50 causal
    # sequences of 30-500 rows and, in a second batch, 30 decode-shaped
    # requests; forward with the loss, the separate and the automatic backward
    import numpy as np
    r = np.random.default_rng(14)
    for causal, q_len, k_len in (
            (True, *(2 * [[int(r.integers(30, 500)) for _ in range(50)]])),
            (False, [int(r.integers(1, 33)) for _ in range(30)], [int(r.integers(300, 4000)) for _ in range(30)])):
        qo, ko = [0, *np.cumsum(q_len).tolist()], [0, *np.cumsum(k_len).tolist()]
        H, nq, nk = 8, qo[-1], ko[-1]
        name = f"graph-packed-{'causal' if causal else 'decode'}"
        print(name, flush=True)
        gen = torch.Generator(device=cuda_device).manual_seed(15)
        q1, q2 = (torch.randn((H, nq, 128), generator=gen, device=cuda_device).to(torch.bfloat16) for _ in range(2))
        k1, k2 = (torch.randn((H, nk, 128), generator=gen, device=cuda_device).to(torch.bfloat16) for _ in range(2))
        g = torch.randn((H, nq), generator=gen, device=cuda_device) / 100
        weights = torch.rand((H, nq), device=cuda_device)
        lk = dict(q_off=qo, k_off=ko)

        def step():
            kl, l1, l2, loss = sk.streamkl_fwd_loss(q1, k1, q2, k2, causal, weights, **lk)
            dq, dk = sk.streamkl_bwd(1, q1, k1, q2, k2, causal, kl, l1, l2, g, bwd_mode=sk.BWD_SEPARATE, **lk)
            dqa, dka = sk.streamkl_bwd(2, q1, k1, q2, k2, causal, kl, l1, l2, g, **lk)
            return kl, l1, l2, loss, dq, dk, dqa, dka

        # the automatic backward may add dQ with atomics (decode-shaped or
        # fused elements)
        w = workloads.Workload(name, len(q_len), H, nq, nk, 128, 128, "bf16", causal, 0.5, False, 8)
        _replays(w, step, (q1, k1, q2, k2, g), exact=(True,) * 6 + (False, True), rtol=1e-5)
