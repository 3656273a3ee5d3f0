"""The allocation-free forward (streamkl_fwd_loss_noalloc) against the entry
point it is a variant of (streamkl_fwd_loss with a caller workspace),
through the C ABI: two calls in a row, the second with a smaller input,
then the plain forward through it, then a request too large for its scratch."""
import ctypes

import numpy as np
import pytest
import torch

import workloads
from attention_kl_divergence_amd import streamkl as sk

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)


def _lib():
    lib = sk.library()
    vp, i32, f32 = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    lib.streamkl_fwd_loss_noalloc.argtypes = [vp, vp, vp, vp, i32, f32, f32, vp, vp, vp, vp, vp,
                                              ctypes.POINTER(sk.Shape), ctypes.POINTER(sk.Launch), vp]
    lib.streamkl_fwd_loss_noalloc.restype = i32
    return lib


def _ptr(t):
    return t.data_ptr() if t is not None else None


def _outs(w, dev, fill=7.0):
    f32 = dict(device=dev, dtype=torch.float32)
    return tuple(torch.full((w.B, w.H, w.n_q), fill, **f32) for _ in range(3)) + (torch.full((), fill, **f32),)


def _noalloc(lib, q1, k1, q2, k2, causal, weights, out, num_splits=0, with_loss=True, shp=None):
    shp = sk.shape_of(q1, k1, q2, k2) if shp is None else shp
    ln = sk.Launch(num_splits, 0, None, 0)
    return lib.streamkl_fwd_loss_noalloc(_ptr(q1), _ptr(k1), _ptr(q2), _ptr(k2), int(causal), 0.0, 0.0,
                                         _ptr(weights), *(_ptr(t) for t in out[:3]),
                                         _ptr(out[3]) if with_loss else None, ctypes.byref(shp), ctypes.byref(ln),
                                         sk._stream(q1.device))


def test_noalloc_matches_workspace_entry_point(cuda_device):
    lib = _lib()
    # a split-K decode shape (split partials and loss partials in the scratch),
    # then a smaller unsplit shape, then a split shape with weights
    cases = [
        workloads.Workload("na-dec", 1, 32, 16, 20000, 128, 128, "bf16", False, 0.5, False, 21),
        workloads.Workload("na-small", 1, 2, 100, 300, 64, 64, "f32", True, 0.5, False, 22),
        workloads.Workload("na-split", 1, 3, 200, 5000, 128, 64, "bf16", False, 0.5, True, 23),
    ]
    for i, w in enumerate(cases):
        q1, k1, q2, k2 = workloads.generate(w, cuda_device)
        wt = workloads.upstream_grad(w, cuda_device, "random") if i == 2 else None
        shp = sk.shape_of(q1, k1, q2, k2)
        _say(f"call {i}: {w.name} splits {sk.fwd_plan(shp, w.causal)}")
        ref = sk.streamkl_fwd_loss(q1, k1, q2, k2, w.causal, wt)
        out = _outs(w, cuda_device)
        torch.cuda.synchronize()
        # free device memory around the call alone (every tensor exists already)
        free0 = torch.cuda.mem_get_info(cuda_device)[0]
        assert _noalloc(lib, q1, k1, q2, k2, w.causal, wt, out) == sk.OK
        torch.cuda.synchronize()
        assert torch.cuda.mem_get_info(cuda_device)[0] == free0, f"{w.name}: the call changed free device memory"
        for a, b, n in zip(out, ref, ("kl", "lse1", "lse2", "loss")):
            assert torch.equal(a, b), f"{w.name}: {n} differs from streamkl_fwd_loss"
    # the plain forward through it (no loss): the same rows as streamkl_fwd
    w = cases[0]
    q1, k1, q2, k2 = workloads.generate(w, cuda_device)
    out = _outs(w, cuda_device)
    assert _noalloc(lib, q1, k1, q2, k2, False, None, out, with_loss=False) == sk.OK
    kl, l1, l2 = sk.streamkl_fwd(q1, k1, q2, k2, False)
    torch.cuda.synchronize()
    assert torch.equal(out[0], kl) and torch.equal(out[1], l1) and torch.equal(out[2], l2)
    assert (out[3] == 7.0).all()  # no loss requested: not written


def test_noalloc_rejects_requests_beyond_its_scratch(cuda_device):
    """An explicit split count whose partials exceed the 4 MiB scratch returns
    STREAMKL_ERR_WORKSPACE and writes nothing; an automatic one falls back."""
    lib = _lib()
    w = workloads.Workload("na-big", 1, 32, 32, 100000, 128, 128, "bf16", False, 0.5, False, 24)
    q1, k1, q2, k2 = workloads.generate(w, cuda_device)
    out = _outs(w, cuda_device)
    splits = 2048  # 20 B * 32 heads * 32 rows * 2048 splits = 40 MiB of partials
    assert _noalloc(lib, q1, k1, q2, k2, False, None, out, num_splits=splits) == sk.ERR_WORKSPACE
    torch.cuda.synchronize()
    assert all((t == 7.0).all() for t in out)
    assert _noalloc(lib, q1, k1, q2, k2, False, None, out) == sk.OK
    ref = sk.streamkl_fwd_loss(q1, k1, q2, k2, False)
    torch.cuda.synchronize()
    for a, b in zip(out, ref):
        assert torch.equal(a, b)


def test_noalloc_ragged_batches(cuda_device):
    """A ragged batch of decode-shaped requests (grouped split-K partials in
    the scratch), longer query ranges and an empty element, padded and
    packed: every output equal to streamkl_fwd_loss with a workspace, padded
    rows cleared over earlier contents."""
    lib = _lib()
    q_len = [16, 1, 0, 200, 9, 32, 64, 5]
    k_len = [3000, 700, 40, 900, 5000, 2048, 2500, 64]
    B, H = len(q_len), 8
    w = workloads.Workload("na-ragged", B, H, max(q_len), max(k_len), 128, 128, "bf16", False, 0.5, False, 25)
    q1, k1, q2, k2 = workloads.generate(w, cuda_device)
    wt = torch.rand((B, H, w.n_q), device=cuda_device)

    def pack(t, lens):
        return torch.cat([t[b, :, :n] for b, n in enumerate(lens)], dim=1).contiguous()

    qo, ko = [0, *np.cumsum(q_len).tolist()], [0, *np.cumsum(k_len).tolist()]
    P = [pack(t, n) for t, n in zip((q1, k1, q2, k2), (q_len, k_len, q_len, k_len))]
    layouts = [("padded", (q1, k1, q2, k2), wt, sk.shape_of(q1, k1, q2, k2).set_lengths(q_len, k_len),
                dict(q_len=q_len, k_len=k_len)),
               ("packed", P, pack(wt, q_len), sk.packed_shape_of(*P, qo, ko), dict(q_off=qo, k_off=ko))]
    for name, t, wts, shp, kw in layouts:
        _say(f"ragged {name}: fwd plan {sk.fwd_plan(shp, False)}")
        ref = sk.streamkl_fwd_loss(*t, False, wts, **kw)
        out = tuple(torch.full_like(r, 7.0) for r in ref)
        assert _noalloc(lib, *t, False, wts, out, shp=shp) == sk.OK
        torch.cuda.synchronize()
        for a, b, n in zip(out, ref, ("kl", "lse1", "lse2", "loss")):
            assert torch.equal(a, b), f"{name}: {n} differs from streamkl_fwd_loss"


def test_noalloc_under_graph_capture(cuda_device):
    """The allocation-free forward captured in a HIP graph (split-K decode
    partials and loss partials in its static scratch): three replays, the
    inputs rewritten in place by eager work before each, every output
    bitwise equal to streamkl_fwd_loss run eagerly on the same inputs."""
    lib = _lib()
    w = workloads.Workload("na-graph", 1, 16, 16, 12000, 128, 128, "bf16", False, 0.5, True, 26)
    q1, k1, q2, k2 = workloads.generate(w, cuda_device)
    wt = workloads.upstream_grad(w, cuda_device, "random")
    out = _outs(w, cuda_device)
    _say(f"graph {w.name} splits {sk.fwd_plan(sk.shape_of(q1, k1, q2, k2), w.causal)}")
    # warm up on a side stream, then capture
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        assert _noalloc(lib, q1, k1, q2, k2, w.causal, wt, out) == sk.OK
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        assert _noalloc(lib, q1, k1, q2, k2, w.causal, wt, out) == sk.OK
    gen = torch.Generator(device=cuda_device)
    for r in range(3):
        gen.manual_seed(2000 + r)
        for t in (q1, k1, q2, k2):
            t.copy_(torch.randn(t.shape, generator=gen, device=cuda_device).to(t.dtype))
        graph.replay()
        torch.cuda.synchronize()
        got = [t.clone() for t in out]
        ref = sk.streamkl_fwd_loss(q1, k1, q2, k2, w.causal, wt)
        torch.cuda.synchronize()
        for a, b, n in zip(got, ref, ("kl", "lse1", "lse2", "loss")):
            assert torch.equal(a, b), f"replay {r}: {n} differs from the eager streamkl_fwd_loss"
    del graph
