"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Small shapes are compared element by element on every row; they span several
tiles (64-key forward tiles, 128-row workgroups) and ragged tails.  The named
workloads run at full size in the launch configuration the benchmark uses
and are compared on sampled heads and rows (and, under causal masks, on the
tail key rows whose dK the oracle can afford).
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from attention_kl_divergence_amd import streamkl as sk
from parity import check_forward_rows, check_grad, head_inputs, to_np

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)


def run_full(w, dev, g_kind="random", splits=(0,), modes=(sk.BWD_FUSED, sk.BWD_SEPARATE), settings=(1, 2)):
    q1, k1, q2, k2 = workloads.generate(w, dev)
    g = workloads.upstream_grad(w, dev, g_kind)
    outs = {}
    for sp in splits:
        _say(f"  fwd {w.name} splits={sp}")
        kl, l1, l2 = sk.streamkl_fwd(q1, k1, q2, k2, w.causal, num_splits=sp)
        torch.cuda.synchronize()
        outs[sp] = (to_np(kl), to_np(l1), to_np(l2))
    kl, l1, l2 = sk.streamkl_fwd(q1, k1, q2, k2, w.causal)
    grads = {}
    for s in settings:
        for m in modes:
            _say(f"  bwd {w.name} setting={s} mode={m}")
            dq, dk = sk.streamkl_bwd(s, q1, k1, q2, k2, w.causal, kl, l1, l2, g, bwd_mode=m)
            torch.cuda.synchronize()
            grads[(s, m)] = (to_np(dq), to_np(dk))
    gn = to_np(g)
    for b in range(w.B):
        for h in range(w.H):
            hi = head_inputs(q1, k1, q2, k2, b, h)
            ref = oracle.head_forward(*hi, w.causal)
            for sp, (okl, ol1, ol2) in outs.items():
                check_forward_rows(f"{w.name} b{b}h{h} sp{sp}", okl[b, h], ol1[b, h], ol2[b, h], ref, w.torch_dtype)
            for s in settings:
                rdq, rdk = oracle.head_backward(s, *hi, w.causal, gn[b, h])
                for m in modes:
                    dq, dk = grads[(s, m)]
                    check_grad(f"{w.name} b{b}h{h} s{s} m{m} dQ", dq[b, h], rdq)
                    check_grad(f"{w.name} b{b}h{h} s{s} m{m} dK", dk[b, h], rdk)
    return outs, grads


SMALL = [
    # name, dtype, d1, d2, causal, B, H, n_q, n_k
    ("f32-d64-nc", "f32", 64, 64, False, 1, 2, 200, 300),
    ("f32-d64-c", "f32", 64, 64, True, 1, 2, 200, 300),
    ("f32-d128-c", "f32", 128, 128, True, 2, 1, 129, 129),
    ("f32-d64x128-nc", "f32", 64, 128, False, 1, 1, 33, 65),
    ("bf16-d128-c", "bf16", 128, 128, True, 1, 2, 300, 300),
    ("bf16-d128-nc", "bf16", 128, 128, False, 1, 2, 257, 517),
    ("bf16-d128-c-rect", "bf16", 128, 128, True, 1, 2, 100, 333),
    ("bf16-d64-c", "bf16", 64, 64, True, 2, 2, 190, 190),
    ("bf16-d128x64-c", "bf16", 128, 64, True, 1, 2, 260, 260),
    ("bf16-d64x128-nc", "bf16", 64, 128, False, 1, 2, 70, 129),
    ("bf16-n1", "bf16", 128, 128, False, 1, 2, 1, 1),
    ("bf16-n17-c", "bf16", 128, 128, True, 1, 2, 17, 17),
    ("bf16-q1-k1000", "bf16", 128, 128, False, 1, 3, 1, 1000),
    ("bf16-d128-nc-tall", "bf16", 128, 128, False, 1, 2, 400, 130),
    ("f32-d128x64-nc-tall", "f32", 128, 64, False, 1, 1, 150, 40),
    # query ranges of at most 32 rows: the one-wave-per-split decode kernel
    ("bf16-dec-q16-k2000", "bf16", 128, 128, False, 1, 2, 16, 2000),
    ("bf16-dec-q32-k1500-c", "bf16", 128, 128, True, 1, 2, 32, 1500),
    ("bf16-dec-d128x64-q5-k777-c", "bf16", 128, 64, True, 1, 2, 5, 777),
    ("bf16-dec-d64x128-q31-k300", "bf16", 64, 128, False, 2, 1, 31, 300),
    # decode backward with several key tiles per workgroup: 8 workgroups per
    # head at 32 heads (5 tiles each, ragged tail), and one workgroup per head
    # at 256 heads (24 tiles, causal)
    ("bf16-dec-h32-q16-k5000", "bf16", 128, 128, False, 1, 32, 16, 5000),
    ("bf16-dec-b4h64-q7-k3000-c", "bf16", 128, 128, True, 4, 64, 7, 3000),
    # medium sizes, every row: several 256-key dK workgroups and 256-row dQ
    # workgroups, many query and key tiles (an odd count, a ragged last one)
    # and the causal frontier crossing workgroups, square and rectangular
    ("bf16-d128-c-1500", "bf16", 128, 128, True, 1, 2, 1500, 1500),
    ("bf16-d128x64-nc-1100x1700", "bf16", 128, 64, False, 1, 1, 1100, 1700),
    ("bf16-d64-c-700x2100", "bf16", 64, 64, True, 1, 2, 700, 2100),
]


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_small_shapes_full_parity(case, cuda_device):
    name, dt, d1, d2, causal, B, H, n_q, n_k = case
    w = workloads.Workload(name, B, H, n_q, n_k, d1, d2, dt, causal, 0.5, d1 != d2, 7)
    run_full(w, cuda_device, splits=(0, 1, 3))


@pytest.mark.parametrize("kind", ["mean", "random"])
def test_f32_512_workload_full(kind, cuda_device):
    """The fp32 H=1 N=512 d=64 non-causal workload: forward and setting-1 backward, every row."""
    w = workloads.WORKLOADS["h1-n512-d64-f32"]
    run_full(w, cuda_device, g_kind=kind, splits=(0, 1, 4))


# ----------------------------------------------------------------------------- full-size, sampled

def sample_rows(n, k=96, seed=0):
    r = np.random.default_rng(seed)
    extra = r.choice(n, size=min(k, n), replace=False)
    return np.unique(np.concatenate([[0, 1, n - 1], extra]).clip(0, n - 1))


def oracle_row_stats(hi, causal, block=64):
    """oracle.head_forward over every query row of one head, row blocks in
    parallel threads (BLAS one thread each), for checks that need the LSE of
    all rows."""
    import concurrent.futures as cf
    import os

    from threadpoolctl import threadpool_limits
    n_q = hi[0].shape[0]
    chunks = np.array_split(np.arange(n_q), max(1, n_q // 2048))
    with threadpool_limits(limits=1):
        with cf.ThreadPoolExecutor(max_workers=min(16, os.cpu_count() or 4)) as ex:
            parts = list(ex.map(lambda rows: oracle.head_forward(*hi, causal, rows=rows, block=block), chunks))
    return tuple(np.concatenate([p[i] for p in parts]) for i in range(3))


def run_sampled(w, dev, settings, heads=None, mode=sk.BWD_AUTO, dk_tail=2048, nrows=96, key_shift=0.0):
    _say(f"generate {w.name}")
    q1, k1, q2, k2 = workloads.generate(w, dev)
    if key_shift:
        # a component shared by every key (KL and the gradients do not change)
        k1, k2 = ((k.float() + key_shift).to(k.dtype) for k in (k1, k2))
    g = workloads.upstream_grad(w, dev, "random")
    _say(f"fwd {w.name}")
    kl, l1, l2 = sk.streamkl_fwd(q1, k1, q2, k2, w.causal)
    torch.cuda.synchronize()
    heads = heads or [0, w.H - 1]
    rows = sample_rows(w.n_q, nrows)
    block = max(16, (1 << 24) // w.n_k)
    grads = {}
    for s in settings:
        _say(f"bwd {w.name} setting {s} mode {mode} (plan {sk.bwd_plan(sk.shape_of(q1, k1, q2, k2), w.causal, s, mode)})")
        dq, dk = sk.streamkl_bwd(s, q1, k1, q2, k2, w.causal, kl, l1, l2, g, bwd_mode=mode)
        torch.cuda.synchronize()
        grads[s] = (dq, dk)
    for h in heads:
        hi = head_inputs(q1, k1, q2, k2, 0, h)
        gh = to_np(g[0, h])
        _say(f"oracle {w.name} head {h}: {len(rows)} rows")
        ref = oracle.head_forward(*hi, w.causal, rows=rows, block=block)
        check_forward_rows(f"{w.name} h{h}", to_np(kl[0, h])[rows], to_np(l1[0, h])[rows], to_np(l2[0, h])[rows],
                           ref, w.torch_dtype)
        for s in settings:
            dq, dk = grads[s]
            rdq, _ = oracle.head_backward(s, *hi, w.causal, gh, rows=rows, block=block)
            check_grad(f"{w.name} h{h} s{s} dQ rows", to_np(dq[0, h])[rows], rdq)
            if w.causal and dk_tail:
                keys = np.arange(w.n_k - dk_tail, w.n_k)
                _say(f"oracle {w.name} head {h}: dK tail {dk_tail}")
                rdk = oracle.head_backward_dk_rows(s, *hi, w.causal, gh, key_rows=keys, block=block)
                check_grad(f"{w.name} h{h} s{s} dK tail", to_np(dk[0, h])[keys], rdk)
            # every row of dS sums to zero, so the key-sum of dK vanishes up to
            # the bf16 rounding of dS
            dkh = dk[0, h].double()
            colsum = dkh.sum(dim=0).norm().item()
            _say(f"  |sum_j dK_j| / |dK| = {colsum / max(dkh.norm().item(), 1e-30):.3e}")
            assert colsum <= 1e-2 * dkh.norm().item(), f"{w.name} h{h} s{s}: |sum_j dK_j| = {colsum:.3e}"
    return kl, grads


def _tile_scaled_inputs(kind, n_q, n_k, d, seed, tile_rows):
    """Q near a common direction and K scaled per key tile of the forward
    (tile_rows keys): "rising" moves the row maxima of the logits up by about
    80 (base-2 units, default scale) per tile; "sinking" puts every logit near
    -270, where terms taken against an offset of 0 would all underflow."""
    r = np.random.default_rng(seed)
    q = 1.0 + 0.3 * r.standard_normal((n_q, d))
    k = 1.0 + 0.3 * r.standard_normal((n_k, d))
    tile = np.arange(n_k) // tile_rows
    unit = np.log2(np.e) * np.sqrt(d)  # base-2 logit of q . k per unit of key scale (q, k near all-ones)
    if kind == "rising":
        scale = (80.0 * tile + 1.0) / unit
    else:
        scale = (-290.0 + 1.0 * tile) / unit
    return q, k * scale[:, None]


# (dtype, head dim, key rows per forward tile of the long-range kernel)
FAR_CASES = [("bf16", 128, 128), ("f32", 64, 64)]


@pytest.mark.parametrize("dtype,d,tile_rows", FAR_CASES, ids=[f"{c[0]}-d{c[1]}" for c in FAR_CASES])
@pytest.mark.parametrize("kind", ["rising", "sinking"])
@pytest.mark.parametrize("causal", [False, True])
def test_forward_row_maxima_far_from_the_first_tile(kind, causal, dtype, d, tile_rows, cuda_device):
    """Logit maxima that move by hundreds (base 2) from one key tile to the
    next, or all far below 0: the forward kernels hold the offsets over
    later tiles and must raise them when a tile's terms pass their bound, and
    take the first tile's own maxima.  Every row against the oracle, the
    unsplit long-range form and the split form."""
    n_q, n_k, H = 512, 8 * tile_rows, 2  # eight key tiles
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    ins = []
    for h in range(H):
        q1, k1 = _tile_scaled_inputs(kind, n_q, n_k, d, 40 + h, tile_rows)
        q2, k2 = _tile_scaled_inputs(kind, n_q, n_k, d, 50 + h, tile_rows)
        ins.append((q1, 0.9 * k1, q2, k2))
    to = lambda i: torch.tensor(np.stack([x[i] for x in ins])[None], dtype=tdt,  # noqa: E731
                                device=cuda_device).contiguous()
    q1, k1, q2, k2 = (to(i) for i in range(4))
    for sp in (1, 0):
        _say(f"  fwd {kind} {dtype} d{d} causal={causal} splits={sp}")
        kl, l1, l2 = (to_np(t) for t in sk.streamkl_fwd(q1, k1, q2, k2, causal, num_splits=sp))
        for h in range(H):
            hi = head_inputs(q1, k1, q2, k2, 0, h)
            ref = oracle.head_forward(*hi, causal)
            assert np.isfinite(ref[0]).all()
            check_forward_rows(f"{kind} {dtype} c{int(causal)} sp{sp} h{h}", kl[0, h], l1[0, h], l2[0, h], ref, tdt)


def test_workload_8k_causal_both_settings(cuda_device):
    w = workloads.WORKLOADS["h32-n8k-d128-bf16-causal"]
    run_sampled(w, cuda_device, settings=(1, 2), heads=[0, 13, 31], nrows=256)


def test_workload_8k_causal_shifted_keys(cuda_device):
    """The 8K workload with 32 added to every key coordinate, both settings,
    separate mode: dQ stays within the 1e-2 bound (the bf16 rounding of dS
    meets K - kbar, not the shifted K)."""
    w = workloads.WORKLOADS["h32-n8k-d128-bf16-causal"]
    run_sampled(w, cuda_device, settings=(1, 2), heads=[0, 31], nrows=128, key_shift=32.0)


def test_workload_8k_causal_fused_mode(cuda_device):
    """The fused backward (dQ by fp32 atomics from the key-outer kernel) at a
    full workload size, both settings."""
    w = workloads.WORKLOADS["h32-n8k-d128-bf16-causal"]
    run_sampled(w, cuda_device, settings=(1, 2), heads=[0, 31], nrows=128, mode=sk.BWD_FUSED)


def test_workload_64k_causal_setting1(cuda_device):
    w = workloads.WORKLOADS["h32-n64k-d128-bf16-causal"]
    run_sampled(w, cuda_device, settings=(1,))


def test_workload_64k_noncausal_setting1(cuda_device):
    """The 64K non-causal workload: sampled rows of KL, LSE and dQ on two
    heads, and dK of 256 sampled keys (first, last and random ones) of head 0
    against the oracle over all 65536 query rows."""
    w = workloads.WORKLOADS["h32-n64k-d128-bf16"]
    _, grads = run_sampled(w, cuda_device, settings=(1,), dk_tail=0)
    q1, k1, q2, k2 = workloads.generate(w, cuda_device)
    g = workloads.upstream_grad(w, cuda_device, "random")
    hi = head_inputs(q1, k1, q2, k2, 0, 0)
    _say("oracle row statistics of head 0, all 65536 rows")
    stats = oracle_row_stats(hi, False)
    keys = sample_rows(w.n_k, 253, seed=3)
    _say(f"oracle dK of {len(keys)} keys over all rows")
    rdk = oracle.head_dk_keys(1, *hi, False, to_np(g[0, 0]), keys, stats, block=4096)
    dk = to_np(grads[1][1][0, 0])[keys]
    assert np.linalg.norm(dk) > 0
    check_grad(f"{w.name} h0 s1 dK sampled keys", dk, rdk)


@pytest.mark.parametrize("name", ["decode-h32-q1-k128k-d128-bf16", "decode-h32-q16-k128k-d128-bf16",
                                  "decode-h32-q1-k512k-d128-bf16", "decode-h32-q16-k512k-d128-bf16"])
def test_workload_decode_splitk(name, cuda_device):
    w = workloads.WORKLOADS[name]
    q1, k1, q2, k2 = workloads.generate(w, cuda_device)
    shp = sk.shape_of(q1, k1, q2, k2)
    plan = sk.fwd_plan(shp, False)
    _say(f"{name}: auto split plan {plan}")
    assert plan > 1
    res = {}
    for sp in (0, 1, 2, 7, 64):
        kl, l1, l2 = sk.streamkl_fwd(q1, k1, q2, k2, False, num_splits=sp)
        res[sp] = (to_np(kl), to_np(l1), to_np(l2))
    torch.cuda.synchronize()
    for h in (0, w.H - 1):
        hi = head_inputs(q1, k1, q2, k2, 0, h)
        ref = oracle.head_forward(*hi, False, block=16)
        for sp, (kl, l1, l2) in res.items():
            check_forward_rows(f"{name} h{h} sp{sp}", kl[0, h], l1[0, h], l2[0, h], ref, w.torch_dtype)
    # the split count changes only fp32 rounding
    for sp in (1, 2, 7, 64):
        assert np.abs(res[sp][0] - res[0][0]).max() < 1e-4


@pytest.mark.parametrize("name", ["decode-bwd-h32-q1-k512k-d128-bf16", "decode-bwd-h32-q16-k512k-d128-bf16"])
def test_workload_decode_backward(name, cuda_device):
    """Decode-shaped backward at full size, both settings, in the launch
    configuration the benchmark uses (the decode backward kernel: every key
    tile once, dQ summed per workgroup).  Two heads are compared with the
    oracle on every query row and every key's dK."""
    w = workloads.WORKLOADS[name]
    q1, k1, q2, k2 = workloads.generate(w, cuda_device)
    g = workloads.upstream_grad(w, cuda_device, "random")
    shp = sk.shape_of(q1, k1, q2, k2)
    kl, l1, l2 = sk.streamkl_fwd(q1, k1, q2, k2, w.causal)
    grads = {}
    for s in (1, 2):
        assert sk.bwd_plan(shp, w.causal, s) == sk.BWD_FUSED
        _say(f"bwd {name} setting {s}")
        dq, dk = sk.streamkl_bwd(s, q1, k1, q2, k2, w.causal, kl, l1, l2, g)
        torch.cuda.synchronize()
        grads[s] = (dq, dk)
    gn = to_np(g)
    for h in (0, w.H - 1):
        hi = head_inputs(q1, k1, q2, k2, 0, h)
        for s in (1, 2):
            _say(f"oracle {name} head {h} setting {s}")
            rdq, rdk = oracle.head_backward(s, *hi, w.causal, gn[0, h], block=16)
            check_grad(f"{name} h{h} s{s} dQ", to_np(grads[s][0][0, h]), rdq)
            check_grad(f"{name} h{h} s{s} dK", to_np(grads[s][1][0, h]), rdk)


def test_workload_512k_two_head_dims_setting2(cuda_device):
    w = workloads.WORKLOADS["h32-n512k-d128x64-bf16-causal"]
    run_sampled(w, cuda_device, settings=(2,), heads=[0, 31], nrows=64, dk_tail=1024)
