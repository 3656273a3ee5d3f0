"""Benchmark of the attention-KL hot path on one MI355X.

One step = the StreamKL forward (KL, LSE1, LSE2) plus the setting-1
backward (dQ2, dK2) over one batch of synthetic inputs already resident in
HBM.  Default workload: B=1, H=32, N_Q=N_K=65536, d=128, bf16, causal.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

Prints ONE JSON line.  `value` is algorithmic TFLOP/s of the whole step:
forward 2(d1+d2) and setting-1 backward 2(d1+d2)+4*d2 FLOPs per visible
(query, key) pair; recomputation and masked-tile waste are not credited.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 matrix peak
MFMA_F32_PEAK_TFLOPS = 157.3     # MI355X dense fp32 matrix peak
HBM_PEAK_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="h32-n64k-d128-bf16-causal")
    ap.add_argument("--bwd-mode", default="auto", choices=["auto", "fused", "separate"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--joint", action="store_true",
                    help="for workloads that train both models (settings 1 and 2), run the joint backward "
                         "(one key-outer pass for dK1 and dK2, then dQ1 and dQ2) instead of two backward calls")
    ap.add_argument("--cpu-rows", type=int, default=6144, help="query rows of the oracle sample")
    ap.add_argument("--compare-modes", action="store_true",
                    help="after the timed steps, time each backward setting once in the mode the plan "
                         "did not pick (fused vs separate) and report it as alt_bwd_ms")
    ap.add_argument("--packed", action="store_true",
                    help="ragged workloads: the sequences one after another in every head, with row offsets, "
                         "instead of padded tensors with lengths")
    ap.add_argument("--copy-ref-mib", type=int, default=0,
                    help="launch one plain device copy of this size first (the counter reference "
                         "for the HBM traffic summary)")
    return ap.parse_args()


def pairs_of(w):
    if w.lengths:  # ragged batch: each element with its own length (query = key)
        return sum(w.H * (n * (n + 1) // 2 if w.causal else n * n) for n in w.lengths)
    n_q, n_k = w.n_q, w.n_k
    if not w.causal:
        return w.B * w.H * n_q * n_k
    return w.B * w.H * (n_q * (n_q + 1) // 2 + n_q * (n_k - n_q))


def cpu_baseline(w, rows_wanted, head_bytes=None, gpu=None):
    """The fp64 oracle on the host: forward + backward of the step's settings
    for a bounded sample (the last rows of head 0, which see the full key
    range), reported as algorithmic TFLOP/s like the GPU value.  With
    head_bytes (the algorithmic HBM bytes of one head's step, for the
    bandwidth-bound decode shapes) the sample must be whole heads and the rate
    is in GB/s.  gpu: head 0's inputs as the GPU received them and its outputs
    ({"inputs": [q1, k1, q2, k2], "g", "kl", "lse1", "lse2", "dq": {setting:
    array}}, host arrays, g the step's upstream gradient); the oracle runs on
    those inputs and the errors of the GPU's rows against it are returned too."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    hi = gpu["inputs"]
    n_q, n_k = hi[0].shape[0], hi[1].shape[0]
    g = gpu["g"]
    rows = np.arange(max(0, n_q - rows_wanted), n_q)
    block = max(1, min(64, (1 << 22) // n_k))
    t0 = time.perf_counter()
    ref = oracle.head_forward(*hi, w.causal, rows=rows, block=block)
    rdq = {}
    for setting in w.settings:
        rdq[setting], _ = oracle.head_backward(setting, *hi, w.causal, g, rows=rows, block=block)
    dt = time.perf_counter() - t0
    vis = oracle.valid_mask(rows, n_q, n_k, w.causal).sum()
    qk = 2 * (w.d1 + w.d2)
    flops = float(vis) * (qk + sum(qk + 4 * (w.d2 if st == 1 else w.d1) for st in w.settings))
    steps = "".join(f" + setting-{st} backward" for st in w.settings)
    if head_bytes is not None and len(rows) == n_q:
        res = {"value": head_bytes / dt / 1e9, "unit": "GB/s", "cores": int(threads), "kind": "oracle",
               "seconds": dt,
               "sample": f"numpy fp64 oracle, forward{steps} of one whole head ({n_q} query rows over {n_k} keys),"
                         " rated by that head's algorithmic HBM bytes"}
    else:
        res = {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
               "seconds": dt,
               "sample": f"numpy fp64 oracle, forward{steps} of the last {len(rows)} query rows of head 0 over all"
                         f" {n_k} keys ({int(vis)} visible pairs)"}
    # the GPU's rows against the oracle: max and 99th percentile of the
    # per-row errors, and the largest ratio to the tolerance (<= 1 passes)
    a, r = (1e-4, 1e-3) if w.dtype == "f32" else (1e-3, 1e-2)
    dkl = np.abs(gpu["kl"][rows] - ref[0])
    err = {"rows": int(len(rows)),
           "kl_abs_max": float(dkl.max()), "kl_abs_p99": float(np.percentile(dkl, 99)),
           "kl_tol_ratio_max": float((dkl / (a + r * np.abs(ref[0]))).max())}
    for name, i in (("lse1", 1), ("lse2", 2)):
        d = np.abs(gpu[name][rows] - ref[i])
        err[f"{name}_abs_max"], err[f"{name}_abs_p99"] = float(d.max()), float(np.percentile(d, 99))
    for setting, dq in gpu["dq"].items():
        got, want = dq[rows], rdq[setting]
        rowerr = np.linalg.norm(got - want, axis=1) / np.maximum(np.linalg.norm(want, axis=1), 1e-300)
        err[f"dq{setting}_rel_l2"] = float(np.linalg.norm(got - want) / np.linalg.norm(want))
        err[f"dq{setting}_row_rel_max"] = float(rowerr.max())
        err[f"dq{setting}_row_rel_p99"] = float(np.percentile(rowerr, 99))
    return res, err


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(json.dumps({"error": "this build runs on one GPU only: the attention-KL path shards by heads "
                                   "with no communication, so N GPUs run N independent copies; "
                                   "run with --gpus 1"}))
        return 2
    import torch
    import workloads
    from attention_kl_divergence_amd import streamkl as sk

    w = workloads.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    q1, k1, q2, k2 = workloads.generate(w, dev)
    g = workloads.upstream_grad(w, dev, "mean")
    # ragged workloads: the same lengths for queries and keys of each element
    lens = dict(q_len=list(w.lengths), k_len=list(w.lengths)) if w.lengths else {}
    kv = k1.shape[1]
    packed = args.packed
    if packed:
        if not w.lengths:
            print(json.dumps({"error": f"--packed needs a ragged workload; {w.name} has none"}))
            return 2
        # element b's rows [0, n_b) of every head, one element after another
        pack = lambda t: torch.cat([t[b, :, :n] for b, n in enumerate(w.lengths)], dim=1).contiguous()  # noqa: E731
        q1, k1, q2, k2, g = (pack(t) for t in (q1, k1, q2, k2, g))
        torch.cuda.empty_cache()
        off = [0]
        for n in w.lengths:
            off.append(off[-1] + n)
        lens = dict(q_off=off, k_off=off)
        shp = sk.packed_shape_of(q1, k1, q2, k2, off, off)
        rows_q, rows_k = (w.H, off[-1]), (kv, off[-1])  # per-row outputs, dK leading dims
    else:
        shp = sk.shape_of(q1, k1, q2, k2).set_lengths(**lens)
        rows_q, rows_k = (w.B, w.H, w.n_q), (w.B, kv, w.n_k)
    mode = {"auto": sk.BWD_AUTO, "fused": sk.BWD_FUSED, "separate": sk.BWD_SEPARATE}[args.bwd_mode]
    splits = sk.fwd_plan(shp, w.causal)

    f32 = dict(device=dev, dtype=torch.float32)
    kl, l1, l2 = (torch.empty(rows_q, **f32) for _ in range(3))
    ws_bytes = sk.fwd_workspace_bytes(shp, w.causal)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)

    # Each kernel is launched by its own ABI call so HIP events on the launch
    # stream bracket exactly one kernel (split-K adds its merge kernel).
    calls = [("fwd", lambda: sk.streamkl_fwd(q1, k1, q2, k2, w.causal, out=(kl, l1, l2), workspace=ws, **lens))]
    modes = {}
    joint = args.joint and tuple(sorted(w.settings)) == (1, 2)
    if joint:
        jo = (torch.empty((*rows_q, w.d1), **f32), torch.empty((*rows_k, w.d1), **f32),
              torch.empty((*rows_q, w.d2), **f32), torch.empty((*rows_k, w.d2), **f32))
        calls.append(("bwdj_dk", lambda: sk.streamkl_bwd_joint(q1, k1, q2, k2, w.causal, kl, l1, l2, g,
                                                                bwd_mode=sk.BWD_DK_ONLY, out=(None, jo[1], None, jo[3]),
                                                                **lens)))
        calls.append(("bwdj_dq", lambda: sk.streamkl_bwd_joint(q1, k1, q2, k2, w.causal, kl, l1, l2, g,
                                                                bwd_mode=sk.BWD_DQ_ONLY, out=(jo[0], None, jo[2], None),
                                                                **lens)))
    grads = {}  # setting -> (dQ, dK) buffers of the timed calls
    if joint:
        grads = {2: (jo[0], jo[1]), 1: (jo[2], jo[3])}
    for setting in (() if joint else w.settings):
        ds = w.d2 if setting == 1 else w.d1
        dq = torch.empty((*rows_q, ds), **f32)
        dk = torch.empty((*rows_k, ds), **f32)
        grads[setting] = (dq, dk)
        plan = sk.bwd_plan(shp, w.causal, setting, mode)
        modes[setting] = plan

        def mk(m, o, st=setting):
            return lambda: sk.streamkl_bwd(st, q1, k1, q2, k2, w.causal, kl, l1, l2, g, bwd_mode=m, out=o, **lens)
        if plan == sk.BWD_FUSED:
            calls.append((f"bwd{setting}_fused", mk(sk.BWD_FUSED, (dq, dk))))
        else:
            calls.append((f"bwd{setting}_dk", mk(sk.BWD_DK_ONLY, (None, dk))))
            calls.append((f"bwd{setting}_dq", mk(sk.BWD_DQ_ONLY, (dq, None))))

    if args.copy_ref_mib > 0:
        n = args.copy_ref_mib * (1 << 20) // 4
        src = torch.ones(n, **f32)
        dst = torch.empty(n, **f32)
        torch.cuda.synchronize()
        torch.mul(src, 1.0, out=dst)  # reads and writes copy_ref_mib MiB
        torch.cuda.synchronize()
        del src, dst

    # the part's own rates, measured before the timed region: the bf16
    # matrix-core rate with no operand traffic and the shader clock it holds,
    # and the v_exp_f32 rate (attention_kl_divergence_amd/csrc/probes.hip)
    from attention_kl_divergence_amd import profiling
    try:
        pm = profiling.probe_mfma(1, iters=100000)
        pe = profiling.probe_exp(2, iters=20000)
        probe = {"mfma_bf16_tflops": round(pm["tflops"], 1), "sclk_mhz": round(pm["sclk_mhz"]),
                 "spec_peak_at_sclk_tflops": round(MFMA_BF16_PEAK_TFLOPS * pm["sclk_mhz"] / 2400.0, 1),
                 "exp_per_ns": round(pe["exp_per_ns"], 1)}
    except Exception as e:  # the bench line still reports the spec peaks
        probe = {"error": str(e)}

    for _ in range(args.warmup):
        for _, c in calls:
            c()
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream(dev)
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in calls]
          for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        for (name, c), (e0, e1) in zip(calls, ev[s]):
            e0.record(stream)
            c()
            e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    per_call = {name: sum(ev[s][i][0].elapsed_time(ev[s][i][1]) for s in range(args.steps)) / args.steps
                for i, (name, _) in enumerate(calls)}
    ms_step = wall * 1e3 / args.steps
    pairs = pairs_of(w)
    qk = 2 * (w.d1 + w.d2)
    # algorithmic FLOPs each call is credited with (the logit recompute of the
    # separate mode's dQ kernel is not credited)
    credit = {"fwd": qk * pairs}
    for setting in w.settings:
        ds = w.d2 if setting == 1 else w.d1
        credit[f"bwd{setting}_fused"] = (qk + 4 * ds) * pairs
        credit[f"bwd{setting}_dk"] = (qk + 2 * ds) * pairs
        credit[f"bwd{setting}_dq"] = 2 * ds * pairs
    credit["bwdj_dk"] = (qk + 2 * (w.d1 + w.d2)) * pairs
    credit["bwdj_dq"] = 2 * (w.d1 + w.d2) * pairs
    flops_step = sum(credit[n] for n, _ in calls)
    peak = MFMA_BF16_PEAK_TFLOPS if w.dtype == "bf16" else MFMA_F32_PEAK_TFLOPS
    value = flops_step / (ms_step * 1e-3) / 1e12
    esz = 2 if w.dtype == "bf16" else 4
    fwd_bytes = w.B * w.H * ((w.n_q + w.n_k) * (w.d1 + w.d2) * esz + 12 * w.n_q)

    dom = max(per_call, key=per_call.get)
    # the forward kernel the library picks: one wave per key split for short
    # bf16 query ranges, the 8-wave ping-pong form for long unsplit ones
    if splits > 1 and w.dtype == "bf16" and w.n_q <= 32:
        fwd_kernel = "fwd_decode_kernel"
    elif splits == 1 and w.n_q > 128 and not (w.dtype == "f32" and w.d1 + w.d2 > 128):
        fwd_kernel = "fwd_pp_kernel"
    else:
        fwd_kernel = "fwd_kernel"
    # decode shapes (bf16, at most 32 query rows): the split-K forward and the
    # decode backward, both bound by HBM bandwidth
    decode = w.dtype == "bf16" and w.n_q <= 32
    kernel_names = {"fwd": fwd_kernel, "bwdj_dk": "bwd_dk_kernel<JOINT>", "bwdj_dq": "bwd_dq_kernel"}
    for setting in w.settings:
        kernel_names[f"bwd{setting}_fused"] = "bwd_decode_kernel" if decode else "bwd_dk_kernel<FUSED>"
        kernel_names[f"bwd{setting}_dk"] = "bwd_dk_kernel"
        kernel_names[f"bwd{setting}_dq"] = "bwd_dq_kernel"
    # algorithmic HBM bytes of each call: every input read once, every output
    # written once (the backward reads K1, K2, Q1, Q2 and four row vectors and
    # writes dQ_s and dK_s in fp32)
    nbytes = {"fwd": fwd_bytes}
    for setting in w.settings:
        ds = w.d2 if setting == 1 else w.d1
        b = w.B * w.H * ((w.n_q + w.n_k) * (w.d1 + w.d2) * esz + 16 * w.n_q + (w.n_q + w.n_k) * ds * 4)
        nbytes[f"bwd{setting}_fused"] = b
    if decode:
        dname = max((n for n, _ in calls), key=lambda n: per_call[n])
        ach = nbytes[dname] / (per_call[dname] * 1e-3) / 1e9
        kn = kernel_names[dname]
        if dname == "fwd" and splits > 1:
            kn += " + splitk_merge_kernel"
        roof = {"bound": "hbm", "kernel": kn,
                "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBS, 4),
                "traffic": None, "avg_ms": round(per_call[dname], 4)}
    else:
        ach = credit[dom] / (per_call[dom] * 1e-3) / 1e12
        roof = {"bound": "mfma", "kernel": kernel_names[dom], "achieved": round(ach, 2), "peak": peak,
                "unit": "TFLOP/s", "frac": round(ach / peak, 4), "traffic": None,
                "avg_ms": round(per_call[dom], 4)}

    # measured HBM bytes per launch of that kernel (calibrated TCC counters),
    # valid only for the kernel sources they were taken with
    summ = profiling.load_summary(w.name)
    kname = roof["kernel"].split(" + ")[0]
    if summ and summ.get("source_digest") == profiling.kernel_source_digest() and kname in summ["kernels"]:
        t = summ["kernels"][kname]
        roof["traffic"] = int(t.get("fetch_bytes", 0) + t.get("write_bytes", 0))
        roof["traffic_unit"] = "bytes per launch: FETCH_SIZE + WRITE_SIZE, copy-calibrated"

    extra_hbm = 3 * 4 * kl.numel() + ws_bytes
    # the two bf16 probability matrices a materialising implementation would hold
    qk_cells = sum(n * n for n in w.lengths) if w.lengths else w.B * w.n_q * w.n_k
    names = {sk.BWD_FUSED: "fused", sk.BWD_SEPARATE: "separate"}
    headline = w.name == "h32-n64k-d128-bf16-causal"
    out = {
        "metric": ("attn-KL fwd/bwd TFLOP/s + % bf16 MFMA peak, H32 d128 causal 64K" if headline
                   else (("attn-KL decode forward + backward HBM GB/s" if w.settings
                          else "attn-KL split-K forward HBM GB/s") if decode else "attn-KL fwd/bwd TFLOP/s")),
        "value": round(sum(nbytes[n] for n, _ in calls) / (ms_step * 1e-3) / 1e9, 1) if decode else round(value, 2),
        "unit": "GB/s" if decode else "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "n_q": w.n_q, "n_k": w.n_k, "d1": w.d1, "d2": w.d2,
                   "causal": w.causal, "bwd_settings": list(w.settings),
                   "bwd_modes": {str(k): names[v] for k, v in modes.items()} if not joint else {"1+2": "joint"},
                   "fwd_splits": splits, "parallelism": "single GPU",
                   **({"kv_heads": kv} if kv != w.H else {}),
                   **({"lengths": list(w.lengths), "layout": "packed" if packed else "padded"}
                      if w.lengths else {})},
        "pct_of_mfma_peak": round(100 * value / peak, 2),
        "per_kernel_ms": {k: round(v, 4) for k, v in per_call.items()},
        "algorithmic_tflop_per_step": round(flops_step / 1e12, 4),
        "extra_hbm_bytes": extra_hbm,
        "materialised_bytes_avoided": 2 * 2 * w.H * qk_cells,
        "roofline": roof,
        "device_probe": probe,
    }
    if "mfma_bf16_tflops" in probe and not decode:
        out["pct_of_measured_mfma_peak"] = round(100 * value / probe["mfma_bf16_tflops"], 2)
        roof["frac_of_measured_peak"] = round(roof["achieved"] / probe["mfma_bf16_tflops"], 4)
    # exponentials each call evaluates per visible pair (P1 and P2, or P1
    # alone in setting 2) against the measured v_exp_f32 rate
    exps = {"fwd": 2, "bwdj_dk": 2, "bwdj_dq": 3}
    for setting in w.settings:
        for kind in ("fused", "dk", "dq"):
            exps[f"bwd{setting}_{kind}"] = 2 if setting == 1 else 1
    if "exp_per_ns" in probe:
        out["transcendental"] = {
            n: {"exp_per_ns": round(exps[n] * pairs / (per_call[n] * 1e6), 1),
                "frac": round(exps[n] * pairs / (per_call[n] * 1e6) / probe["exp_per_ns"], 4)}
            for n in per_call if n in exps}
    if decode:
        # the pages' two ablations on decode shapes: the split-K forward against
        # one workgroup sweep per query block (num_splits = 1), and the fused
        # backward against the separate dK + dQ kernels
        def once(fn):
            fn()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            torch.cuda.synchronize()
            return e0.elapsed_time(e1)
        abl = {"fwd_split_ms": round(per_call["fwd"], 4)}
        t1 = once(lambda: sk.streamkl_fwd(q1, k1, q2, k2, w.causal, num_splits=1, **lens))
        abl["fwd_one_split_ms"] = round(t1, 4)
        abl["split_speedup"] = round(t1 / per_call["fwd"], 2)
        for setting in w.settings:
            name = f"bwd{setting}_fused"
            if name in per_call:
                t2 = once(lambda: sk.streamkl_bwd(setting, q1, k1, q2, k2, w.causal, kl, l1, l2, g,
                                                  bwd_mode=sk.BWD_SEPARATE, **lens))
                abl[f"bwd{setting}_separate_ms"] = round(t2, 4)
                abl[f"bwd{setting}_fused_speedup"] = round(t2 / per_call[name], 2)
        out["ablation"] = abl
    # device memory the library takes beyond the caller's buffers: none (it
    # never allocates); checked with the driver's free-memory count around a step
    free0 = torch.cuda.mem_get_info(dev)[0]
    for _, c in calls:
        c()
    torch.cuda.synchronize()
    out["library_device_allocation_bytes"] = int(free0 - torch.cuda.mem_get_info(dev)[0])
    if args.compare_modes:
        alt = {}
        for setting in (() if joint else w.settings):
            ds = w.d2 if setting == 1 else w.d1
            other = sk.BWD_SEPARATE if modes[setting] == sk.BWD_FUSED else sk.BWD_FUSED
            dq = torch.empty((*rows_q, ds), **f32)
            dk = torch.empty((*rows_k, ds), **f32)
            run = lambda: sk.streamkl_bwd(setting, q1, k1, q2, k2, w.causal, kl, l1, l2, g,  # noqa: E731
                                          bwd_mode=other, out=(dq, dk), **lens)
            run()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            run()
            e1.record(stream)
            torch.cuda.synchronize()
            alt[f"bwd{setting}_{names[other]}"] = round(e0.elapsed_time(e1), 3)
        out["alt_bwd_ms"] = alt
    if not args.no_cpu_baseline:
        # about 4e8 visible pairs of oracle work (10-20 s on the host) at most
        hb = sum(nbytes[n] for n, _ in calls) / (w.B * w.H) if decode else None
        n0 = w.lengths[0] if w.lengths else w.n_q  # rows (= keys of a ragged element) of batch element 0
        nk0 = w.lengths[0] if w.lengths else w.n_k
        # head 0 of element 0 (a packed element 0 starts at row 0 of every head)
        host = lambda t, n: (t[0] if packed else t[0, 0]).float().cpu().numpy().astype("float64")[:n]  # noqa: E731
        gpu = {"inputs": [host(q1, n0), host(k1, nk0), host(q2, n0), host(k2, nk0)], "g": host(g, n0),
               "kl": host(kl, n0), "lse1": host(l1, n0), "lse2": host(l2, n0),
               "dq": {st: host(grads[st][0], n0) for st in w.settings if st in grads}}
        out["cpu_baseline"], out["oracle_errors"] = cpu_baseline(w, min(args.cpu_rows, max(1, int(4e8 // nk0))),
                                                                 hb, gpu)
    print(json.dumps(out))
    return 0


if __name__ == "__main__":
    sys.exit(main())
