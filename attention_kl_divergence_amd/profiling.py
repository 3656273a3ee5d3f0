"""HBM traffic per kernel launch from rocprofv3 counter runs.

The TCC counters FETCH_SIZE and WRITE_SIZE (KiB per dispatch) are taken in
two separate `rocprofv3 --pmc` runs of `bench.py --copy-ref-mib N`, which
launches one plain device copy of known size (read N MiB, write N MiB)
before the timed steps.  Each counter is scaled by known/measured for that
copy dispatch, then averaged over the launches of each StreamKL kernel.

    python -m attention_kl_divergence_amd.profiling traffic \\
        --fetch <fetch run>/run_counter_collection.csv \\
        --write <write run>/run_counter_collection.csv \\
        --copy-mib N --workload NAME --command "..." --out profiles/<file>.md

The summary carries a digest of the kernel sources and build flags; the
benchmark reports the traffic figure only while that digest still matches.
"""
from __future__ import annotations

import argparse
import collections
import csv
import hashlib
import json
import os
import re
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
PROFILES = os.path.join(ROOT, "profiles")

# kernels whose traffic is summarised: label -> pattern on the kernel name as
# rocprofv3 reports it (mangled, e.g. ...bwd_dk_kernelIDF16bLi128ELi128ELi1ELb0E...,
# or demangled, e.g. streamkl::bwd_dk_kernel<__bf16, 128, 128, 1, false, 64>)
KERNELS = [
    ("fwd_decode_kernel", r"fwd_decode_kernel"),
    ("fwd_pp_kernel", r"fwd_pp_kernel"),
    ("fwd_kernel", r"fwd_kernel"),
    ("bwd_dk_kernel<JOINT>", r"bwd_dk_kernel(I.*Li3ELb0E|<[^>]*, 3, false)"),
    ("bwd_dk_kernel", r"bwd_dk_kernel(I.*Lb0E|<[^>]*false)"),
    ("bwd_dk_kernel<FUSED>", r"bwd_dk_kernel(I.*Lb1E|<[^>]*true)"),
    ("bwd_dq_kernel", r"bwd_dq_kernel"),
    ("bwd_decode_kernel", r"bwd_decode_kernel"),
    ("splitk_merge_kernel", r"splitk_merge_kernel"),
]
# the reference copy: torch.mul(src, 1.0, out=dst), the last such dispatch
# before the first StreamKL kernel
COPY_PATTERN = r"MulFunctor"
STREAMKL_PATTERN = r"streamkl"


def kernel_source_digest() -> str:
    """sha256 over the kernel sources and the device compile flags."""
    from . import build
    h = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)):
        if name.endswith((".hpp", ".hip", ".h")):
            h.update(name.encode())
            with open(os.path.join(CSRC, name), "rb") as f:
                h.update(f.read())
    h.update(" ".join(build.FLAGS).encode())
    return h.hexdigest()


def _rows(path):
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def _per_dispatch(rows, counter):
    """{dispatch id: (kernel name, value)} for one counter (summed over instances)."""
    out = {}
    for r in rows:
        if r["Counter_Name"] != counter:
            continue
        d = int(r["Dispatch_Id"])
        name = r["Kernel_Name"]
        v = float(r["Counter_Value"])
        if d in out:
            out[d] = (name, out[d][1] + v)
        else:
            out[d] = (name, v)
    return out


def _label(name):
    for label, pat in KERNELS:
        if re.search(pat, name):
            return label
    return None


def traffic(fetch_csv, write_csv, copy_mib):
    """Calibrated HBM bytes per launch: {label: {"fetch_bytes", "write_bytes", "launches"}}."""
    known = copy_mib * 1024 * 1024
    res = {}
    factors = {}
    for counter, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        per = _per_dispatch(_rows(path), counter)
        first = min((d for d, (n, _) in per.items() if re.search(STREAMKL_PATTERN, n)), default=None)
        copies = [d for d, (n, _) in per.items() if re.search(COPY_PATTERN, n) and (first is None or d < first)]
        if not copies:
            raise SystemExit(f"no reference copy dispatch in {path}")
        measured = per[max(copies)][1] * 1024.0
        factors[counter] = known / measured
        acc = collections.defaultdict(list)
        for name, v in per.values():
            lab = _label(name)
            if lab:
                acc[lab].append(v * 1024.0 * factors[counter])
        key = "fetch_bytes" if counter == "FETCH_SIZE" else "write_bytes"
        for lab, vals in acc.items():
            res.setdefault(lab, {})[key] = sum(vals) / len(vals)
            res[lab]["launches"] = len(vals)
    return res, factors


def load_summary(workload):
    """The JSON block of profiles/traffic_<workload>.md, or None."""
    path = os.path.join(PROFILES, f"traffic_{workload}.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"```json\n(.*?)\n```", text, re.S)
    return json.loads(m.group(1)) if m else None


def kernel_summary(stats_csv, bench_log, workload, command):
    """Markdown summary of a rocprofv3 --kernel-trace --stats run of bench.py
    (library kernels only) next to the bench line the same run printed."""
    rows = [r for r in _rows(stats_csv) if re.search(STREAMKL_PATTERN, r["Name"])]
    total = sum(float(r["TotalDurationNs"]) for r in rows) or 1.0
    bench = None
    with open(bench_log) as f:
        for line in f:
            if line.startswith("{") and '"metric"' in line:
                bench = json.loads(line)
    lines = [f"# Kernel time summary, workload {workload}", "",
             "Command (run from /tmp with TMPDIR=/tmp on one MI355X):", "", "```", command, "```", "",
             "Source: `run_kernel_stats.csv`; library kernels only (the input generators' kernels are omitted).", "",
             "| kernel | calls | average ms | min ms | max ms | share of library time |", "|---|---|---|---|---|---|"]
    for r in sorted(rows, key=lambda r: -float(r["TotalDurationNs"])):
        name = re.sub(r"^_ZN8streamkl", "", r["Name"])
        lines.append(f"| `{name}` | {r['Calls']} | {float(r['AverageNs']) / 1e6:.3f} | {float(r['MinNs']) / 1e6:.3f} | "
                     f"{float(r['MaxNs']) / 1e6:.3f} | {100 * float(r['TotalDurationNs']) / total:.1f}% |")
    if bench:
        roof = bench.get("roofline", {})
        lines += ["", "The same run's bench line (HIP events on the launch stream), per call in ms: " +
                  ", ".join(f"{k} {v}" for k, v in bench.get("per_kernel_ms", {}).items()) + ".",
                  f"Dominant kernel: {roof.get('kernel')} at {roof.get('avg_ms')} ms per launch, "
                  f"{roof.get('achieved')} {roof.get('unit')} ({100 * roof.get('frac', 0):.1f}% of {roof.get('peak')})."]
        dom = roof.get("kernel", "").split(" + ")[0]
        pat = dict(KERNELS).get(dom)
        match = [r for r in rows if pat and re.search(pat, r["Name"])]
        if match and roof.get("avg_ms"):
            avg = float(match[0]["AverageNs"]) / 1e6
            lines.append(f"rocprofv3 average for it: {avg:.3f} ms "
                         f"({100 * (roof['avg_ms'] - avg) / avg:+.2f}% bench vs profiler).")
    lines.append("")
    return "\n".join(lines)


# SQ counter sets for `counters`, one rocprofv3 --pmc pass each (at most 8 SQ
# counters per pass)
COUNTER_SETS = [
    "SQ_WAVES SQ_WAVE_CYCLES SQ_BUSY_CYCLES SQ_INSTS_VALU SQ_INSTS_MFMA SQ_INSTS_LDS SQ_INSTS_SALU "
    "SQ_VALU_MFMA_BUSY_CYCLES",
    "SQ_ACTIVE_INST_VALU SQ_ACTIVE_INST_ANY SQ_WAIT_INST_ANY SQ_WAIT_ANY SQ_VALU_MFMA_COEXEC_CYCLES "
    "SQ_ACTIVE_INST_LDS SQ_WAIT_INST_LDS SQ_INSTS_VALU_TRANS_F32",
]


def _gpu_topology(agent_csv):
    for r in _rows(agent_csv):
        if r["Agent_Type"] == "GPU":
            cus = int(r["Cu_Count"])
            return {"cus": cus, "simds": cus * int(r["Simd_Per_Cu"]), "ses": int(r["Num_Shader_Banks"])}
    raise SystemExit(f"no GPU agent in {agent_csv}")


def counters(csvs, agent_csv):
    """Per-kernel SQ counter averages per dispatch and derived utilisations.

    SQ_BUSY_CYCLES sums over shader engines, so /SEs is the dispatch length in
    cycles (T).  SQ_VALU_MFMA_BUSY_CYCLES and SQ_VALU_MFMA_COEXEC_CYCLES sum
    over SIMDs: /SIMDs/T is the fraction of the dispatch the matrix cores are
    busy, resp. busy while the VALU also issues.  VALU issue rate: non-MFMA
    VALU instructions per SIMD per cycle (a wave64 fp32 VALU op occupies a
    SIMD for at least 4 cycles, so 0.25 is the ceiling)."""
    topo = _gpu_topology(agent_csv)
    agg = collections.defaultdict(lambda: collections.defaultdict(float))
    disp = collections.defaultdict(set)
    for path in csvs:
        for r in _rows(path):
            lab = _label(r["Kernel_Name"])
            if not lab:
                continue
            agg[lab][r["Counter_Name"]] += float(r["Counter_Value"])
            disp[(lab, path)].add(r["Dispatch_Id"])
    out = {}
    for lab, c in agg.items():
        n = {}
        for path in csvs:
            if disp.get((lab, path)):
                n[path] = len(disp[(lab, path)])
        # every pass ran the same launches; average per dispatch of its own pass
        per = {}
        for name, v in c.items():
            cnt = max(n.values()) if n else 1
            per[name] = v / cnt
        t = per.get("SQ_BUSY_CYCLES", 0.0) / topo["ses"]
        d = {"dispatch_cycles": t}
        if t > 0:
            d["mfma_busy"] = per.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) / topo["simds"] / t
            d["mfma_valu_coexec"] = per.get("SQ_VALU_MFMA_COEXEC_CYCLES", 0.0) / topo["simds"] / t
            valu = per.get("SQ_INSTS_VALU", 0.0) - per.get("SQ_INSTS_MFMA", 0.0)
            d["valu_issue_per_simd_cycle"] = valu / topo["simds"] / t
        if per.get("SQ_WAVE_CYCLES"):
            d["lds_wait_share"] = per.get("SQ_WAIT_INST_LDS", 0.0) / per["SQ_WAVE_CYCLES"]
        for k in ("SQ_INSTS_MFMA", "SQ_INSTS_VALU", "SQ_INSTS_VALU_TRANS_F32", "SQ_INSTS_LDS", "SQ_INSTS_SALU"):
            if k in per:
                d[k] = per[k]
        out[lab] = d
    return out, topo


# ---- device probes (libstreamkl_probes.so): the part's own rates ----

MFMA_FLOP = 2 * 32 * 32 * 16  # one v_mfma_f32_32x32x16_bf16


def _probes():
    import ctypes
    path = os.path.join(HERE, "libstreamkl_probes.so")
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m attention_kl_divergence_amd.build`")
    lib = ctypes.CDLL(path)
    vp, i32, u32 = ctypes.c_void_p, ctypes.c_int, ctypes.c_uint32
    lib.streamkl_probe_mfma.argtypes = [vp, vp, i32, i32, vp]
    lib.streamkl_probe_exp.argtypes = [vp, i32, i32, vp]
    lib.streamkl_probe_atomic.argtypes = [vp, u32, i32, i32, vp]
    lib.streamkl_probe_wall_clock_khz.argtypes = [ctypes.POINTER(ctypes.c_int)]
    for f in (lib.streamkl_probe_mfma, lib.streamkl_probe_exp, lib.streamkl_probe_atomic,
              lib.streamkl_probe_wall_clock_khz):
        f.restype = i32
    return lib


def _timed_launch(launch):
    """ms of one launch (after one warm-up launch), HIP events on the stream."""
    import torch
    launch()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    launch()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1)


def probe_mfma(waves_per_simd: int = 1, iters: int = 200000) -> dict:
    """bf16 matrix-core rate with no operand traffic (TFLOP/s over the whole
    chip) and the shader clock it ran at (MHz, median over workgroups)."""
    import ctypes

    import torch
    lib = _probes()
    dev = torch.device("cuda:0")
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    blocks = cus * waves_per_simd  # 4-wave workgroups: one wave per SIMD each
    out = torch.empty(blocks * 256, device=dev)
    clk = torch.zeros(2 * blocks, dtype=torch.int64, device=dev)
    stream = torch.cuda.current_stream(dev).cuda_stream

    def run():
        e = lib.streamkl_probe_mfma(out.data_ptr(), clk.data_ptr(), blocks, iters, stream)
        if e:
            raise RuntimeError(f"streamkl_probe_mfma: hipError {e}")
    ms = _timed_launch(run)
    khz = ctypes.c_int(0)
    if lib.streamkl_probe_wall_clock_khz(ctypes.byref(khz)) or khz.value <= 0:
        raise RuntimeError("wall clock rate unavailable")
    c = clk.view(-1, 2).double().cpu()
    mhz = (c[:, 0] / (c[:, 1] / (khz.value * 1e3))).median().item() / 1e6
    flops = blocks * 4 * iters * 4 * MFMA_FLOP
    return {"tflops": flops / ms / 1e9, "sclk_mhz": mhz, "ms": ms, "waves_per_simd": waves_per_simd,
            "cycles_per_mfma": mhz * 1e6 * ms * 1e-3 / (iters * 4 * waves_per_simd)}


def probe_exp(waves_per_simd: int = 2, iters: int = 40000) -> dict:
    """v_exp_f32 throughput over the whole chip (exponentials per ns)."""
    import torch
    lib = _probes()
    dev = torch.device("cuda:0")
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    blocks = cus * waves_per_simd
    out = torch.empty(blocks * 256, device=dev)
    stream = torch.cuda.current_stream(dev).cuda_stream

    def run():
        e = lib.streamkl_probe_exp(out.data_ptr(), blocks, iters, stream)
        if e:
            raise RuntimeError(f"streamkl_probe_exp: hipError {e}")
    ms = _timed_launch(run)
    n = blocks * 256 * iters * 8
    return {"exp_per_ns": n / ms / 1e6, "ms": ms, "waves_per_simd": waves_per_simd}


def probe_atomic(window_mib: int, iters: int = 2000) -> dict:
    """fp32 device-scope atomic adds, 64 consecutive floats per wave at
    scattered 256-byte slots of a window: payload GB/s."""
    import torch
    lib = _probes()
    dev = torch.device("cuda:0")
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    slots = window_mib * (1 << 20) // 256
    win = torch.zeros(slots * 64, device=dev)
    blocks = cus * 8
    stream = torch.cuda.current_stream(dev).cuda_stream

    def run():
        e = lib.streamkl_probe_atomic(win.data_ptr(), slots, blocks, iters, stream)
        if e:
            raise RuntimeError(f"streamkl_probe_atomic: hipError {e}")
    ms = _timed_launch(run)
    return {"gbs": blocks * 256 * iters * 4 / ms / 1e6, "ms": ms, "window_mib": window_mib}


def device_probes() -> str:
    """Markdown summary of the probes (matrix-core rate and clock, exponential
    rate, atomic payload rate)."""
    m1, m2 = probe_mfma(1), probe_mfma(2)
    e1, e2 = probe_exp(1), probe_exp(2)
    at = [probe_atomic(w) for w in (1, 64, 1024)]
    cus = 256
    rows = [
        f"| bf16 MFMA 32x32x16, no operand traffic, 1 wave per SIMD | {m1['tflops']:.1f} TFLOP/s | "
        f"sclk {m1['sclk_mhz']:.0f} MHz, {m1['cycles_per_mfma']:.1f} cycles per MFMA |",
        f"| same, 2 waves per SIMD | {m2['tflops']:.1f} TFLOP/s | sclk {m2['sclk_mhz']:.0f} MHz, "
        f"{m2['cycles_per_mfma']:.1f} cycles per MFMA issued on a SIMD |",
        f"| spec bf16 dense peak scaled to that clock (2516.6 x sclk / 2400 MHz) | "
        f"{2516.6 * m1['sclk_mhz'] / 2400:.1f} TFLOP/s | |",
        f"| v_exp_f32, 8 chains per lane, 1 wave per SIMD | {e1['exp_per_ns']:.0f} exp/ns | "
        f"{e1['exp_per_ns'] / (cus * 4) / (m1['sclk_mhz'] / 1e3):.2f} exp per SIMD-cycle at that sclk |",
        f"| same, 2 waves per SIMD | {e2['exp_per_ns']:.0f} exp/ns | "
        f"{e2['exp_per_ns'] / (cus * 4) / (m1['sclk_mhz'] / 1e3):.2f} exp per SIMD-cycle |",
    ] + [f"| fp32 atomic add, 64 floats per wave at scattered 256 B slots, {a['window_mib']} MiB window | "
         f"{a['gbs']:.0f} GB/s payload | |" for a in at]
    return "\n".join([
        "# Device probes on one MI355X", "",
        "Command: `python -m attention_kl_divergence_amd.profiling probes --out profiles/device_probes.md`",
        "(kernels in `attention_kl_divergence_amd/csrc/probes.hip`; HIP events around one launch",
        "after one warm-up launch; the shader clock is the shader-cycle counter against the",
        "constant-rate wall clock over wave 0's matrix loop of each workgroup, median).", "",
        "| probe | rate | notes |", "|---|---|---|", *rows, "",
        "```json", json.dumps({"mfma_1": m1, "mfma_2": m2, "exp_1": e1, "exp_2": e2, "atomic": at}, indent=1),
        "```", ""])


def copy_bandwidth() -> str:
    """Markdown table of plain device copies and one-directional streams on
    cuda:0: the practical ceiling of a kernel that reads and writes in equal
    amounts.  HIP events around 5 back-to-back launches; bytes = read + write."""
    import torch
    dev = torch.device("cuda:0")

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(5):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / 5

    rows = []
    for gib in (1, 4, 8):
        n = gib * (1 << 30) // 4
        src = torch.ones(n, device=dev)
        dst = torch.empty(n, device=dev)
        for name, fn in (("`dst.copy_(src)`", lambda: dst.copy_(src)),
                         ("`torch.mul(src, 1.0, out=dst)`", lambda: torch.mul(src, 1.0, out=dst))):
            ms = timed(fn)
            rows.append(f"| {name} | {gib} GiB | {ms:.3f} | {2 * n * 4 / ms / 1e6:.0f} |")
        del src, dst
    n = 8 * (1 << 30) // 4
    x = torch.ones(n, device=dev)
    ms = timed(lambda: x.sum())
    rows.append(f"| `x.sum()` (read only) | 8 GiB | {ms:.3f} | {n * 4 / ms / 1e6:.0f} |")
    ms = timed(lambda: x.fill_(1.0))
    rows.append(f"| `x.fill_(1.0)` (write only) | 8 GiB | {ms:.3f} | {n * 4 / ms / 1e6:.0f} |")
    return "\n".join([
        "# Plain device copies on one MI355X (the ceiling of a 1:1 read/write stream)", "",
        "Command: `python -m attention_kl_divergence_amd.profiling copybw --out profiles/copy_bandwidth.md`",
        "(torch ops on fp32 tensors; HIP events around 5 back-to-back launches, bytes = read + write).", "",
        "| op | size | ms | GB/s |", "|---|---|---|---|", *rows, "",
        "The decode backward reads K1 and K2 (bf16) and writes dK (fp32) in equal",
        "byte counts, the mix of the elementwise `mul` above.", ""])


# Shapes of the backward mode sweep: (H, n_q, n_k, causal, setting), d = 128
# bf16.  Causal prefill from 512 to 32K rows, non-causal, short query ranges
# against long key ranges (where the fused mode's dQ working set is small),
# and fewer heads.
MODE_SWEEP = [
    (32, 512, 512, True, 1), (32, 1024, 1024, True, 1), (32, 2048, 2048, True, 1),
    (32, 4096, 4096, True, 1), (32, 8192, 8192, True, 1), (32, 8192, 8192, True, 2),
    (32, 16384, 16384, True, 1), (32, 32768, 32768, True, 1),
    (32, 4096, 4096, False, 1), (32, 16384, 16384, False, 1),
    (32, 16, 65536, False, 1), (32, 64, 65536, False, 1), (32, 256, 65536, False, 1),
    (32, 1024, 65536, False, 1), (8, 8192, 8192, True, 1), (4, 32768, 32768, True, 1),
]


def mode_sweep(shapes=MODE_SWEEP) -> str:
    """Markdown table: the fused and separate backward timed on cuda:0 for each
    shape (best of 3 launches, HIP events on the launch stream), the mode the
    library's plan picks, and what that pick costs against the faster one."""
    import torch
    sys.path.insert(0, ROOT)
    import workloads
    from . import streamkl as sk
    dev = torch.device("cuda:0")

    def best_ms(fn, n=3):
        fn()
        torch.cuda.synchronize()
        best = float("inf")
        for _ in range(n):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            best = min(best, e0.elapsed_time(e1))
        return best

    name = {sk.BWD_FUSED: "fused", sk.BWD_SEPARATE: "separate"}
    rows, regrets = [], []
    for H, n_q, n_k, causal, setting in shapes:
        w = workloads.Workload("mode-sweep", 1, H, n_q, n_k, 128, 128, "bf16", causal, 0.5, False, 7, (setting,))
        q1, k1, q2, k2 = workloads.generate(w, dev)
        g = workloads.upstream_grad(w, dev, "mean")
        kl, l1, l2 = sk.streamkl_fwd(q1, k1, q2, k2, causal)
        t = {}
        for m in (sk.BWD_FUSED, sk.BWD_SEPARATE):
            t[m] = best_ms(lambda m=m: sk.streamkl_bwd(setting, q1, k1, q2, k2, causal, kl, l1, l2, g, bwd_mode=m))
        pick = sk.bwd_plan(sk.shape_of(q1, k1, q2, k2), causal, setting)
        fast = min(t, key=t.get)
        regret = t[pick] / t[fast] - 1.0
        regrets.append(regret)
        rows.append(f"| {H} | {n_q} | {n_k} | {'yes' if causal else 'no'} | {setting} | {t[sk.BWD_FUSED]:.3f} | "
                    f"{t[sk.BWD_SEPARATE]:.3f} | {name[pick]} | {name[fast]} | {100 * regret:.1f}% |")
        del q1, k1, q2, k2, g, kl, l1, l2
        torch.cuda.empty_cache()
    hit = sum(r == 0.0 for r in regrets)
    return "\n".join([
        "# Backward mode plan against measurement, one MI355X", "",
        "Command: `python -m attention_kl_divergence_amd.profiling modes --out profiles/bwd_mode_plan.md`", "",
        "d1 = d2 = 128, bf16, B = 1, inputs from `workloads.generate` (seed 7, student = teacher + 0.5 noise),",
        "upstream gradient 1/N_Q per row.  Each mode is the best of 3 launches (HIP events on the launch",
        "stream).  The plan (`streamkl_bwd_plan`, the cost model that AUTO runs) sees only the shape and the",
        "CU count; query ranges of at most 32 rows run the decode kernel in the fused mode.", "",
        "| H | N_Q | N_K | causal | setting | fused ms | separate ms | plan picks | faster | cost of the pick |",
        "|---|---|---|---|---|---|---|---|---|---|", *rows, "",
        f"The plan picks the faster mode on {hit} of {len(rows)} shapes; the largest cost of a pick is "
        f"{100 * max(regrets):.1f}%.", ""])


def _best_ms(fn, n=3):
    """Best of n timed calls of fn (after one untimed), HIP events on torch's
    current stream, where the binding launches."""
    import torch
    fn()
    torch.cuda.synchronize()
    best = float("inf")
    for _ in range(n):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        fn()
        e1.record()
        torch.cuda.synchronize()
        best = min(best, e0.elapsed_time(e1))
    return best


# ragged batches for the backward plan: (label, B, H, causal, q range, k range
# or None for k = q, seed); lengths uniform in each range
RAGGED_SWEEP = [
    ("short prefill", 64, 32, True, (256, 2048), None, 1),
    ("medium prefill", 16, 32, True, (1024, 8192), None, 2),
    ("long prefill", 4, 32, True, (8192, 32768), None, 3),
    ("chunks vs long keys", 32, 32, False, (64, 512), (8192, 65536), 4),
    ("few rows vs long keys", 8, 32, False, (64, 192), (32768, 65536), 5),
    ("decode", 64, 32, False, (1, 32), (2048, 32768), 6),
]


def ragged_mode_sweep(batches=RAGGED_SWEEP) -> str:
    """Markdown table: the setting-1 backward of ragged batches in the
    automatic mode against the separate mode (grouped launches) and the
    fused mode (decode-shaped elements grouped, the others one launch each),
    best of 3 launches each on cuda:0."""
    import numpy as np
    import torch
    sys.path.insert(0, ROOT)
    import workloads
    from . import streamkl as sk
    dev = torch.device("cuda:0")
    best_ms = _best_ms
    rows, regrets = [], []
    for label, B, H, causal, qr, kr, seed in batches:
        r = np.random.default_rng(seed)
        q_len = [int(x) for x in r.integers(qr[0], qr[1] + 1, size=B)]
        k_len = list(q_len) if kr is None else [int(x) for x in r.integers(kr[0], kr[1] + 1, size=B)]
        w = workloads.Workload("ragged-modes", B, H, max(q_len), max(k_len), 128, 128, "bf16", causal, 0.5, False,
                               7)
        q1, k1, q2, k2 = workloads.generate(w, dev)
        g = workloads.upstream_grad(w, dev, "mean")
        lens = dict(q_len=q_len, k_len=k_len)
        kl, l1, l2 = sk.streamkl_fwd(q1, k1, q2, k2, causal, **lens)
        t = {m: best_ms(lambda m=m: sk.streamkl_bwd(1, q1, k1, q2, k2, causal, kl, l1, l2, g, bwd_mode=m, **lens))
             for m in (sk.BWD_AUTO, sk.BWD_SEPARATE, sk.BWD_FUSED)}
        fast = min(t[sk.BWD_SEPARATE], t[sk.BWD_FUSED])
        regret = t[sk.BWD_AUTO] / fast - 1.0
        regrets.append(regret)
        kdesc = "= N_Q" if kr is None else f"{kr[0]}-{kr[1]}"
        rows.append(f"| {label} | {B} | {qr[0]}-{qr[1]} | {kdesc} | {'yes' if causal else 'no'} | "
                    f"{t[sk.BWD_AUTO]:.3f} | {t[sk.BWD_SEPARATE]:.3f} | {t[sk.BWD_FUSED]:.3f} | "
                    f"{100 * regret:+.1f}% |")
        del q1, k1, q2, k2, g, kl, l1, l2
        torch.cuda.empty_cache()
    return "\n".join([
        "# Backward mode plan on ragged batches, one MI355X", "",
        "Command: `python -m attention_kl_divergence_amd.profiling modes --ragged "
        "--out profiles/bwd_mode_plan_ragged.md`", "",
        "H = 32, d1 = d2 = 128, bf16, setting 1, inputs from `workloads.generate` (seed 7), upstream",
        "gradient 1/N_Q per row; each batch draws its lengths uniformly from the ranges shown (fixed seeds).",
        "Automatic: the separate-mode kernels grouped over the batch when the cost model puts that at or",
        "below each element in its own best mode, else each element on its own plan; decode-shaped elements",
        "(at most 32 query rows) run the grouped decode backward.  Separate: every element in grouped",
        "launches.  Fused: decode-shaped elements grouped, the others one fused launch each.  Best of 3",
        "launches each (HIP events on the launch stream).", "",
        "| batch | B | N_Q | N_K | causal | automatic ms | separate ms | fused ms | automatic against the faster |",
        "|---|---|---|---|---|---|---|---|---|", *rows, "",
        f"The largest cost of the automatic choice against the faster forced mode is {100 * max(regrets):+.1f}%.",
        ""])


# ragged batches for the layout comparison: (label, B, causal, q range, k range
# or None for k = q, seed); H = 32, d = 128, bf16
LAYOUT_SWEEP = [
    ("short prefill", 64, True, (256, 2048), None, 3),
    ("medium prefill", 32, True, (1024, 4096), None, 4),
    ("tiny prefill", 16, True, (64, 512), None, 5),
    ("decode", 64, False, (1, 16), (512, 8192), 6),
]


def layout_sweep(batches=LAYOUT_SWEEP) -> str:
    """Markdown table: one forward plus setting-1 backward (automatic mode)
    of ragged batches in padded tensors against the same sequences packed,
    best of 5 each on cuda:0."""
    import numpy as np
    import torch
    sys.path.insert(0, ROOT)
    import workloads
    from . import streamkl as sk
    dev = torch.device("cuda:0")

    def pack(x, lens):
        return torch.cat([x[b, :, :n] for b, n in enumerate(lens)], dim=1).contiguous()

    rows = []
    for label, B, causal, qr, kr, seed in batches:
        r = np.random.default_rng(seed)
        q_len = [int(x) for x in r.integers(qr[0], qr[1] + 1, size=B)]
        k_len = list(q_len) if kr is None else [int(x) for x in r.integers(kr[0], kr[1] + 1, size=B)]
        w = workloads.Workload("ragged-layout", B, 32, max(q_len), max(k_len), 128, 128, "bf16", causal, 0.5,
                               False, 9)
        q1, k1, q2, k2 = workloads.generate(w, dev)
        g = workloads.upstream_grad(w, dev, "mean")
        lens = (q_len, k_len, q_len, k_len)
        P = [pack(x, n) for x, n in zip((q1, k1, q2, k2), lens)]
        gp = pack(g, q_len)
        pad = dict(q_len=q_len, k_len=k_len)
        pk = dict(q_off=[0, *np.cumsum(q_len).tolist()], k_off=[0, *np.cumsum(k_len).tolist()])

        def step(t, gg, kw):
            kl, l1, l2 = sk.streamkl_fwd(*t, causal, **kw)
            sk.streamkl_bwd(1, *t, causal, kl, l1, l2, gg, **kw)

        t_pad = _best_ms(lambda: step((q1, k1, q2, k2), g, pad), 5)
        t_pk = _best_ms(lambda: step(P, gp, pk), 5)
        mib = [sum(x.numel() * x.element_size() for x in ts) / 2 ** 20 for ts in ((q1, k1, q2, k2), P)]
        kdesc = "= N_Q" if kr is None else f"{kr[0]}-{kr[1]}"
        rows.append(f"| {label} | {B} | {qr[0]}-{qr[1]} | {kdesc} | {'yes' if causal else 'no'} | {t_pad:.3f} | "
                    f"{t_pk:.3f} | {t_pad / t_pk:.2f} | {mib[0]:.0f} | {mib[1]:.0f} |")
        del q1, k1, q2, k2, g, P, gp
        torch.cuda.empty_cache()
    return "\n".join([
        "# Ragged batches padded and packed, one MI355X", "",
        "Command: `python -m attention_kl_divergence_amd.profiling packed --out profiles/ragged_packed_layout.md`",
        "",
        "H = 32, d1 = d2 = 128, bf16, inputs from `workloads.generate` (seed 9), upstream gradient 1/N_Q per",
        "row; each batch draws its lengths uniformly from the ranges shown (fixed seeds).  One step is",
        "`streamkl_fwd` plus the setting-1 `streamkl_bwd` in the automatic mode, on the padded tensors with",
        "per-sequence lengths and on the same sequences packed with row offsets.  Best of 5 steps each",
        "(HIP events on the launch stream).  Memory: Q1, K1, Q2, K2 in each layout.", "",
        "| batch | B | N_Q | N_K | causal | padded ms | packed ms | speed-up | padded MiB | packed MiB |",
        "|---|---|---|---|---|---|---|---|---|---|", *rows, ""])


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    k = sub.add_parser("kernels")
    k.add_argument("--stats", required=True)
    k.add_argument("--bench-log", required=True)
    k.add_argument("--workload", required=True)
    k.add_argument("--command", required=True)
    k.add_argument("--out", required=True)
    t = sub.add_parser("traffic")
    t.add_argument("--fetch", required=True)
    t.add_argument("--write", required=True)
    t.add_argument("--copy-mib", type=int, required=True)
    t.add_argument("--workload", required=True)
    t.add_argument("--command", required=True, help="the commands that produced the two csv files")
    t.add_argument("--out", required=True)
    c = sub.add_parser("counters")
    c.add_argument("--csv", nargs="+", required=True, help="run_counter_collection.csv of each pass")
    c.add_argument("--agent", required=True, help="run_agent_info.csv of any pass")
    c.add_argument("--workload", required=True)
    c.add_argument("--command", required=True)
    c.add_argument("--out", required=True)
    sub.add_parser("digest")
    cb = sub.add_parser("copybw", help="read+write bandwidth of plain device copies (needs a GPU)")
    cb.add_argument("--out", default=None)
    pb = sub.add_parser("probes", help="matrix-core, exponential and atomic rates of the part (needs a GPU)")
    pb.add_argument("--out", default=None)
    md = sub.add_parser("modes", help="fused vs separate backward over a sweep of shapes, against the plan (needs a GPU)")
    md.add_argument("--out", default=None)
    md.add_argument("--ragged", action="store_true", help="ragged batches instead of single problems")
    pl = sub.add_parser("packed", help="ragged batches padded against packed (needs a GPU)")
    pl.add_argument("--out", default=None)
    args = ap.parse_args(argv)
    if args.cmd == "packed":
        text = layout_sweep()
        if args.out:
            with open(args.out, "w") as fo:
                fo.write(text)
        print(text)
        return 0
    if args.cmd == "modes":
        text = ragged_mode_sweep() if args.ragged else mode_sweep()
        if args.out:
            with open(args.out, "w") as fo:
                fo.write(text)
        print(text)
        return 0
    if args.cmd == "probes":
        text = device_probes()
        if args.out:
            with open(args.out, "w") as fo:
                fo.write(text)
        print(text)
        return 0
    if args.cmd == "copybw":
        text = copy_bandwidth()
        if args.out:
            with open(args.out, "w") as fo:
                fo.write(text)
        print(text)
        return 0
    if args.cmd == "counters":
        res, topo = counters(args.csv, args.agent)
        lines = [f"# SQ counters per kernel, workload {args.workload}", "",
                 "Commands (run from /tmp with TMPDIR=/tmp on one MI355X; one rocprofv3 --pmc pass per set):", "",
                 "```", args.command, "```", "",
                 f"Topology from the agent info: {topo['cus']} CUs, {topo['simds']} SIMDs, {topo['ses']} shader "
                 "engines.  Per dispatch: T = SQ_BUSY_CYCLES / engines; MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / "
                 "SIMDs / T; co-exec = SQ_VALU_MFMA_COEXEC_CYCLES / SIMDs / T (matrix cores busy while the VALU "
                 "issues); VALU issue = non-MFMA VALU instructions / SIMDs / T (ceiling 0.25 for fp32 wave64); "
                 "LDS wait = SQ_WAIT_INST_LDS / SQ_WAVE_CYCLES.", "",
                 "| kernel | T (cycles) | MFMA busy | co-exec | VALU issue / SIMD-cycle | LDS wait | MFMA instr | "
                 "VALU instr | exp2 instr | LDS instr |", "|---|---|---|---|---|---|---|---|---|---|"]
        for lab, d in sorted(res.items()):
            f = lambda k, fmt="{:.1%}": fmt.format(d[k]) if k in d else "-"  # noqa: E731
            lines.append(f"| {lab} | {d['dispatch_cycles']:.0f} | {f('mfma_busy')} | {f('mfma_valu_coexec')} | "
                         f"{f('valu_issue_per_simd_cycle', '{:.3f}')} | {f('lds_wait_share')} | "
                         f"{f('SQ_INSTS_MFMA', '{:.3g}')} | {f('SQ_INSTS_VALU', '{:.3g}')} | "
                         f"{f('SQ_INSTS_VALU_TRANS_F32', '{:.3g}')} | {f('SQ_INSTS_LDS', '{:.3g}')} |")
        lines += ["", "```json", json.dumps({"workload": args.workload, "source_digest": kernel_source_digest(),
                                              "kernels": res}, indent=1), "```", ""]
        with open(args.out, "w") as fo:
            fo.write("\n".join(lines))
        print(args.out)
        return 0
    if args.cmd == "digest":
        print(kernel_source_digest())
        return 0
    if args.cmd == "kernels":
        with open(args.out, "w") as f:
            f.write(kernel_summary(args.stats, args.bench_log, args.workload, args.command))
        print(args.out)
        return 0
    res, factors = traffic(args.fetch, args.write, args.copy_mib)
    block = {"workload": args.workload, "source_digest": kernel_source_digest(),
             "copy_reference_mib": args.copy_mib,
             "scale": {k: round(v, 5) for k, v in factors.items()},
             "kernels": {k: {kk: (round(vv) if kk != "launches" else vv) for kk, vv in v.items()}
                         for k, v in res.items()}}
    lines = [f"# HBM traffic per launch, workload {args.workload}", "",
             "Counters FETCH_SIZE and WRITE_SIZE (KiB per dispatch) from two separate",
             "rocprofv3 --pmc runs, each scaled by known/measured for a plain device",
             f"copy of {args.copy_mib} MiB launched in the same run "
             f"(FETCH scale {factors['FETCH_SIZE']:.4f}, WRITE scale {factors['WRITE_SIZE']:.4f}).", "",
             "Commands:", "", "```", args.command, "```", "",
             "FETCH_SIZE counts the L2 misses of each dispatch (served by the",
             "memory-side cache or HBM), WRITE_SIZE the bytes written back.", "",
             "| kernel | launches | read past L2 (MB) | written (MB) |", "|---|---|---|---|"]
    for k, v in sorted(res.items()):
        lines.append(f"| {k} | {v.get('launches', 0)} | {v.get('fetch_bytes', 0) / 1e6:.1f} | "
                     f"{v.get('write_bytes', 0) / 1e6:.1f} |")
    lines += ["", "```json", json.dumps(block, indent=1), "```", ""]
    with open(args.out, "w") as f:
        f.write("\n".join(lines))
    print(args.out)
    return 0


if __name__ == "__main__":
    sys.exit(main())
