"""Build libstreamkl.so (HIP, gfx950) in-tree with hipcc.

The kernels are instantiated per (dtype, d1, d2) in separate translation
units compiled in parallel, then linked with the C-ABI host layer into one
shared library next to this file.

    python -m attention_kl_divergence_amd.build [--jobs N]
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libstreamkl.so")
# device probes of the measurement side (matrix-core, exponential and atomic
# rates), a library of their own so the product's ABI stays the header's
PROBES = os.path.join(HERE, "libstreamkl_probes.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17",
    "-munsafe-fp-atomics",
    # keep MFMA accumulators in VGPRs (no accvgpr copies before the VALU softmax)
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    # no value in these kernels is NaN by design (masked lanes are selected
    # away), so max/min need no NaN-quieting and fold into v_max3_f32
    "-fno-honor-nans",
    # packed fp32 VALU forms are disabled for all device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]

VARIANTS = [
    ("float", "f32", 64, 64), ("float", "f32", 64, 128), ("float", "f32", 128, 64), ("float", "f32", 128, 128),
    ("__bf16", "bf16", 64, 64), ("__bf16", "bf16", 64, 128), ("__bf16", "bf16", 128, 64), ("__bf16", "bf16", 128, 128),
]


def _run(cmd):
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in p.stdout.splitlines() if "packed-fp32-ops" not in l)
    if p.returncode != 0:
        raise RuntimeError("command failed:\n" + " ".join(cmd) + "\n" + out)
    return out


def build(jobs: int | None = None, verbose: bool = False) -> str:
    if not os.path.exists(HIPCC):
        raise RuntimeError(f"hipcc not found at {HIPCC}")
    os.makedirs(BUILD, exist_ok=True)
    jobs = jobs or min(len(VARIANTS) + 1, os.cpu_count() or 4, 16)
    cmds, objs = [], []
    for t, tn, d1, d2 in VARIANTS:
        obj = os.path.join(BUILD, f"inst_{tn}_{d1}_{d2}.o")
        cmds.append([HIPCC, *FLAGS, f"-DSKL_T={t}", f"-DSKL_TN={tn}", f"-DSKL_D1={d1}", f"-DSKL_D2={d2}",
                     "-c", os.path.join(CSRC, "inst.hip"), "-o", obj])
        objs.append(obj)
    api_obj = os.path.join(BUILD, "api.o")
    # the host layer checks float arguments for NaN: it keeps IEEE NaN semantics
    cmds.append([HIPCC, *[f for f in FLAGS if f != "-fno-honor-nans"], "-c", os.path.join(CSRC, "api.hip"),
                 "-o", api_obj])
    objs.append(api_obj)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        outs = list(ex.map(_run, cmds))
    if verbose:
        for o in outs:
            if o.strip():
                print(o)
    tmp = LIB + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs])
    shutil.move(tmp, LIB)
    tmp = PROBES + ".tmp"
    _run([HIPCC, *[f for f in FLAGS if f != "-fno-honor-nans"], "-shared", os.path.join(CSRC, "probes.hip"),
          "-o", tmp])
    shutil.move(tmp, PROBES)
    return LIB


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=None)
    ap.add_argument("-v", "--verbose", action="store_true")
    args = ap.parse_args(argv)
    print(build(args.jobs, args.verbose))


if __name__ == "__main__":
    sys.exit(main())
