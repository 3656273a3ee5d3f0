"""Test-only build of the host layer with AddressSanitizer and
UndefinedBehaviorSanitizer, for the host checks of the C ABI.

The host half of attention_kl_divergence_amd/csrc/api.hip (argument
validation, planning, workspace sizing, launch set-up) is compiled with the
sanitizers (host side only: every sanitizer flag on the hipcc line is
preceded by -Xarch_host, so device code is built as usual), then linked with
the kernel objects of the regular build and tests/abi_host_check.c into one
host program by clang++ (a host-only link line that names no .hip file).
It runs on a machine without a GPU: every call it makes fails validation
before touching a device, or only plans and sizes.

    python tests/host_check_build.py      # builds and runs it
"""
from __future__ import annotations

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

from attention_kl_divergence_amd import build as b  # noqa: E402

OUT = os.path.join(ROOT, "_build", "asan")
EXE = os.path.join(OUT, "abi_host_check")
CLANGXX = "/opt/rocm/llvm/bin/clang++"
SAN = ["address", "undefined"]


def build() -> str:
    insts = [os.path.join(b.BUILD, f"inst_{tn}_{d1}_{d2}.o") for _, tn, d1, d2 in b.VARIANTS]
    if not all(os.path.exists(o) for o in insts):
        b.build()
    os.makedirs(OUT, exist_ok=True)
    api = os.path.join(OUT, "api_san.o")
    host_san = []
    for s in SAN:
        host_san += ["-Xarch_host", f"-fsanitize={s}"]
    host_san += ["-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer",
                 "-Xarch_host", "-g"]
    flags = [f for f in b.FLAGS if f != "-fno-honor-nans"]
    b._run([b.HIPCC, *flags, *host_san, "-c", os.path.join(b.CSRC, "api.hip"), "-o", api])
    link = [CLANGXX, "-x", "c++", os.path.join(ROOT, "tests", "abi_host_check.c"), "-x", "none", api, *insts,
            "-I", os.path.join(ROOT, "include"), "-g", "-fno-omit-frame-pointer", "-fno-sanitize-recover=all",
            "-L/opt/rocm/lib", "-Wl,-rpath,/opt/rocm/lib", "-lamdhip64", "-o", EXE]
    link[1:1] = [f"-fsanitize={s}" for s in SAN]
    b._run(link)
    return EXE


def run() -> subprocess.CompletedProcess:
    env = dict(os.environ)
    # the HIP runtime's own start-up allocations are not the host layer's leaks
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    return subprocess.run([EXE], env=env, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, timeout=300)


if __name__ == "__main__":
    build()
    p = run()
    print(p.stdout)
    sys.exit(p.returncode)
