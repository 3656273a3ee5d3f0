"""Calls from several host threads at once.

The host layer keeps one shared table of device properties (filled once,
under a lock) and a per-thread last-HIP-error slot; everything else a call
needs lives on its stack.  ctypes releases the GIL for the duration of each
foreign call, so threads here enter the library concurrently.  Each thread
runs its own problem on its own stream (torch's current stream is per
thread); the results must be bitwise those of the same calls made one after
the other on one thread (the forward and the separate backward are
deterministic).
"""
import threading

import pytest
import torch

import workloads
from attention_kl_divergence_amd import streamkl as sk

pytestmark = pytest.mark.gpu


def _problem(i, dev):
    causal = i % 2 == 0
    n_q, n_k = (300 + 37 * i, 300 + 37 * i) if causal else (150 + 11 * i, 420 + 5 * i)
    d1, d2 = (128, 64) if i % 3 == 0 else (128, 128)
    w = workloads.Workload(f"thread{i}", 1, 2 + i % 3, n_q, n_k, d1, d2, "bf16", causal, 0.5, d1 != d2, 60 + i)
    q1, k1, q2, k2 = workloads.generate(w, dev)
    g = workloads.upstream_grad(w, dev, "random")
    return w, (q1, k1, q2, k2, g)


def _run(w, t):
    q1, k1, q2, k2, g = t
    kl, l1, l2 = sk.streamkl_fwd(q1, k1, q2, k2, w.causal, num_splits=1 + w.seed % 3)
    out = [kl, l1, l2]
    for setting in (1, 2):
        dq, dk = sk.streamkl_bwd(setting, q1, k1, q2, k2, w.causal, kl, l1, l2, g, bwd_mode=sk.BWD_SEPARATE)
        out += [dq, dk]
    return out


def test_concurrent_threads_match_sequential(cuda_device):
    n = 6
    probs = [_problem(i, cuda_device) for i in range(n)]
    ref = [_run(w, t) for w, t in probs]
    torch.cuda.synchronize()
    got = [None] * n
    errors = []
    start = threading.Barrier(n)

    def worker(i):
        try:
            torch.cuda.set_device(cuda_device)
            stream = torch.cuda.Stream()
            start.wait()
            with torch.cuda.stream(stream):
                for _ in range(3):
                    res = _run(*probs[i])
                stream.synchronize()
            got[i] = res
        except Exception as e:  # reported in the main thread
            errors.append((i, repr(e)))

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(n)]
    for th in threads:
        th.start()
    for th in threads:
        th.join(timeout=120)
    assert not any(th.is_alive() for th in threads), "a worker thread did not finish"
    assert not errors, errors
    for i in range(n):
        for j, (a, b) in enumerate(zip(got[i], ref[i])):
            assert torch.equal(a, b), f"{probs[i][0].name}: output {j} differs from the sequential run"
