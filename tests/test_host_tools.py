"""Host-side tools: the traffic calibration behind roofline.traffic, the
summary format the benchmark reads back, and the benchmark's one-GPU guard."""
import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

from attention_kl_divergence_amd import build, profiling  # noqa: E402

FIELDS = ["Correlation_Id", "Dispatch_Id", "Agent_Id", "Queue_Id", "Process_Id", "Thread_Id", "Grid_Size",
          "Kernel_Id", "Kernel_Name", "Workgroup_Size", "LDS_Block_Size", "Scratch_Size", "VGPR_Count",
          "Accum_VGPR_Count", "SGPR_Count", "Counter_Name", "Counter_Value", "Start_Timestamp", "End_Timestamp"]

MUL = "void at::native::vectorized_elementwise_kernel<4, at::native::BinaryFunctor<float, float, float, " \
      "at::native::binary_internal::MulFunctor<float> >, std::array<char*, 3ul> >"
DK = "_ZN8streamkl13bwd_dk_kernelIDF16bLi128ELi128ELi1ELb0ELi64EEEvNS_7BwdArgsE"
DK_FUSED = "_ZN8streamkl13bwd_dk_kernelIDF16bLi128ELi128ELi1ELb1ELi64EEEvNS_7BwdArgsE"
FWD_PP = "_ZN8streamkl13fwd_pp_kernelIDF16bLi128ELi128ELi64EEEvNS_7FwdArgsE"
FWD = "_ZN8streamkl10fwd_kernelIDF16bLi128ELi128ELi64EEEvNS_7FwdArgsE"
DEC = "void streamkl::fwd_decode_kernel<128, 128>(streamkl::FwdArgs)"


def write_csv(path, counter, rows):
    """rows: (dispatch id, kernel name, [values per counter instance]) in KiB."""
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=FIELDS)
        w.writeheader()
        for d, name, vals in rows:
            for v in vals:
                w.writerow({k: 0 for k in FIELDS} | {"Dispatch_Id": d, "Kernel_Name": name,
                                                     "Counter_Name": counter, "Counter_Value": v})


def test_traffic_calibration(tmp_path):
    # 1024 MiB reference copy: FETCH reads half (scale 2), WRITE reads it exactly (scale 1);
    # an earlier, smaller MulFunctor must not be taken as the reference, and a
    # dispatch's instances are summed
    fetch = tmp_path / "f.csv"
    write = tmp_path / "w.csv"
    write_csv(fetch, "FETCH_SIZE", [(1, MUL, [100.0]), (2, MUL, [262144.0, 262144.0]),
                                    (3, DK, [1000.0]), (4, DK, [3000.0]), (5, FWD_PP, [50.0]),
                                    (6, DK_FUSED, [7.0]), (7, FWD, [9.0]), (8, DEC, [11.0])])
    write_csv(write, "WRITE_SIZE", [(1, MUL, [10.0]), (2, MUL, [1048576.0]),
                                    (3, DK, [64.0]), (4, DK, [64.0]), (5, FWD_PP, [2.0]),
                                    (6, DK_FUSED, [1.0]), (7, FWD, [3.0]), (8, DEC, [5.0])])
    res, factors = profiling.traffic(str(fetch), str(write), 1024)
    assert factors["FETCH_SIZE"] == pytest.approx(2.0)
    assert factors["WRITE_SIZE"] == pytest.approx(1.0)
    assert res["bwd_dk_kernel"]["launches"] == 2
    assert res["bwd_dk_kernel"]["fetch_bytes"] == pytest.approx(2.0 * 2000.0 * 1024)
    assert res["bwd_dk_kernel"]["write_bytes"] == pytest.approx(64.0 * 1024)
    assert res["fwd_pp_kernel"]["fetch_bytes"] == pytest.approx(2.0 * 50.0 * 1024)
    # the fused key-outer kernel and the plain forward get their own labels
    assert res["bwd_dk_kernel<FUSED>"]["fetch_bytes"] == pytest.approx(2.0 * 7.0 * 1024)
    assert res["fwd_kernel"]["write_bytes"] == pytest.approx(3.0 * 1024)
    # the decode forward (demangled name) is not taken for the plain forward
    assert res["fwd_decode_kernel"]["fetch_bytes"] == pytest.approx(2.0 * 11.0 * 1024)
    assert res["fwd_kernel"]["launches"] == 1


def test_traffic_needs_a_reference_copy(tmp_path):
    fetch = tmp_path / "f.csv"
    write_csv(fetch, "FETCH_SIZE", [(1, DK, [1.0])])
    with pytest.raises(SystemExit):
        profiling.traffic(str(fetch), str(fetch), 1024)


def test_summary_round_trip(tmp_path, monkeypatch):
    fetch = tmp_path / "f.csv"
    write = tmp_path / "w.csv"
    write_csv(fetch, "FETCH_SIZE", [(1, MUL, [524288.0]), (2, DK, [10.0])])
    write_csv(write, "WRITE_SIZE", [(1, MUL, [1048576.0]), (2, DK, [5.0])])
    out = tmp_path / "traffic_wl.md"
    assert profiling.main(["traffic", "--fetch", str(fetch), "--write", str(write), "--copy-mib", "1024",
                           "--workload", "wl", "--command", "cmd", "--out", str(out)]) == 0
    monkeypatch.setattr(profiling, "PROFILES", str(tmp_path))
    summ = profiling.load_summary("wl")
    assert summ["workload"] == "wl"
    assert summ["source_digest"] == profiling.kernel_source_digest()
    assert summ["kernels"]["bwd_dk_kernel"]["fetch_bytes"] == 20 * 1024
    assert summ["kernels"]["bwd_dk_kernel"]["write_bytes"] == 5 * 1024
    assert profiling.load_summary("missing") is None


def test_source_digest_tracks_device_flags(monkeypatch):
    d0 = profiling.kernel_source_digest()
    assert d0 == profiling.kernel_source_digest()
    monkeypatch.setattr(build, "FLAGS", build.FLAGS + ["-DSOMETHING_ELSE"])
    assert profiling.kernel_source_digest() != d0


def test_committed_summaries_parse():
    for name in os.listdir(os.path.join(ROOT, "profiles")):
        if name.startswith("traffic_") and name.endswith(".md"):
            summ = profiling.load_summary(name[len("traffic_"):-len(".md")])
            assert summ is not None and summ["kernels"], name
            assert summ["scale"]["FETCH_SIZE"] > 0 and summ["scale"]["WRITE_SIZE"] > 0


def test_bench_refuses_more_than_one_gpu():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert p.returncode == 2
    msg = json.loads(p.stdout.strip().splitlines()[-1])
    assert "one GPU" in msg["error"]


def test_counter_utilisations(tmp_path):
    # 4 CUs x 4 SIMDs, 2 shader engines; one dK dispatch per pass
    agent = tmp_path / "agent.csv"
    with open(agent, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Agent_Type", "Cu_Count", "Simd_Per_Cu", "Num_Shader_Banks"])
        w.writeheader()
        w.writerow({"Agent_Type": "CPU", "Cu_Count": 0, "Simd_Per_Cu": 0, "Num_Shader_Banks": 0})
        w.writerow({"Agent_Type": "GPU", "Cu_Count": 4, "Simd_Per_Cu": 4, "Num_Shader_Banks": 2})
    p1 = tmp_path / "p1.csv"
    p2 = tmp_path / "p2.csv"
    with open(p1, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=FIELDS)
        w.writeheader()
        for name, v in (("SQ_BUSY_CYCLES", 2000.0), ("SQ_VALU_MFMA_BUSY_CYCLES", 8000.0), ("SQ_INSTS_MFMA", 250.0),
                        ("SQ_INSTS_VALU", 1050.0), ("SQ_WAVE_CYCLES", 4000.0)):
            w.writerow({k: 0 for k in FIELDS} | {"Dispatch_Id": 3, "Kernel_Name": DK, "Counter_Name": name,
                                                 "Counter_Value": v})
    with open(p2, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=FIELDS)
        w.writeheader()
        for name, v in (("SQ_VALU_MFMA_COEXEC_CYCLES", 1600.0), ("SQ_WAIT_INST_LDS", 400.0)):
            w.writerow({k: 0 for k in FIELDS} | {"Dispatch_Id": 3, "Kernel_Name": DK, "Counter_Name": name,
                                                 "Counter_Value": v})
    res, topo = profiling.counters([str(p1), str(p2)], str(agent))
    assert topo == {"cus": 4, "simds": 16, "ses": 2}
    d = res["bwd_dk_kernel"]
    assert d["dispatch_cycles"] == pytest.approx(1000.0)          # 2000 / 2 engines
    assert d["mfma_busy"] == pytest.approx(0.5)                   # 8000 / 16 SIMDs / 1000
    assert d["mfma_valu_coexec"] == pytest.approx(0.1)
    assert d["valu_issue_per_simd_cycle"] == pytest.approx(0.05)  # (1050 - 250) / 16 / 1000
    assert d["lds_wait_share"] == pytest.approx(0.1)


@pytest.mark.parametrize("name,label", [
    ("_ZN8streamkl13bwd_dk_kernelIDF16bLi128ELi128ELi3ELb0ELi64EEEvNS_7BwdArgsE", "bwd_dk_kernel<JOINT>"),
    ("void streamkl::bwd_dk_kernel<__bf16, 128, 128, 3, false, 64>(streamkl::BwdArgs)", "bwd_dk_kernel<JOINT>"),
    ("void streamkl::bwd_dk_kernel<__bf16, 128, 128, 1, false, 64>(streamkl::BwdArgs)", "bwd_dk_kernel"),
    ("void streamkl::bwd_dk_kernel<__bf16, 128, 128, 2, true, 64>(streamkl::BwdArgs)", "bwd_dk_kernel<FUSED>"),
    ("void streamkl::bwd_decode_kernel<128, 128, 1>(streamkl::BwdArgs)", "bwd_decode_kernel"),
    ("void streamkl::fwd_decode_kernel<128, 128>(streamkl::FwdArgs)", "fwd_decode_kernel"),
    ("_ZN8streamkl13bwd_dq_kernelIDF16bLi128ELi128ELi1ELi64EEEvNS_7BwdArgsE", "bwd_dq_kernel"),
])
def test_kernel_labels(name, label):
    """Each library kernel's profiler name maps to the label its traffic and
    time are reported under (the joint and fused dK kernels apart from the
    plain one)."""
    assert profiling._label(name) == label


def test_bench_pair_counts():
    """Visible pairs: causal N(N+1)/2 per head, rectangular bottom-right
    causal, and per-sequence lengths for ragged workloads."""
    sys.path.insert(0, ROOT)
    import bench
    import workloads
    w = workloads.WORKLOADS["h32-n64k-d128-bf16-causal"]
    assert bench.pairs_of(w) == 32 * 65536 * 65537 // 2
    r = w.with_(n_q=100, n_k=333)
    assert bench.pairs_of(r) == 32 * (100 * 101 // 2 + 100 * 233)
    assert bench.pairs_of(w.with_(causal=False, n_q=7, n_k=9)) == 32 * 63
    rag = workloads.WORKLOADS["ragged-b4-h32-n32k-d128-bf16-causal"]
    assert bench.pairs_of(rag) == 32 * sum(n * (n + 1) // 2 for n in (8192, 16384, 4096, 32768))
    # grouped key heads do not change the pairs
    assert bench.pairs_of(workloads.WORKLOADS["h32-kv8-n64k-d128-bf16-causal"]) == bench.pairs_of(w)
