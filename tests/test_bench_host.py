"""Host-side logic of bench.py, without a GPU: the algorithmic byte counts the
roofline divides by, the traffic summary built from two rocprofv3 counter files,
the digest check that voids a stale summary, and the refusal of --gpus N > 1."""
import csv
import importlib.util
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_algorithmic_bytes_by_hand(bench):
    W = bench.WORKLOADS
    # MX 8192^3: codes of A and B, one E8M0 code per 32 elements of each, bf16 C
    assert bench.gemm_bytes(W["mx8192"]) == 2 * 8192 * 8192 + 2 * 8192 * 256 + 2 * 8192 * 8192
    # row-wise 4096^3: one fp32 scale per row of A and per row of B
    assert bench.gemm_bytes(W["rowwise4096"]) == 2 * 4096 * 4096 + 4 * 8192 + 2 * 4096 * 4096
    # M = 128, N = K = 4096, per-tensor: the 18.35 MB the skinny roofline uses
    sk = bench.gemm_bytes(W["skinny128"])
    assert sk == 128 * 4096 + 4096 * 4096 + 8 + 2 * 128 * 4096 == 18350088
    # grouped: every expert's weights and row scales
    g = W["grouped_moe"]
    assert bench.gemm_bytes(g) == (g.M * g.K + g.groups * g.N * g.K + 4 * (g.M + g.groups * g.N)
                                   + 2 * g.M * g.N)
    # FP4 codes take half a byte, the MX output one byte plus a code per 32 columns
    w = W["mx8192"]
    assert bench.gemm_bytes(w, 0.5) == 8192 * 8192 + 2 * 8192 * 256 + 2 * 8192 * 8192
    assert bench.gemm_bytes_mxout(w) == (bench.gemm_bytes(w) - 8192 * 8192 + 8192 * 256)
    assert bench.gemm_bytes_qout(w) == bench.gemm_bytes(w) - 8192 * 8192 + 4 * 8192


def _counter_csv(path, counter, rows):
    with open(path, "w", newline="") as fh:
        wr = csv.DictWriter(fh, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name",
                                            "Counter_Value"])
        wr.writeheader()
        for i, (name, value) in enumerate(rows):
            wr.writerow({"Dispatch_Id": i, "Kernel_Name": name, "Counter_Name": counter,
                         "Counter_Value": value})


def test_traffic_summary_scales_by_the_copy(bench, tmp_path, monkeypatch):
    """The GEMM's mean FETCH_SIZE / WRITE_SIZE (KiB) is scaled so that the three
    1 GiB calibration copies (the copy kernel's largest dispatches) count 1 GiB
    each; the copy's small dispatches and other kernels are ignored."""
    gemm = "void fp8gemm::(anonymous namespace)::gemm_kernel<Cfg>(fp8gemm::GemmProblem, int, int)"
    copy = "__amd_rocclr_copyBuffer"
    other = "fp8gemm::quant_mx_kernel<0>"
    gib_kib = (1 << 30) / 1024
    fetch = [(gemm, 1000.0), (gemm, 1200.0), (copy, 4.0), (other, 99.0)] + \
            [(copy, gib_kib / 2)] * 3
    write = [(gemm, 300.0), (gemm, 500.0), (copy, 2.0), (other, 7.0)] + [(copy, gib_kib)] * 3
    f, w = tmp_path / "f.csv", tmp_path / "w.csv"
    _counter_csv(f, "FETCH_SIZE", fetch)
    _counter_csv(w, "WRITE_SIZE", write)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "kernel_source_digest", lambda: "d1g35t")
    bench.summarize_traffic("mx8192", str(f), str(w), command="cmd")
    rec = json.load(open(tmp_path / "profiles" / "gemm_mx8192_traffic.json"))
    assert rec["kernel"] == gemm and rec["gemm_dispatches"] == 2
    assert rec["fetch_scale"] == 2.0 and rec["write_scale"] == 1.0
    assert rec["hbm_fetch_bytes_per_launch"] == 1100 * 1024 * 2
    assert rec["hbm_write_bytes_per_launch"] == 400 * 1024
    assert rec["hbm_bytes_per_launch"] == 1100 * 2048 + 400 * 1024
    assert rec["kernel_source_digest"] == "d1g35t" and rec["command"] == "cmd"
    # the bench reads the figure back while the digest matches, and drops it after
    assert bench.measured_traffic("mx8192") == rec["hbm_bytes_per_launch"]
    monkeypatch.setattr(bench, "kernel_source_digest", lambda: "changed")
    assert bench.measured_traffic("mx8192") is None
    assert bench.measured_traffic("rowwise4096") is None        # no summary at all


def test_traffic_summary_needs_one_gemm_and_one_copy(bench, tmp_path, monkeypatch):
    f, w = tmp_path / "f.csv", tmp_path / "w.csv"
    _counter_csv(f, "FETCH_SIZE", [("fp8gemm::quant_row_kernel<1, 0>", 1.0)])
    _counter_csv(w, "WRITE_SIZE", [("fp8gemm::quant_row_kernel<1, 0>", 1.0)])
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    with pytest.raises(SystemExit):
        bench.summarize_traffic("mx8192", str(f), str(w), command="")
    assert not (tmp_path / "profiles").exists()


def test_committed_summaries_match_the_kernel_sources(bench):
    """Every committed traffic summary was taken on the kernel sources in the tree
    (otherwise the bench reports traffic null)."""
    digest = bench.kernel_source_digest()
    stale = []
    for w in ("mx8192", "rowwise4096", "skinny128", "grouped_moe"):
        rec = json.load(open(os.path.join(ROOT, "profiles", f"gemm_{w}_traffic.json")))
        assert rec["hbm_bytes_per_launch"] == rec["hbm_fetch_bytes_per_launch"] + \
            rec["hbm_write_bytes_per_launch"]
        if rec["kernel_source_digest"] != digest:
            stale.append(w)
    if stale:
        pytest.skip(f"kernel sources changed since the counters of {stale} were taken "
                    "(the bench reports traffic null for them until they are taken again)")


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and not r.stdout.strip()
