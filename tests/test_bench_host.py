"""bench.py's host-side logic, without a GPU: the one-GPU guard, the source files a counter
record is tied to, the traffic lookup, and the summary of rocprofv3 FETCH_SIZE / WRITE_SIZE
runs into the traffic record (on synthetic counter files, written to a temporary record)."""
import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=60)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


@pytest.mark.parametrize("kernel", ["gemm_qkv", "attention", "gemm_o_resid", "layernorm",
                                    "gemm_ffn1_gelu", "gemm_ffn2_resid", "ln2_reduce",
                                    "attention_half", "ln2_mlp_resid", "window_attention"])
def test_kernel_sources_exist_and_digest_is_stable(kernel):
    files = bench.kernel_sources(kernel)
    assert all(os.path.isfile(os.path.join(ROOT, f)) for f in files)
    assert any(f.endswith(".hip") for f in files)
    d = bench.kernel_sources_digest(kernel)
    assert len(d) == 64 and d == bench.kernel_sources_digest(kernel)


def test_traffic_record_is_well_formed():
    with open(os.path.join(ROOT, "profiles", "hbm_traffic.json")) as f:
        rec = json.load(f)
    assert rec["calibration"]["fetch_factor"] > 0 and rec["calibration"]["write_factor"] > 0
    for k in rec["kernels"]:
        assert k["bytes_per_launch"] > 0 and k["algorithmic_bytes"] > 0
        assert abs(k["ratio"] - k["bytes_per_launch"] / k["algorithmic_bytes"]) < 0.01
        assert len(k["sources_sha256"]) == 64
    # a record of another workload, or one whose sources changed, is not reported
    assert bench.measured_traffic("no_such_workload", "f16", "gemm_qkv") is None


def _counter_dir(tmp, name, counter, rows):
    d = tmp / name
    d.mkdir()
    with open(d / "bench_counter_collection.csv", "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name",
                                          "Counter_Value"])
        w.writeheader()
        for i, (kname, v) in enumerate(rows):
            # two rows per dispatch (e.g. two counter instances): the summary adds them
            w.writerow(dict(Dispatch_Id=i, Kernel_Name=kname, Counter_Name=counter,
                            Counter_Value=v / 2))
            w.writerow(dict(Dispatch_Id=i, Kernel_Name=kname, Counter_Name=counter,
                            Counter_Value=v / 2))
    return str(d)


def test_summarise_traffic_scales_by_the_calibration_copy(tmp_path, monkeypatch):
    """Two kernels, each launched once untimed and twice timed (reps 2), then three 256 MiB
    copies: the counters are averaged over the timed launches and scaled so that a copy reads
    and writes exactly 256 MiB."""
    table = {"workload": "synthetic", "dtype": "f16", "reps": 2,
             "kernels": [{"name": "gemm_qkv", "bytes": 1000.0},
                         {"name": "attention", "bytes": 3000.0}]}
    tpath = tmp_path / "table.json"
    tpath.write_text(json.dumps(table))
    k1, k2 = "_ZN3tel_gemm_a", "_ZN3tel_attn_b"
    # the copies count half of 256 MiB on FETCH and a quarter on WRITE: factors 2 and 4
    fetch = [(k1, 999.0), (k1, 10.0), (k1, 30.0), (k2, 999.0), (k2, 50.0), (k2, 50.0)] + \
        [("__amd_rocclr_copyBuffer", 128 * 1024.0)] * 3
    write = [(k1, 999.0), (k1, 1.0), (k1, 1.0), (k2, 999.0), (k2, 2.0), (k2, 4.0)] + \
        [("__amd_rocclr_copyBuffer", 64 * 1024.0)] * 3
    fdir = _counter_dir(tmp_path, "fetch", "FETCH_SIZE", fetch)
    wdir = _counter_dir(tmp_path, "write", "WRITE_SIZE", write)
    out = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_JSON", str(out))
    bench.summarise_traffic(fdir, wdir, str(tpath))
    rec = json.loads(out.read_text())
    assert rec["calibration"]["fetch_factor"] == pytest.approx(2.0)
    assert rec["calibration"]["write_factor"] == pytest.approx(4.0)
    by = {k["kernel"]: k for k in rec["kernels"]}
    # gemm: fetch (10 + 30) / 2 = 20 KiB x 2, write 1 KiB x 4 -> 44 KiB
    assert by["gemm_qkv"]["bytes_per_launch"] == 44 * 1024
    assert by["gemm_qkv"]["symbol"] == k1
    # attention: fetch 50 KiB x 2, write 3 KiB x 4 -> 112 KiB
    assert by["attention"]["bytes_per_launch"] == 112 * 1024
    assert by["attention"]["sources_sha256"] == bench.kernel_sources_digest("attention")
