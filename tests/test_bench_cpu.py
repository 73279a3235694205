"""bench.py's host-side pieces, on the CPU: the counter summary (scaling by the calibration
copy, instruction counts per symbol), stale-profile detection, and the one-GPU guard."""
import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

pytestmark = pytest.mark.filterwarnings("ignore")


def _write_counters(path, workload, rows):
    os.makedirs(path, exist_ok=True)
    with open(os.path.join(path, f"{workload}_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Grid_Size", "Counter_Name",
                                          "Counter_Value"])
        w.writeheader()
        for r in rows:
            w.writerow(r)


def test_summarize_counters_scales_by_the_calibration_copy(tmp_path):
    wl = "tiny"
    prof = tmp_path / "prof"
    copy_grid = (256 << 20) // 2048
    # FETCH_SIZE reads half of the copy's 256 MiB, WRITE_SIZE all of it.  The calibration
    # copies come after the last decode; a copy with the same grid before it is another copy
    _write_counters(prof / f"pmc_FETCH_SIZE_{wl}", wl, [
        {"Dispatch_Id": 1, "Kernel_Name": "__amd_rocclr_copyBuffer", "Grid_Size": copy_grid,
         "Counter_Name": "FETCH_SIZE", "Counter_Value": 2907.0},
        {"Dispatch_Id": 2, "Kernel_Name": "__amd_rocclr_copyBuffer", "Grid_Size": 64,
         "Counter_Name": "FETCH_SIZE", "Counter_Value": 9.0},
        {"Dispatch_Id": 3, "Kernel_Name": "void shn::k_decode<1, shn::Bytes, shn::KSegs<1> >(x)",
         "Grid_Size": 1024, "Counter_Name": "FETCH_SIZE", "Counter_Value": 100.0},
        {"Dispatch_Id": 4, "Kernel_Name": "void shn::k_decode<1, shn::Bytes, shn::KSegs<1> >(x)",
         "Grid_Size": 1024, "Counter_Name": "FETCH_SIZE", "Counter_Value": 300.0},
        {"Dispatch_Id": 5, "Kernel_Name": "__amd_rocclr_copyBuffer", "Grid_Size": copy_grid,
         "Counter_Name": "FETCH_SIZE", "Counter_Value": 131072.0}])
    _write_counters(prof / f"pmc_WRITE_SIZE_{wl}", wl, [
        {"Dispatch_Id": 1, "Kernel_Name": "__amd_rocclr_copyBuffer", "Grid_Size": copy_grid,
         "Counter_Name": "WRITE_SIZE", "Counter_Value": 5789.0},
        {"Dispatch_Id": 3, "Kernel_Name": "void shn::k_decode<1, shn::Bytes, shn::KSegs<1> >(x)",
         "Grid_Size": 1024, "Counter_Name": "WRITE_SIZE", "Counter_Value": 64.0},
        {"Dispatch_Id": 5, "Kernel_Name": "__amd_rocclr_copyBuffer", "Grid_Size": copy_grid,
         "Counter_Name": "WRITE_SIZE", "Counter_Value": 262144.0}])
    n = sum(x.size for x in bench.make_segments(wl))
    _write_counters(prof / f"pmc_SQ_{wl}", wl, [
        {"Dispatch_Id": 1, "Kernel_Name": "void shn::k_decode<1, shn::Bytes, shn::KSegs<1> >(x)",
         "Grid_Size": 1024, "Counter_Name": "SQ_INSTS_VALU", "Counter_Value": float(n)},
        {"Dispatch_Id": 2, "Kernel_Name": "void shn::k_encode_chunks<1>(x)", "Grid_Size": 1024,
         "Counter_Name": "SQ_INSTS_VALU", "Counter_Value": float(2 * n)}])
    out = tmp_path / "out"
    os.makedirs(out)
    bench.summarize_counters(wl, str(prof), str(out))
    rec = json.load(open(out / f"decode_traffic_{wl}.json"))
    assert rec["FETCH_SIZE"]["scale"] == pytest.approx(2.0)
    assert rec["WRITE_SIZE"]["scale"] == pytest.approx(1.0)
    # (mean 200 KiB x 2 + 64 KiB x 1) in bytes
    assert rec["hbm_bytes_per_launch"] == pytest.approx((200.0 * 2 + 64.0) * 1024)
    assert rec["kernel"] == "k_decode"   # the tiny workload's one launch has 16 chunks
    assert rec["instructions"]["k_decode"]["valu_per_symbol"] == pytest.approx(64.0)
    assert rec["instructions"]["k_encode_chunks"]["valu_per_symbol"] == pytest.approx(128.0)
    assert rec["kernels_sha256_16"] == bench.kernels_hash(wl)


def test_profiles_taken_from_other_sources_are_ignored(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    os.makedirs(tmp_path / "profiles")
    with open(tmp_path / "profiles" / "decode_traffic_weight.json", "w") as f:
        json.dump({"kernels_sha256_16": "not-this-source", "hbm_bytes_per_launch": 1.0}, f)
    monkeypatch.setattr(bench, "kernels_hash", lambda workload="model": "this-source")
    assert bench.traffic_from_profile("weight") is None
    with open(tmp_path / "profiles" / "decode_traffic_weight.json", "w") as f:
        json.dump({"kernels_sha256_16": "this-source", "hbm_bytes_per_launch": 5.0,
                   "instructions": {"k_decode": {"valu_per_symbol": 19.5}}}, f)
    assert bench.traffic_from_profile("weight") == 5.0
    assert bench.valu_per_symbol_from_profile("weight") == 19.5


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert line["n_gpus"] == 2 and "one GPU" in line["error"]


def test_decode_kernel_follows_the_launch_size():
    """The library decodes launches below 16,384 chunks with the half-wavefront kernel and
    larger ones with the row kernel; bench.py names (and profiles) the one a workload runs."""
    assert bench.launch_chunks("weight") == 1024
    assert bench.launch_chunks("kv_cache") == 16 * 512
    assert bench.launch_chunks("model") >= bench.HALF_DECODE_MAX_CHUNKS
    assert bench.decode_kernel("weight")["name"] == "k_decode"
    assert bench.decode_kernel("model")["name"] == "k_decode_rows"
    assert bench.kernels_hash("weight") != bench.kernels_hash("model")
