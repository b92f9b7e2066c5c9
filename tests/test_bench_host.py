"""CPU tests of bench.py's host logic: the single-GPU guard and the
calibration of rocprofv3 counter runs into HBM bytes."""
import csv
import importlib.util
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


@pytest.mark.parametrize("argv", [["--gpus", "2"], ["--gpus", "8"]])
def test_more_than_one_gpu_is_refused(argv):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *argv], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "single GPU" in r.stderr
    assert r.stdout == ""


def _write_run(d, counter, rows):
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "run_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for i, (name, vals) in enumerate(rows):
            for v in vals:  # one row per shader engine / instance, summed per dispatch
                w.writerow({"Dispatch_Id": i, "Kernel_Name": name, "Counter_Name": counter, "Counter_Value": v})


def test_traffic_summary_calibrates_by_the_copy(tmp_path, monkeypatch):
    """A copy of N MiB that reads as N/2 MiB of FETCH_SIZE gives factor 2; the
    split's per-dispatch KiB (summed over instances, averaged over launches)
    are scaled by it; counters of other kernels are ignored."""
    b = _bench()
    monkeypatch.setattr(b, "PROFILE_DIR", str(tmp_path))
    calib_mib = 4
    copy = ("void at::native::elementwise_kernel<...>", [calib_mib * 1024 / 4] * 2)   # reads half
    fetch_rows = [copy] * 6 + [("split_mfma_kernel<128, 2, false, 4>", [100.0, 50.0]),
                               ("split_mfma_kernel<128, 2, false, 4>", [110.0, 40.0]),
                               ("quantize_tile_kernel", [9999.0])]
    write_rows = [("void at::native::elementwise_kernel<...>", [calib_mib * 1024.0])] * 5 + \
                 [("split_mfma_kernel<128, 2, false, 4>", [8.0]), ("split_mfma_kernel<128, 2, false, 4>", [12.0])]
    _write_run(str(tmp_path / "fetch"), "FETCH_SIZE", fetch_rows)
    _write_run(str(tmp_path / "write"), "WRITE_SIZE", write_rows)
    b.traffic_summary(str(tmp_path / "fetch"), str(tmp_path / "write"), 3, calib_mib, "cmds")
    from int4_kv_cache_quant_amd import synth
    rec = json.load(open(tmp_path / f"traffic_split_mfma_{synth.WORKLOADS[3].name}.json"))
    assert rec["fetch_factor"] == pytest.approx(2.0)
    assert rec["fetch_kib_per_launch_raw"] == pytest.approx(150.0)
    assert rec["fetch_bytes_per_launch"] == pytest.approx(150.0 * 2.0 * 1024)
    assert rec["write_factor"] == pytest.approx(1.0)
    assert rec["write_bytes_per_launch"] == pytest.approx(10.0 * 1024)
    assert rec["hbm_bytes_per_launch"] == pytest.approx(150.0 * 2.0 * 1024 + 10.0 * 1024)
    assert rec["fetch_launches"] == 2 and rec["write_launches"] == 2
    # workload 3: 131072 tokens x 8 KV heads x (64 + 16) bytes for K and V, and q
    assert rec["algorithmic_bytes_per_launch"] == 131072 * 8 * 2 * (64 + 16) + 64 * 128 * 2
    assert rec["kernel_source_sha"] == b.source_sha("split_mfma")
    # the bench reads it back only while the kernel source is unchanged
    assert b.traffic_from_profile("split_mfma", synth.WORKLOADS[3].name) == pytest.approx(rec["hbm_bytes_per_launch"])
    rec["kernel_source_sha"] = "0" * 16
    json.dump(rec, open(tmp_path / f"traffic_split_mfma_{synth.WORKLOADS[3].name}.json", "w"))
    assert b.traffic_from_profile("split_mfma", synth.WORKLOADS[3].name) is None


def test_traffic_summary_of_the_b_bit_split(tmp_path, monkeypatch):
    """The same calibration for the 2-bit MFMA split: its own dispatches, its
    algorithmic bytes (D/4 bytes of codes per token and head), its own file."""
    b = _bench()
    monkeypatch.setattr(b, "PROFILE_DIR", str(tmp_path))
    copy = ("void at::native::elementwise_kernel<...>", [1024.0])
    fetch_rows = [copy] * 5 + [("split_bits_mfma_kernel<128, 2>", [300.0]), ("split_mfma_kernel<128, 2, false, 4>", [1.0])]
    write_rows = [copy] * 5 + [("split_bits_mfma_kernel<128, 2>", [4.0])]
    _write_run(str(tmp_path / "fetch"), "FETCH_SIZE", fetch_rows)
    _write_run(str(tmp_path / "write"), "WRITE_SIZE", write_rows)
    b.traffic_summary(str(tmp_path / "fetch"), str(tmp_path / "write"), 3, 1, "cmds", "split_bits_mfma", 2)
    from int4_kv_cache_quant_amd import synth
    rec = json.load(open(tmp_path / f"traffic_split_bits_mfma_{synth.WORKLOADS[3].name}-2bit.json"))
    assert rec["fetch_kib_per_launch_raw"] == pytest.approx(300.0) and rec["fetch_launches"] == 1
    assert rec["algorithmic_bytes_per_launch"] == 131072 * 8 * 2 * (32 + 16) + 64 * 128 * 2
    assert rec["kernel_source_sha"] == b.source_sha("split_bits_mfma")
    assert b.traffic_from_profile("split_bits_mfma", synth.WORKLOADS[3].name, 2) == pytest.approx(
        rec["hbm_bytes_per_launch"])


def test_traffic_summary_needs_the_calibration_copy(tmp_path, monkeypatch):
    b = _bench()
    monkeypatch.setattr(b, "PROFILE_DIR", str(tmp_path))
    _write_run(str(tmp_path / "fetch"), "FETCH_SIZE", [("split_mfma_kernel", [1.0])])
    _write_run(str(tmp_path / "write"), "WRITE_SIZE", [("split_mfma_kernel", [1.0])])
    with pytest.raises(SystemExit):
        b.traffic_summary(str(tmp_path / "fetch"), str(tmp_path / "write"), 3, 4, "")


def test_committed_traffic_reads_the_cache_once():
    """The committed counter summary of the split kernel: fetched bytes within
    2% of the algorithmic bytes (skipped while the summary predates the
    current split source, which the bench then reports as null traffic)."""
    b = _bench()
    from int4_kv_cache_quant_amd import synth
    path = os.path.join(ROOT, "profiles", f"traffic_split_mfma_{synth.WORKLOADS[3].name}.json")
    rec = json.load(open(path))
    if rec["kernel_source_sha"] != b.source_sha("split_mfma"):
        pytest.skip("the counter summary predates the current split kernel source")
    assert 1.0 <= rec["fetch_bytes_per_launch"] / rec["algorithmic_bytes_per_launch"] < 1.02
