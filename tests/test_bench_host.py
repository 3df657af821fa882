"""Host-side logic of bench.py (no GPU): the one-GPU rule and the HBM-traffic
calibration that turns rocprofv3 FETCH_SIZE / WRITE_SIZE readings into bytes."""
import csv
import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def _counter_dir(tmp_path, name, rows):
    d = tmp_path / name
    d.mkdir()
    with open(d / "run_counter_collection.csv", "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for kernel, value in rows:
            w.writerow({"Kernel_Name": kernel, "Counter_Name": name, "Counter_Value": value})
    return str(d)


def test_record_traffic_scales_each_counter_by_the_copy(tmp_path, monkeypatch):
    # The calibration copy moves COPY_BYTES each way.  Here FETCH_SIZE reads
    # half of that for the copy (factor 2) and WRITE_SIZE all of it (factor 1);
    # the pass reads as 3000 and 1500 KiB on its two launches (mean 2250).
    copy_kib = bench.COPY_BYTES / 1024
    fetch = _counter_dir(tmp_path, "FETCH_SIZE", [
        ("__amd_rocclr_copyBuffer", copy_kib / 2),
        ("void rs::(anonymous namespace)::onesweep_kernel<1024, 28, 1, true, false, false>(PassArgs)", 3000.0),
        ("void rs::(anonymous namespace)::onesweep_kernel<1024, 28, 1, true, false, false>(PassArgs)", 1500.0),
        ("void rs::(anonymous namespace)::upsweep_kernel<false>(...)", 100.0)])
    write = _counter_dir(tmp_path, "WRITE_SIZE", [
        ("__amd_rocclr_copyBuffer", copy_kib),
        ("void rs::(anonymous namespace)::onesweep_kernel<1024, 28, 1, true, false, false>(PassArgs)", 4000.0),
        ("void rs::(anonymous namespace)::upsweep_kernel<false>(...)", 1.0)])
    out = tmp_path / "traffic.json"
    out.write_text(json.dumps({"other_workload": {"kept": True}}))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(out))
    bench.record_traffic("pairs_u32_2p28", fetch, write)
    table = json.loads(out.read_text())
    assert table["other_workload"] == {"kept": True}
    e = table["pairs_u32_2p28"]
    assert e["kernel"] == "onesweep"
    assert e["calibration"]["fetch_factor"] == 2.0 and e["calibration"]["write_factor"] == 1.0
    assert e["fetch_bytes_per_launch"] == 2250 * 1024 * 2
    assert e["write_bytes_per_launch"] == 4000 * 1024
    assert e["traffic_bytes_per_launch"] == 2250 * 1024 * 2 + 4000 * 1024
    assert e["upsweep_fetch_bytes_per_launch"] == 100 * 1024 * 2
    assert e["algorithmic_bytes_per_launch"] == 16 * (1 << 28)
    assert e["source_sha"] == bench.source_hash()


def test_source_hash_is_stable_and_short():
    h = bench.source_hash()
    assert h == bench.source_hash()
    assert len(h) == 16 and all(c in "0123456789abcdef" for c in h)
