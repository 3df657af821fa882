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


def test_output_checks_accept_correct_and_reject_broken_outputs():
    import numpy as np
    rng = np.random.default_rng(0)
    n = 5000
    keys = rng.integers(0, 2**32, n, dtype=np.uint32)
    vals = np.arange(n, dtype=np.uint32)
    perm = np.argsort(keys, kind="stable").astype(np.uint32)
    assert bench.check_output("pairs_u32", keys, vals, keys[perm], perm, 0, 0, 32)
    broken = perm.copy()
    broken[[10, 11]] = broken[[11, 10]]
    assert not bench.check_output("pairs_u32", keys, vals, keys[broken], broken, 0, 0, 32)
    x = rng.standard_normal(n).astype(np.float32)
    keep = x > 0
    part = np.concatenate([x[keep], x[~keep]])
    pv = np.concatenate([vals[keep], vals[~keep]])
    assert bench.check_output("partition", x.view(np.uint32), vals, part, pv, int(keep.sum()), 0, 0)
    assert not bench.check_output("partition", x.view(np.uint32), vals, part, pv[::-1].copy(),
                                  int(keep.sum()), 0, 0)
    comp = np.concatenate([x[keep], np.zeros((~keep).sum(), np.float32)])
    assert bench.check_output("compact", x.view(np.uint32), None, comp, None, int(keep.sum()), 0, 0)
    sc = (np.cumsum(keys.astype(np.uint64)) & np.uint64(0xFFFFFFFF)).astype(np.uint32)
    exc = np.concatenate([[0], sc[:-1]]).astype(np.uint32)
    assert bench.check_output("scan", keys, None, exc, None, 0, 0, 0)
    assert not bench.check_output("scan", keys, None, sc, None, 0, 0, 0)
    k64 = rng.integers(0, 2**45, n, dtype=np.uint64)
    v64 = rng.integers(0, 100, n, dtype=np.uint32)     # values are not positions
    p64 = np.argsort(k64, kind="stable")
    assert bench.check_output("pairs_u64", k64, v64, k64[p64], v64[p64], 0, 0, 45)
    f = rng.standard_normal(n).astype(np.float32)
    fo = np.argsort(bench.f32_order(f.view(np.uint32)), kind="stable").astype(np.uint32)
    assert bench.check_output("pairs_f32", f.view(np.uint32), vals, f[fo], fo, 0, 0, 32)


def test_bench_functions_read_only_defined_names():
    """Every name a function of bench.py reads without assigning it is a
    module-level name or a builtin (the GPU-only code paths of the bench run
    on the GPU only, so a stray name there would otherwise surface there)."""
    import builtins
    import symtable

    import bench
    with open(bench.__file__) as f:
        top = symtable.symtable(f.read(), bench.__file__, "exec")
    missing = []

    def walk(table):
        for child in table.get_children():
            if child.get_type() == "function":
                for sym in child.get_symbols():
                    name = sym.get_name()
                    if (sym.is_referenced() and sym.is_global() and not hasattr(bench, name)
                            and not hasattr(builtins, name)):
                        missing.append((child.get_name(), name))
            walk(child)

    walk(top)
    assert not missing, missing


def test_source_hash_ignores_comments_only(tmp_path):
    import bench
    src = tmp_path / "k.hip"
    src.write_text("int f(int x) {\n    return x + 1;   // one more\n}\n")
    h0 = bench.source_hash(str(tmp_path))
    src.write_text("/* a block\n   comment */\nint f(int x) {\n  return x + 1;  // changed note\n}\n")
    assert bench.source_hash(str(tmp_path)) == h0
    src.write_text("int f(int x) {\n    return x + 2;\n}\n")
    assert bench.source_hash(str(tmp_path)) != h0
