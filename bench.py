"""Throughput of the stable LSD radix sort (and its companions) on one MI355X.

Default workload: 2^28 uniform u32 keys with u32 values (original indices),
full 32-bit keys, 4 passes of 8-bit digits.  One step = one whole
rs_sort_pairs_u32 call (fill, upsweep histogram, 4 one-sweep passes) with
inputs, outputs and temp already resident in HBM.  Prints one JSON line.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME | --all]
                  [--no-cpu-baseline] [--no-check] [--copy-calibration]
  python bench.py --workload NAME --record-traffic FETCH_DIR WRITE_DIR

The roofline entry is for the dominant kernel of the workload (the one-sweep
pass for sorts, the one-workgroup tile sort for sorts of at most 16384 keys,
the bucket sort for hybrid sorts of at most 3 * 2^20 keys, the compaction
kernel for compaction): its algorithmic bytes per launch over
its mean duration, timed with HIP events that the library
records around each of its launches on the call's stream during the last
twentieth (at least one) of the timed steps, inside the same timed region
(recording them in every step would add about 2 us per launch to the time per
step).  Algorithmic bytes: 16 B per key per pass for key-value sorts (read and
write key and value), 8 B for keys-only sorts, 8 B per element for compaction
(read the input, write the output including the zero tail).  The default line also
carries "keys_u32_2p28": the keys-only sort of the same 2^28 keys, timed the
same way.  The CPU baseline is the oracle (single-threaded C) on the same
workload, repeated for about 10 s.  --all prints one line per workload (the
default line first).
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
TILE_SORT_MAX = 16384  # sorts up to this size run in one workgroup (one launch)
HYBRID_MAX = 3 << 20   # up to this size a sort is one top-digit pass + one LDS sort per bucket
PROFILES = os.path.join(ROOT, "profiles")
TRAFFIC_FILE = os.path.join(PROFILES, "traffic.json")
CSRC = os.path.join(ROOT, "sorting_lsd_radix_amd", "csrc")

# name: (description, kind, n, begin_bit, end_bit)
WORKLOADS = {
    "pairs_u32_2p28": ("uniform u32 key-value pairs, n=2^28, bits [0,32), 4 passes",
                       "pairs_u32", 1 << 28, 0, 32),
    "keys_u32_2p28": ("uniform u32 keys only, n=2^28, bits [0,32), 4 passes",
                      "keys_u32", 1 << 28, 0, 32),
    "pairs_f32_2p28": ("N(0,1) f32 keys with injected +-0 and +-1e-38, index values, n=2^28, "
                       "4 passes", "pairs_f32", 1 << 28, 0, 32),
    "pairs_zipf_2p26": ("Zipf(1.2) u32 keys over 65536 values, index values, n=2^26, "
                        "bits [0,16), 2 passes", "pairs_u32", 1 << 26, 0, 16),
    "pairs_u32_2p20": ("uniform u32 key-value pairs, n=2^20, bits [0,32), 4 passes",
                       "pairs_u32", 1 << 20, 0, 32),
    "compact_f32_2p28": ("compaction of 2^28 f32 (45% positive, 45% negative, 10% +0.0), "
                         "keep x > 0, zero tail, count", "compact", 1 << 28, 0, 0),
    "tile_bitonic_1024": ("1024 uniform u32 keys, one LDS bitonic tile", "bitonic", 1024, 0, 32),
    "tile_radix_1024": ("1024 uniform u32 keys, keys-only radix sort (4 passes)",
                        "keys_u32", 1024, 0, 32),
    "pairs_u64_2p27": ("uniform u64 keys with index values, n=2^27, bits [0,64), 8 passes",
                       "pairs_u64", 1 << 27, 0, 64),
    "splat_pairs_2p22": ("splat tile/depth u64 keys of 2^22 splats (1920x1080, 16x16 tiles; "
                         "24.2M tile entries), splat-index values, bits [0,45), 6 passes",
                         "pairs_u64", 1 << 22, 0, 45),
    "scan_u32_2p28": ("exclusive prefix sum of 2^28 uniform u32 (mod 2^32)", "scan", 1 << 28, 0, 0),
    "partition_f32_2p28": ("stable partition x > 0 of the 2^28 compaction input with index values",
                           "partition", 1 << 28, 0, 0),
}
DEFAULT = "pairs_u32_2p28"


def code_of(text):
    """Source text without its comments and with runs of whitespace as one
    space, so that a change to comments alone keeps the hash."""
    import re
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def source_hash(csrc=CSRC):
    """Hash of the kernel sources' code: the key that ties a recorded traffic
    figure to the kernels it was measured on."""
    h = hashlib.sha256()
    for f in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, f), encoding="utf-8") as fh:
            h.update(f.encode())
            h.update(code_of(fh.read()).encode())
    return h.hexdigest()[:16]


def make_inputs(name):
    import workloads
    _, kind, n, _, _ = WORKLOADS[name]
    if name == "pairs_f32_2p28":
        return workloads.float_pairs(n)
    if name == "pairs_zipf_2p26":
        return workloads.pairs_zipf(n)
    if kind == "compact":
        return workloads.compact_input(n), None
    if kind == "partition":
        return workloads.compact_input(n), workloads.index_values(n)
    if kind == "scan":
        return workloads.uniform_u32(n), None
    if name == "splat_pairs_2p22":
        return workloads.splat_pairs(n)
    if kind == "pairs_u64":
        rng = workloads.rng_for()
        return rng.integers(0, 2**64, n, dtype="uint64"), workloads.index_values(n)
    if n == 1024:
        return workloads.tile_keys(), None
    keys, vals = workloads.headline_pairs(n)
    return keys, (vals if kind != "keys_u32" else None)


def host_cpu():
    """(usable cores, model name) of the host this runs on."""
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count()
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return cores, model


def cpu_baseline(name, keys, vals, budget_s=10.0, sample=None):
    """The oracle on the workload (or its first `sample` elements), repeated
    until about budget_s of CPU time has been spent."""
    import oracle
    _, kind, n, b, e = WORKLOADS[name]
    if sample is None or sample >= keys.size:
        k, v, what = keys, vals, "the whole workload (%d elements)" % keys.size
    else:
        k = keys[:sample].copy()
        v = vals[:sample].copy() if vals is not None else None
        what = "the first %d elements of the workload" % sample
    runs, total = 0, 0.0
    while True:
        t0 = time.perf_counter()
        if kind == "compact":
            oracle.compact_positive_f32(k)
        elif kind == "scan":
            oracle.scan_u32(k)
        elif kind == "partition":
            oracle.select(k, ">", 0.0, v, partition=True)
        elif kind == "pairs_u64":
            oracle.sort_u64(k, v, b, e)
        elif kind == "bitonic":
            oracle.bitonic_tile(k, 1024, b, e)
        elif kind == "pairs_f32":
            oracle.sort_f32(k, v, b, e)
        else:
            oracle.sort_u32(k, v, b, e)
        total += time.perf_counter() - t0
        runs += 1
        if total >= budget_s or runs >= (1000 if k.size <= 4096 else 50):
            break
    per_run = total / runs
    unit = "G elements/s" if kind in ("compact", "scan", "partition") else "Gkeys/s"
    host_cores, model = host_cpu()
    return {"value": round(k.size / per_run / 1e9, 6), "unit": unit, "cores": 1, "kind": "oracle",
            "sample": "%s, %d run(s), %.4f s each; single-threaded C oracle (gcc -O2)"
                      % (what, runs, per_run),
            "host_cores": host_cores, "host_cpu": model}


def f32_order(bits):
    """Unsigned order patterns of float32 bit patterns (IEEE totalOrder)."""
    import numpy as np
    neg = (bits >> np.uint32(31)) != 0
    return np.where(neg, ~bits, bits | np.uint32(0x80000000))


def check_output(kind, keys, vals, k_h, v_h, count, b, e):
    """Properties that define each output uniquely, with numpy only."""
    import numpy as np
    if kind in ("compact", "partition"):
        x = keys.view(np.float32)
        keep = x > np.float32(0)
        k = int(keep.sum())
        got = k_h.view(np.uint32)
        if count != k or not np.array_equal(got[:k], keys.view(np.uint32)[keep]):
            return False
        if kind == "compact":
            return bool(np.all(got[k:] == 0))
        return (np.array_equal(got[k:], keys.view(np.uint32)[~keep]) and
                np.array_equal(v_h, np.concatenate([vals[keep], vals[~keep]])))
    if kind == "scan":
        ref = (np.cumsum(keys.astype(np.uint64)) & np.uint64(0xFFFFFFFF)).astype(np.uint32)
        return k_h[0] == 0 and np.array_equal(k_h[1:], ref[:-1])
    if kind == "bitonic":
        for s0 in range(0, keys.size, 1024):
            if not np.array_equal(k_h[s0:s0 + 1024], np.sort(keys[s0:s0 + 1024], kind="stable")):
                return False
        return True
    # sorts: non-decreasing field, key/value association, stability
    raw = k_h.view(np.uint64 if kind == "pairs_u64" else np.uint32)
    if kind == "pairs_f32":
        order = f32_order(raw)
    elif kind == "pairs_u64":
        order = (raw >> np.uint64(b)) & np.uint64((1 << (e - b)) - 1)
    elif e - b < 32:
        order = raw & np.uint32(((1 << (e - b)) - 1) << b)
    else:
        order = raw
    ok = bool(np.all(order[1:] >= order[:-1]))
    if v_h is None:
        return ok
    src = keys.view(raw.dtype)
    if np.array_equal(vals, np.arange(vals.size, dtype=np.uint32)):
        # values are positions: association and stability
        ok = ok and bool(np.array_equal(raw, src[v_h]))
        eq = order[1:] == order[:-1]
        return ok and bool(np.all(v_h[1:][eq] > v_h[:-1][eq]))
    # other values: the stable order by numpy's stable argsort of the field
    field = (src >> np.uint64(b)) & np.uint64((1 << (e - b)) - 1) if kind == "pairs_u64" else None
    perm = np.argsort(field, kind="stable")
    return ok and bool(np.array_equal(raw, src[perm])) and bool(np.array_equal(v_h, vals[perm]))


def timed_region(step, steps, warmup, stream):
    """Time `steps` calls of step() between two events on `stream`.

    The library's per-launch events are recorded only during the last
    `event_steps` calls: each event still adds about 2 us between launches,
    which would otherwise inflate the time per step of small sorts by up to a
    third.  Returns (ms per step, {kernel: [ms per launch]}, event_steps)."""
    import torch

    import sorting_lsd_radix_amd as rs
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    event_steps = max(1, steps // 20)
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for i in range(steps):
        if i == steps - event_steps:
            rs.rs_timing_enable(True)
        step()
    stop.record(stream)
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(stop)
    records = rs.rs_timing_collect()
    rs.rs_timing_enable(False)
    per_kernel = {}
    for kname, ms in records:
        per_kernel.setdefault(kname, []).append(ms)
    return total_ms / steps, per_kernel, event_steps


def keys_only_companion(kin, n, steps, warmup, stream, pairs_keys_out, check):
    """The keys-only half of the metric on the same device keys: one whole
    rs_sort_keys_u32 call per step (fill, upsweep, 4 passes)."""
    import numpy as np
    import torch

    import sorting_lsd_radix_amd as rs
    kout = torch.empty_like(kin)
    need = rs.rs_sort_keys_u32(None, None, n, 0, 32, None, 0)
    temp = torch.empty(max(need, 1), dtype=torch.uint8, device=kin.device)

    def step():
        rs.rs_sort_keys_u32(kin, kout, n, 0, 32, temp, need, stream)

    ms, per_kernel, _ = timed_region(step, steps, warmup, stream)
    print("bench: keys_u32_2p28 timed %d steps, %.4f ms/step" % (steps, ms), file=sys.stderr,
          flush=True)
    if check:
        # the keys of the checked pair sort are the sorted keys: the keys-only
        # output must equal them
        if not torch.equal(kout, pairs_keys_out):
            print("bench: OUTPUT CHECK FAILED for keys_u32_2p28", file=sys.stderr, flush=True)
            sys.exit(1)
    pass_ms = per_kernel.get("onesweep", [float("nan")])
    pass_ms = sum(pass_ms) / len(pass_ms)
    return {"workload": WORKLOADS["keys_u32_2p28"][0], "value": round(n / (ms * 1e-3) / 1e9, 4),
            "unit": "Gkeys/s", "ms_per_step": round(ms, 5),
            "pass_ms": round(pass_ms, 5),
            "pass_roofline_frac": round(8 * n / (pass_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "whole_step_roofline_frac": round(8 * n * 4 / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "kernel_ms": {k: round(sum(v) / len(v), 5) for k, v in per_kernel.items()}}


def roofline_terms(kind, n, b, e):
    """(dominant kernel, algorithmic bytes per element of one launch of it,
    algorithmic bytes of the whole step) for a workload."""
    passes = (e - b + 7) // 8
    if kind in ("compact", "bitonic", "scan"):
        # read every element once, write every output element once
        return {"compact": "compact", "bitonic": "bitonic", "scan": "scan"}[kind], 8, 8 * n
    if kind == "partition":
        # read and write every element and its value once (the counting read is an overhead)
        return "select", 16, 16 * n
    if kind == "pairs_u64":
        # 8-byte key + 4-byte value, read and written by every pass
        return "onesweep", 24, 24 * n * passes
    bytes_per = 8 if kind == "keys_u32" else 16
    if n <= TILE_SORT_MAX:
        # the whole sort in one workgroup: the keys (and values) cross HBM once each way
        return "tile_sort", bytes_per, bytes_per * n
    if n <= HYBRID_MAX and passes >= 2:
        # hybrid: the bucket sort (one read and one write of every key and value)
        # after the top digit's pass; the metric still counts every pass's bytes
        return "bucket_sort", bytes_per, bytes_per * n * passes
    return "onesweep", bytes_per, bytes_per * n * passes


def run_workload(name, steps, warmup, check, with_cpu, copy_calibration=False):
    import numpy as np
    import torch

    import sorting_lsd_radix_amd as rs

    desc, kind, n, b, e = WORKLOADS[name]
    print("bench: generating %s" % name, file=sys.stderr, flush=True)
    keys, vals = make_inputs(name)
    n = keys.size   # the splat workload's n counts splats; its arrays hold their tile entries
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    is_f32 = kind in ("pairs_f32", "compact", "partition")
    kin = torch.from_numpy(keys.view(np.float32) if is_f32 else keys).to(dev)
    vin = torch.from_numpy(vals).to(dev) if vals is not None else None
    kout = torch.empty_like(kin)
    vout = torch.empty_like(vin) if vin is not None else None
    count = torch.empty(1, dtype=torch.uint32, device=dev)
    gt0 = 0   # bit pattern of the threshold 0.0f
    if kind == "pairs_u32":
        need = rs.rs_sort_pairs_u32(None, None, None, None, n, b, e, None, 0)
    elif kind == "pairs_f32":
        need = rs.rs_sort_pairs_f32(None, None, None, None, n, b, e, None, 0)
    elif kind == "keys_u32":
        need = rs.rs_sort_keys_u32(None, None, n, b, e, None, 0)
    elif kind == "pairs_u64":
        need = rs.rs_sort_pairs(rs.RS_KEY_U64, 0, None, None, None, None, n, b, e, None, 0)
    elif kind == "compact":
        need = rs.rs_compact_positive_f32(None, None, None, n, None, 0)
    elif kind == "scan":
        need = rs.rs_exclusive_scan_u32(None, None, n, None, 0)
    elif kind == "partition":
        need = rs.rs_partition(rs.RS_KEY_F32, rs.RS_OP_GT, gt0, None, None, vin, vout, None, n,
                               None, 0)
    else:
        need = 0
    temp = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)

    def step():
        if kind == "pairs_u32":
            rs.rs_sort_pairs_u32(kin, kout, vin, vout, n, b, e, temp, need, stream)
        elif kind == "pairs_f32":
            rs.rs_sort_pairs_f32(kin, kout, vin, vout, n, b, e, temp, need, stream)
        elif kind == "keys_u32":
            rs.rs_sort_keys_u32(kin, kout, n, b, e, temp, need, stream)
        elif kind == "pairs_u64":
            rs.rs_sort_pairs(rs.RS_KEY_U64, 0, kin, kout, vin, vout, n, b, e, temp, need, stream)
        elif kind == "compact":
            rs.rs_compact_positive_f32(kin, kout, count, n, temp, need, stream)
        elif kind == "scan":
            rs.rs_exclusive_scan_u32(kin, kout, n, temp, need, stream)
        elif kind == "partition":
            rs.rs_partition(rs.RS_KEY_F32, rs.RS_OP_GT, gt0, kin, kout, vin, vout, count, n, temp,
                            need, stream)
        else:
            rs.rs_bitonic_tile(kin, kout, n, 1024, b, e, stream)

    if copy_calibration:
        a = torch.empty(1 << 28, dtype=torch.int32, device=dev).fill_(1)
        c = torch.empty_like(a)
        for _ in range(3):
            c.copy_(a)
        torch.cuda.synchronize()
        del a, c

    ms_per_step, per_kernel, event_steps = timed_region(step, steps, warmup, stream)
    print("bench: %s timed %d steps, %.4f ms/step" % (name, steps, ms_per_step), file=sys.stderr,
          flush=True)

    if check:
        ok = check_output(kind, keys, vals, kout.cpu().numpy(),
                          vout.cpu().numpy() if vout is not None else None,
                          int(count.cpu().numpy()[0]), b, e)
        if not ok:
            print("bench: OUTPUT CHECK FAILED for %s" % name, file=sys.stderr, flush=True)
            sys.exit(1)
        print("bench: output check ok", file=sys.stderr, flush=True)

    dom, bytes_per, algo_total = roofline_terms(kind, n, b, e)
    dom_ms = per_kernel.get(dom, [float("nan")])
    dom_ms = sum(dom_ms) / len(dom_ms)
    algo_bytes = bytes_per * n
    achieved = algo_bytes / (dom_ms * 1e-3) / 1e9
    traffic = None
    if os.path.exists(TRAFFIC_FILE):
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
        entry = t.get(name)
        if entry and entry.get("source_sha") == source_hash():
            traffic = entry.get("traffic_bytes_per_launch")

    if kind == "compact":
        metric, unit, value = ("G elements/s compacted (f32, n=2^28) and % of HBM roofline",
                               "G elements/s", n / (ms_per_step * 1e-3) / 1e9)
    elif kind == "scan":
        metric, unit, value = ("G elements/s prefix-summed (u32, n=2^28) and % of HBM roofline",
                               "G elements/s", n / (ms_per_step * 1e-3) / 1e9)
    elif kind == "partition":
        metric, unit, value = ("G elements/s partitioned (f32 with u32 values, n=2^28) and % of "
                               "HBM roofline", "G elements/s", n / (ms_per_step * 1e-3) / 1e9)
    elif kind == "pairs_u64":
        metric, unit, value = ("Gkeys/s sorted (u64 keys with u32 values) and % of HBM roofline",
                               "Gkeys/s", n / (ms_per_step * 1e-3) / 1e9)
    elif kind == "bitonic" or n <= 4096:
        metric, unit, value = ("microseconds per call (1024-key tile)", "us", ms_per_step * 1e3)
    else:
        metric, unit, value = ("Gkeys/s sorted (u32 keys and u32 key-value, n=2^28) and % of HBM "
                               "roofline", "Gkeys/s", n / (ms_per_step * 1e-3) / 1e9)
    result = {
        "metric": metric,
        "value": round(value, 4),
        "unit": unit,
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": unit != "us",
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"pairs_u32": "u32", "keys_u32": "u32", "bitonic": "u32",
                  "pairs_f32": "f32 keys (bit-pattern integer ops), u32 values",
                  "compact": "f32 (predicate on bit patterns)", "scan": "u32",
                  "partition": "f32 (IEEE comparison), u32 values",
                  "pairs_u64": "u64 keys, u32 values"}[kind],
        "data": "synthetic",
        "config": {"workload": desc, "n": n, "begin_bit": b, "end_bit": e,
                   "passes": (e - b + 7) // 8 if kind not in ("compact", "bitonic", "scan", "partition")
                   else None},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "kernel": dom, "algorithmic_bytes_per_launch": algo_bytes,
                     "mean_launch_ms": round(dom_ms, 5), "timed_launches": len(per_kernel.get(dom, [])),
                     "event_steps": event_steps},
        "whole_step_roofline_frac": round(algo_total / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "kernel_ms": {k: round(sum(v) / len(v), 5) for k, v in per_kernel.items()},
    }
    if name == DEFAULT and not copy_calibration:
        # the metric names keys-only sorts as well: same keys, same step count
        # (not in the counter runs, whose per-kernel means would mix the two sorts' passes)
        result["keys_u32_2p28"] = keys_only_companion(kin, n, steps, warmup, stream, kout, check)
    result["cpu_baseline"] = cpu_baseline(name, keys, vals) if with_cpu else None
    return result


KERNEL_MATCH = {"onesweep": "onesweep_kernel", "upsweep": "upsweep_kernel",
                "compact": "compact_kernel", "tile_sort": "tile_sort_kernel",
                "bucket_sort": "bucket_sort_kernel", "scan": "scan_kernel", "select": "select_kernel",
                "bitonic": "bitonic_tile_kernel", "copy": "__amd_rocclr_copyBuffer"}
COPY_BYTES = 4 << 28   # the --copy-calibration copy moves 1 GiB each way


def record_traffic(name, fetch_dir, write_dir):
    """Per-launch HBM bytes of the workload's dominant kernel from two
    rocprofv3 --pmc runs (FETCH_SIZE, then WRITE_SIZE, both with
    --copy-calibration), each counter scaled by what it reads for the 1 GiB
    device copy of the same run; written to profiles/traffic.json."""
    import csv

    def per_kernel(d):
        out = {}
        with open(os.path.join(d, "run_counter_collection.csv")) as f:
            for r in csv.DictReader(f):
                for k, pat in KERNEL_MATCH.items():
                    if pat in r["Kernel_Name"]:
                        out.setdefault(k, []).append(float(r["Counter_Value"]))
        return {k: sum(v) / len(v) for k, v in out.items()}

    fetch, write = per_kernel(fetch_dir), per_kernel(write_dir)
    desc, kind, n, b, e = WORKLOADS[name]
    dom, bytes_per, _ = roofline_terms(kind, n, b, e)
    f_factor = COPY_BYTES / (fetch["copy"] * 1024)
    w_factor = COPY_BYTES / (write["copy"] * 1024)
    entry = {
        "source_sha": source_hash(),
        "kernel": dom,
        "traffic_bytes_per_launch": round(fetch[dom] * 1024 * f_factor + write[dom] * 1024 * w_factor),
        "fetch_bytes_per_launch": round(fetch[dom] * 1024 * f_factor),
        "write_bytes_per_launch": round(write[dom] * 1024 * w_factor),
        "algorithmic_bytes_per_launch": bytes_per * n,
        "calibration": {"copy_bytes_each_way": COPY_BYTES, "fetch_size_kib": round(fetch["copy"], 1),
                        "write_size_kib": round(write["copy"], 1), "fetch_factor": round(f_factor, 4),
                        "write_factor": round(w_factor, 4)},
        "commands": ["rocprofv3 --pmc %s --output-format csv -d %s -o run -- python3 bench.py --workload %s "
                     "--steps 2 --warmup 1 --no-cpu-baseline --no-check --copy-calibration" % (c, d, name)
                     for c, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir))],
    }
    if "upsweep" in fetch:
        entry["upsweep_fetch_bytes_per_launch"] = round(fetch["upsweep"] * 1024 * f_factor)
        entry["upsweep_write_bytes_per_launch"] = round(write["upsweep"] * 1024 * w_factor)
    table = {}
    if os.path.exists(TRAFFIC_FILE):
        with open(TRAFFIC_FILE) as f:
            table = json.load(f)
    table[name] = entry
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(table, f, indent=2)
        f.write("\n")
    print(json.dumps({name: entry}))


def copy_ceiling(steps=20):
    """Two 1 GiB device streams timed with HIP events: torch's device-to-device
    copy (the runtime's copy kernel) and torch's elementwise bitwise NOT of
    int32 (one read and one write of every byte, vectorised).  The faster is
    the bandwidth a kernel that reads and writes every byte once reaches on
    this GPU, as context for the passes' roofline fractions."""
    import torch
    dev = torch.device("cuda:0")
    a = torch.empty(1 << 28, dtype=torch.int32, device=dev).fill_(1)
    b = torch.empty_like(a)
    moved = 2 * a.numel() * 4
    out = {"metric": "1 GiB read + 1 GiB written", "steps": steps}
    for name, op in (("copy", lambda: b.copy_(a)),
                     ("bitwise_not", lambda: torch.bitwise_not(a, out=b))):
        for _ in range(3):
            op()
        torch.cuda.synchronize()
        start = torch.cuda.Event(enable_timing=True)
        stop = torch.cuda.Event(enable_timing=True)
        start.record()
        for _ in range(steps):
            op()
        stop.record()
        torch.cuda.synchronize()
        ms = start.elapsed_time(stop) / steps
        out[name] = {"ms": round(ms, 5), "GB/s": round(moved / (ms * 1e-3) / 1e9, 1),
                     "frac_of_8TBps": round(moved / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default=DEFAULT, choices=sorted(WORKLOADS))
    ap.add_argument("--all", action="store_true", help="one line per workload")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-check", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (reference for HBM counters)")
    ap.add_argument("--copy-ceiling", action="store_true",
                    help="time two 1 GiB device streams and print their bandwidth (context only)")
    ap.add_argument("--record-traffic", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write profiles/traffic.json for --workload from two rocprofv3 --pmc "
                         "output folders (FETCH_SIZE, WRITE_SIZE) and exit; no GPU needed")
    args = ap.parse_args()

    if args.record_traffic:
        record_traffic(args.workload, *args.record_traffic)
        return
    if args.copy_ceiling:
        print(json.dumps(copy_ceiling()), flush=True)
        return
    if args.gpus != 1:
        print("bench.py measures one GPU only: this library has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    names = [args.workload]
    if args.all:
        names = [DEFAULT] + [w for w in WORKLOADS if w != DEFAULT]
    for name in names:
        small = WORKLOADS[name][2] <= (1 << 20)
        steps = max(args.steps, 100) if small else args.steps
        res = run_workload(name, steps, args.warmup, not args.no_check, not args.no_cpu_baseline,
                           args.copy_calibration and name == names[0])
        print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
