"""Throughput of the stable LSD radix sort on one MI355X.

Default workload: 2^28 uniform u32 keys with u32 values (original indices),
full 32-bit keys, 4 passes of 8-bit digits.  One step = one whole
rs_sort_pairs_u32 call (fill, upsweep histogram, 4 one-sweep passes) with
inputs, outputs and temp already resident in HBM.  Prints one JSON line.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                  [--no-cpu-baseline] [--copy-calibration]

The roofline entry is for the dominant kernel (the one-sweep pass): its
algorithmic bytes per launch (read + write of keys and values, 16 B per key)
over its mean duration, timed with HIP events the library records around
each launch on the call's stream during the timed steps.  The CPU baseline is
the oracle (single-threaded C) on a bounded prefix of the same workload.
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
PROFILES = os.path.join(ROOT, "profiles")
TRAFFIC_FILE = os.path.join(PROFILES, "onesweep_pairs_u32_2p28_traffic.json")
KERNEL_SOURCE = os.path.join(ROOT, "sorting_lsd_radix_amd", "csrc", "radix.hip")

WORKLOADS = {
    # name: (description, n, pairs, is_f32, begin_bit, end_bit)
    "pairs_u32_2p28": ("uniform u32 key-value pairs, n=2^28, bits [0,32), 4 passes",
                       1 << 28, True, False, 0, 32),
    "keys_u32_2p28": ("uniform u32 keys only, n=2^28, bits [0,32), 4 passes",
                      1 << 28, False, False, 0, 32),
    "pairs_f32_2p28": ("N(0,1) f32 keys with injected +-0 and +-1e-38, index values, n=2^28, "
                       "4 passes", 1 << 28, True, True, 0, 32),
    "pairs_zipf_2p26": ("Zipf(1.2) u32 keys over 65536 values, index values, n=2^26, bits [0,16), "
                        "2 passes", 1 << 26, True, False, 0, 16),
    "pairs_u32_2p20": ("uniform u32 key-value pairs, n=2^20, bits [0,32), 4 passes",
                       1 << 20, True, False, 0, 32),
}


def kernel_source_hash():
    h = hashlib.sha256()
    with open(KERNEL_SOURCE, "rb") as f:
        h.update(f.read())
    return h.hexdigest()[:16]


def make_inputs(name):
    import workloads
    desc, n, pairs, is_f32, b, e = WORKLOADS[name]
    if name == "pairs_f32_2p28":
        keys, vals = workloads.float_pairs(n)
    elif name == "pairs_zipf_2p26":
        keys, vals = workloads.pairs_zipf(n)
    else:
        keys, vals = workloads.headline_pairs(n)
    return keys, (vals if pairs else None)


def cpu_baseline(keys, vals, b, e, is_f32, budget_s=12.0, sample=1 << 24):
    """The oracle on the first `sample` elements, repeated up to ~budget_s."""
    import oracle
    k = keys[:sample].copy()
    v = vals[:sample].copy() if vals is not None else None
    runs, total = 0, 0.0
    while True:
        t0 = time.perf_counter()
        if is_f32:
            oracle.sort_f32(k, v, b, e)
        else:
            oracle.sort_u32(k, v, b, e)
        total += time.perf_counter() - t0
        runs += 1
        if total >= budget_s or runs >= 5:
            break
    per_run = total / runs
    return {"value": round(k.size / per_run / 1e9, 6), "unit": "Gkeys/s", "cores": 1,
            "kind": "oracle",
            "sample": "first %d elements of the same workload, %d run(s), %.2f s each; "
                      "single-threaded C LSD counting sort (gcc -O2)" % (k.size, runs, per_run)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="pairs_u32_2p28", choices=sorted(WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-check", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (reference for HBM counters)")
    args = ap.parse_args()

    if args.gpus != 1:
        print("bench.py measures one GPU only: this library has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import sorting_lsd_radix_amd as rs

    desc, n, pairs, is_f32, b, e = WORKLOADS[args.workload]
    print("bench: generating %s" % args.workload, file=sys.stderr, flush=True)
    keys, vals = make_inputs(args.workload)
    dev = torch.device("cuda:0")
    kin = torch.from_numpy(keys.view(np.float32) if is_f32 else keys).to(dev)
    vin = torch.from_numpy(vals).to(dev) if pairs else None
    kout = torch.empty_like(kin)
    vout = torch.empty_like(vin) if pairs else None
    if is_f32:
        need = rs.rs_sort_pairs_f32(None, None, None, None, n, b, e, None, 0)
    elif pairs:
        need = rs.rs_sort_pairs_u32(None, None, None, None, n, b, e, None, 0)
    else:
        need = rs.rs_sort_keys_u32(None, None, n, b, e, None, 0)
    temp = torch.empty(need, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def step():
        if is_f32:
            rs.rs_sort_pairs_f32(kin, kout, vin, vout, n, b, e, temp, need, stream)
        elif pairs:
            rs.rs_sort_pairs_u32(kin, kout, vin, vout, n, b, e, temp, need, stream)
        else:
            rs.rs_sort_keys_u32(kin, kout, n, b, e, temp, need, stream)

    if args.copy_calibration:
        a = torch.empty(1 << 28, dtype=torch.int32, device=dev).fill_(1)
        c = torch.empty_like(a)
        for _ in range(3):
            c.copy_(a)
        torch.cuda.synchronize()
        del a, c

    print("bench: warmup %d" % args.warmup, file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    rs.rs_timing_enable(True)
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for _ in range(args.steps):
        step()
    stop.record(stream)
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(stop)
    records = rs.rs_timing_collect()
    rs.rs_timing_enable(False)
    ms_per_step = total_ms / args.steps
    print("bench: timed %d steps, %.3f ms/step" % (args.steps, ms_per_step), file=sys.stderr,
          flush=True)

    per_kernel = {}
    for name, ms in records:
        per_kernel.setdefault(name, []).append(ms)
    sweep = per_kernel.get("onesweep", [])
    sweep_ms = sum(sweep) / len(sweep) if sweep else float("nan")
    bytes_per_key = 16 if pairs else 8
    algo_bytes = bytes_per_key * n
    achieved = algo_bytes / (sweep_ms * 1e-3) / 1e9
    traffic = None
    if os.path.exists(TRAFFIC_FILE):
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
        if t.get("kernel_source_sha") == kernel_source_hash() and t.get("workload") == args.workload:
            traffic = t.get("traffic_bytes_per_launch")

    if not args.no_check:
        k_h = kout.cpu().numpy()
        if is_f32:
            import oracle
            order = oracle.f32_to_order(k_h.view(np.uint32))
        else:
            order = k_h & np.uint32(((1 << (e - b)) - 1) << b) if e - b < 32 else k_h
        ok = bool(np.all(order[1:] >= order[:-1]))
        if pairs:
            v_h = vout.cpu().numpy()
            ok = ok and bool(np.array_equal(k_h.view(np.uint32), keys.view(np.uint32)[v_h]))
        if not ok:
            print("bench: OUTPUT CHECK FAILED", file=sys.stderr, flush=True)
            sys.exit(1)
        print("bench: output check ok", file=sys.stderr, flush=True)

    result = {
        "metric": "Gkeys/s sorted (u32 key-value, n=2^28) and % of HBM roofline",
        "value": round(n / (ms_per_step * 1e-3) / 1e9, 4),
        "unit": "Gkeys/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "u32" if not is_f32 else "f32 keys (bit-pattern integer ops), u32 values",
        "data": "synthetic",
        "config": {"workload": desc, "n": n, "begin_bit": b, "end_bit": e,
                   "passes": (e - b + 7) // 8, "pairs": pairs},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic,
                     "kernel": "onesweep pass", "algorithmic_bytes_per_launch": algo_bytes,
                     "mean_launch_ms": round(sweep_ms, 5)},
        "whole_sort_roofline_frac": round(algo_bytes * ((e - b + 7) // 8) /
                                          (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "kernel_ms": {k: round(sum(v) / len(v), 5) for k, v in per_kernel.items()},
    }
    if not args.no_cpu_baseline:
        print("bench: cpu baseline", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(keys, vals, b, e, is_f32)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
