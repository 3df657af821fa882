"""The library's measurement hook on the GPU: one record per launch, in launch
order, with plausible durations; recording stops when the hook is disabled
and restarts empty when it is enabled again.  bench.py derives the roofline
from these records, so their count and order are checked here."""
import math

import numpy as np
import pytest

import sorting_lsd_radix_amd as rs
from gpu_helpers import gpu_compact, gpu_sort_keys_u32, gpu_sort_pairs_u32

pytestmark = pytest.mark.gpu


def test_timing_records_one_per_launch_in_order():
    print("timing hook: 2^20 pair sort, 2^20 compaction", flush=True)
    n = 1 << 20
    keys = np.random.default_rng(11).integers(0, 2**32, n, dtype=np.uint32)
    vals = np.arange(n, dtype=np.uint32)
    rs.rs_timing_enable(True)
    try:
        gpu_sort_pairs_u32(keys, vals, 0, 32)
        floats = np.random.default_rng(12).standard_normal(n).astype(np.float32)
        gpu_compact(floats)
        recs = rs.rs_timing_collect()
    finally:
        rs.rs_timing_enable(False)
    names = [name for name, _ in recs]
    # the hybrid path: the top digit's pass, the bucket sort, then the gated
    # multi-pass launch of the LSD passes (which returns at once for uniform keys)
    assert names == ["sort_init", "upsweep", "onesweep", "bucket_sort", "onesweep",
                     "compact_init", "compact"], names
    for name, ms in recs:
        assert math.isfinite(ms) and 0.0 < ms < 100.0, (name, ms)


def test_timing_disable_stops_and_enable_clears():
    print("timing hook: enable/disable", flush=True)
    keys = np.random.default_rng(13).integers(0, 2**32, 1 << 18, dtype=np.uint32)
    rs.rs_timing_enable(True)
    try:
        gpu_sort_keys_u32(keys, 0, 16)   # two passes
        first = rs.rs_timing_collect()
    finally:
        rs.rs_timing_enable(False)
    assert [name for name, _ in first] == ["sort_init", "upsweep", "onesweep", "bucket_sort",
                                           "onesweep"]
    gpu_sort_keys_u32(keys, 0, 32)       # not recorded
    assert len(rs.rs_timing_collect()) == len(first)
    rs.rs_timing_enable(True)
    try:
        assert rs.rs_timing_collect() == []
    finally:
        rs.rs_timing_enable(False)
