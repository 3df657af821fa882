"""The allocation-free compaction entry point against the one with a temp buffer.

rs_compact_positive_f32_noalloc runs the compaction kernels with the
library's static per-device scratch instead of a caller's temp buffer.  Two
calls in a row (the second on a smaller input, so stale tile states and
counters from the first would show) must match rs_compact_positive_f32 and
the oracle bit for bit, through the C ABI.
"""
import numpy as np
import pytest
import torch

import oracle
import sorting_lsd_radix_amd as rs
import workloads
from gpu_helpers import DEV, gpu_compact, host, poisoned, to_dev

pytestmark = pytest.mark.gpu


def noalloc_compact(x):
    n = x.size
    tx = to_dev(x)
    out = poisoned(n, torch.float32)
    cnt = poisoned(1)
    rs.rs_compact_positive_f32_noalloc(tx, out, cnt, n)
    o, c = host(out), int(host(cnt)[0])
    assert np.array_equal(host(tx).view(np.uint32), x.view(np.uint32)), "input modified"
    return o, c


def test_noalloc_compaction_matches_the_temp_buffer_version():
    for n, seed in [(3 * 32768 * 100 + 12345, 1), (32768 + 7, 2), (1000, 3), (0, 4), (65, 5)]:
        print("noalloc compaction n=%d" % n, flush=True)
        x = workloads.signed_mix_f32(n, seed=seed)
        o, c = noalloc_compact(x)
        ro, rc = gpu_compact(x)
        assert c == rc
        assert np.array_equal(o.view(np.uint32), ro.view(np.uint32))
        oo, oc = oracle.compact_positive_f32(x)
        assert c == oc and np.array_equal(o.view(np.uint32), oo.view(np.uint32))


def test_noalloc_compaction_size_limit_and_checks():
    with pytest.raises(rs.RsError) as ei:
        rs.rs_compact_positive_f32_noalloc(0x1000, 0x2000, 0x3000, 1 << 30, 0)
    assert ei.value.status == rs.RS_ERR_UNSUPPORTED_SIZE
    with pytest.raises(rs.RsError) as ei:
        rs.rs_compact_positive_f32_noalloc(0x1000, 0x2000, None, 16, 0)
    assert ei.value.status == rs.RS_ERR_INVALID_VALUE


def test_noalloc_compaction_full_size_then_smaller():
    n = 1 << 28
    print("noalloc compaction n=2^28 then 2^20+3", flush=True)
    x = workloads.compact_input(n)
    o, c = noalloc_compact(x)
    assert c == workloads.signed_mix_expected_count(n)
    ro, rc = oracle.compact_positive_f32(x)
    assert c == rc and np.array_equal(o.view(np.uint32), ro.view(np.uint32))
    del x, o, ro
    y = workloads.signed_mix_f32((1 << 20) + 3, seed=9)
    o2, c2 = noalloc_compact(y)
    r2, rc2 = gpu_compact(y)
    assert c2 == rc2 and np.array_equal(o2.view(np.uint32), r2.view(np.uint32))
