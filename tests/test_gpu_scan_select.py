"""Prefix sums, select and stable partition on the GPU, bit for bit against the oracle.

The scan is one pass with a decoupled look-back over 32768-element tiles
(64-bit tile states; sums wrap modulo 2^32).  Select and partition
generalise the compaction: any of six comparisons on u32, i32 or f32
elements, optional values, 32768- (16384- with values) element tiles; the
partition first counts the kept elements.  Sizes cover one element, tile
edges, ragged tails, the 2^28 workload size and the top of the size range.
"""
import numpy as np
import pytest

import oracle
import pins
import workloads
from gpu_helpers import _raw, gpu_scan, gpu_select

pytestmark = pytest.mark.gpu

ST = 32768    # scan tile
SEL = 32768   # select tile without values (16384 with)


def rng(seed):
    return np.random.default_rng(seed)


@pytest.mark.parametrize("n", [1, 3, 4, 5, 1000, ST - 1, ST, ST + 1, 3 * ST + 7, 256 * ST + 5,
                               (1 << 22) + 13])
@pytest.mark.parametrize("inclusive", [False, True])
def test_scan(n, inclusive):
    print("scan n=%d inclusive=%d" % (n, inclusive), flush=True)
    x = rng(n).integers(0, 2**32, n, dtype=np.uint32)   # large values: the sums wrap
    assert np.array_equal(gpu_scan(x, inclusive), oracle.scan_u32(x, inclusive))


def test_scan_in_place_and_small_values():
    n = 5 * ST + 3
    x = rng(3).integers(0, 4, n, dtype=np.uint32)
    assert np.array_equal(gpu_scan(x, False, inplace=True), oracle.scan_u32(x))
    assert np.array_equal(gpu_scan(x, True, inplace=True), oracle.scan_u32(x, True))


def test_scan_2p28():
    n = 1 << 28
    print("scan n=2^28", flush=True)
    x = rng(28).integers(0, 2**32, n, dtype=np.uint32)
    assert np.array_equal(gpu_scan(x), oracle.scan_u32(x))


def test_scan_top_of_range():
    n = (1 << 30) - 1
    print("scan n=2^30-1", flush=True)
    x = rng(30).integers(0, 16, n, dtype=np.uint32)
    assert np.array_equal(gpu_scan(x, True), oracle.scan_u32(x, True))


def check_select(x, op, t, vals, partition):
    o, v, c = gpu_select(x, op, t, vals, partition)
    if vals is None:
        ro, rc = oracle.select(x, op, t, None, partition)
    else:
        ro, rv, rc = oracle.select(x, op, t, vals, partition)
    assert c == rc, (x.dtype, x.size, op, t, partition)
    m = x.size if partition else c
    assert np.array_equal(_raw(o)[:m], _raw(ro)[:m]), (x.dtype, x.size, op, t, partition)
    if vals is not None:
        assert np.array_equal(v[:m], rv[:m])


@pytest.mark.parametrize("partition", [False, True])
@pytest.mark.parametrize("with_vals", [False, True])
@pytest.mark.parametrize("dtype", [np.uint32, np.int32, np.float32], ids=lambda t: t.__name__)
@pytest.mark.parametrize("n", [1, 7, 1000, SEL // 2 - 1, SEL // 2, SEL + 1, 3 * SEL + 77,
                               (1 << 20) + 3])
def test_select_and_partition(n, dtype, with_vals, partition):
    print("select n=%d %s vals=%d partition=%d" % (n, dtype.__name__, with_vals, partition),
          flush=True)
    r = rng(n + 3)
    x = (pins.random_float_patterns(r, n).view(np.float32) if dtype == np.float32
         else pins.typed_sample(r, dtype, n))
    vals = np.arange(n, dtype=np.uint32) if with_vals else None
    thresholds = {np.uint32: [np.uint32(0x80000000), np.uint32(7)],
                  np.int32: [np.int32(0), np.int32(-5)],
                  np.float32: [np.float32(0.0), np.float32(-1.0), np.float32(np.nan)]}[dtype]
    for i, op in enumerate(["<", "<=", ">", ">=", "==", "!="]):
        check_select(x, op, thresholds[i % len(thresholds)], vals, partition)


def test_select_matches_the_compaction_workload():
    """x > 0 over the 2^28 compaction input: the kept run equals the
    compaction's, the partition puts every rejected element after it."""
    x = workloads.compact_input()
    print("select 2^28: gpu", flush=True)
    o, _, c = gpu_select(x, ">", np.float32(0.0), None, True)
    assert c == workloads.signed_mix_expected_count(x.size)
    print("select 2^28: oracle", flush=True)
    ro, rc = oracle.select(x, ">", np.float32(0.0), None, True)
    assert c == rc and np.array_equal(o.view(np.uint32), ro.view(np.uint32))


def test_partition_is_one_radix_split():
    """Partition on bit b (value & mask < threshold) is one stable radix pass of a 1-bit digit."""
    n = 3 * SEL + 5
    x = rng(8).integers(0, 2**32, n, dtype=np.uint32)
    vals = np.arange(n, dtype=np.uint32)
    o, v, c = gpu_select(x, "<", np.uint32(0x80000000), vals, True)
    rk, rv = oracle.sort_u32(x, vals, 31, 32)
    assert np.array_equal(o, rk) and np.array_equal(v, rv)
    assert c == int((x < np.uint32(0x80000000)).sum())
