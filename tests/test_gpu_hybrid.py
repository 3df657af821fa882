"""The hybrid path for 16384 < n <= 3 * 2^20 keys, bit for bit against the oracle.

One pass on the top digit places the keys in their buckets; one workgroup
per bucket then sorts the lower digits in LDS.  Both run only if no bucket
holds more than 16384 keys; otherwise the gated LSD passes run instead (the
device decides from the digit counts, with no host round trip).  The cases
put the largest bucket exactly at and just past the cap, make buckets end on
and just past a 1024-key row, leave buckets empty, use top digits narrower
than 8 bits, and cross the size limit of the path.
"""
import numpy as np
import pytest

import oracle
import pins
from gpu_helpers import gpu_sort_keys_u32, gpu_sort_pairs_u32, gpu_sort_typed

pytestmark = pytest.mark.gpu

CAP = 16384
HYBRID_MAX = 3 << 20


def rng(seed):
    return np.random.default_rng(seed)


def check(keys, b=0, e=32):
    vals = np.arange(keys.size, dtype=np.uint32)
    k, v = gpu_sort_pairs_u32(keys, vals, b, e)
    rk, rv = oracle.sort_u32(keys, vals, b, e)
    assert np.array_equal(v, rv) and np.array_equal(k, rk), (keys.size, b, e)
    assert np.array_equal(gpu_sort_keys_u32(keys, b, e), rk), (keys.size, b, e)


def with_bucket_sizes(sizes, seed):
    """Keys whose top byte d occurs sizes[d] times, lower bytes random, shuffled."""
    r = rng(seed)
    top = np.repeat(np.arange(len(sizes), dtype=np.uint32), sizes)
    keys = (top << np.uint32(24)) | r.integers(0, 1 << 24, top.size, dtype=np.uint32)
    return keys[r.permutation(keys.size)]


@pytest.mark.parametrize("largest", [CAP - 1, CAP, CAP + 1])
def test_largest_bucket_at_the_cap(largest):
    print("hybrid: largest bucket %d" % largest, flush=True)
    sizes = [3000] * 40
    sizes[17] = largest
    keys = with_bucket_sizes(sizes, largest)
    check(keys)


def test_bucket_sizes_on_row_edges_and_empty_buckets():
    print("hybrid: row edges", flush=True)
    sizes = [0, 1, 63, 64, 65, 1023, 1024, 1025, 2047, 2048, 2049, 0, 0, 4096, 8191, 8192, 8193,
             15360, 15361] + [0] * 200 + [5, 777]
    check(with_bucket_sizes(sizes, 3))


# the top-digit pass uses 8192-key tiles up to 256 of them (n <= 2^21) and
# 16384-key tiles above
@pytest.mark.parametrize("n", [CAP + 1, 100000, (1 << 20) + 17, (2 << 20) - 1, 2 << 20, (2 << 20) + 1,
                               HYBRID_MAX, HYBRID_MAX + 1])
def test_uniform_sizes(n):
    print("hybrid: uniform n=%d" % n, flush=True)
    check(rng(n).integers(0, 2**32, n, dtype=np.uint32))


@pytest.mark.parametrize("b,e", [(0, 12), (0, 9), (3, 20), (16, 32), (0, 16), (20, 32)])
def test_narrow_top_digits(b, e):
    n = 300001
    print("hybrid: bits [%d,%d)" % (b, e), flush=True)
    check(rng(b * 50 + e).integers(0, 2**32, n, dtype=np.uint32), b, e)


@pytest.mark.parametrize("kind", ["zipf", "small_range", "two_values"])
def test_skewed_inputs_take_the_lsd_passes(kind):
    n = (1 << 20) + 5
    print("hybrid fallback: %s" % kind, flush=True)
    r = rng(9)
    if kind == "zipf":
        import workloads
        keys = workloads.zipf_u32(n, seed=4)
    elif kind == "small_range":
        keys = r.integers(0, 1 << 20, n, dtype=np.uint32)   # one top-byte bucket
    else:
        keys = r.integers(0, 2, n, dtype=np.uint32) * np.uint32(0x80000001)
    check(keys)
    check(keys, 0, 16)


@pytest.mark.parametrize("dtype", [np.int32, np.float32], ids=lambda t: t.__name__)
@pytest.mark.parametrize("desc", [False, True])
def test_typed_keys_through_the_hybrid_path(dtype, desc):
    n = 500000
    print("hybrid: %s desc=%d" % (dtype.__name__, desc), flush=True)
    keys = pins.typed_sample(rng(n), dtype, n)
    vals = np.arange(n, dtype=np.uint32)
    k, v = gpu_sort_typed(keys, vals, desc)
    rk, rv = oracle.sort_typed(keys, vals, 0, 32, desc)
    assert np.array_equal(v, rv) and np.array_equal(k.view(np.uint32), rk.view(np.uint32))
