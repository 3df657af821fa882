"""Key types, descending order, 64-bit keys, two-key sorts and digit counts on
the GPU, bit for bit against the oracle.

rs_sort_keys / rs_sort_pairs move u32, i32, f32, u64, i64 and f64 keys in
either direction through the same pass kernels as the u32 sort (an XOR
transform on the first pass's load and its inverse on the last pass's
store; two words per key for 8-byte keys).  rs_sort_two_keys_u32 reads and
writes two word arrays around eight 64-bit passes.  rs_digit_counts exposes
the upsweep kernel's counts, the first step of every sort.  Sizes reach the
one-workgroup sort, every one-sweep tile shape with ragged tails, and 2^27
for 8-byte keys.
"""
import numpy as np
import pytest

import oracle
import pins
import workloads
from gpu_helpers import _raw, gpu_digit_counts, gpu_sort_two_keys, gpu_sort_typed
from test_gpu_parity import HLARGE, KLARGE, LARGE, PLARGE, TILE

pytestmark = pytest.mark.gpu

TYPES32 = [np.uint32, np.int32, np.float32]
TYPES64 = [np.uint64, np.int64, np.float64]
T64 = 16384   # keys per tile of the 64-bit passes


def rng(seed):
    return np.random.default_rng(seed)


def check_typed(keys, desc, b=0, e=None, pairs=True):
    e = keys.dtype.itemsize * 8 if e is None else e
    if pairs:
        vals = np.arange(keys.size, dtype=np.uint32)
        k, v = gpu_sort_typed(keys, vals, desc, b, e)
        rk, rv = oracle.sort_typed(keys, vals, b, e, desc)
        assert np.array_equal(v, rv), ("values", keys.dtype, desc, keys.size, b, e)
    else:
        k = gpu_sort_typed(keys, None, desc, b, e)
        rk = oracle.sort_typed(keys, None, b, e, desc)
    assert np.array_equal(_raw(k), _raw(rk)), ("keys", keys.dtype, desc, keys.size, b, e)


@pytest.mark.parametrize("desc", [False, True])
@pytest.mark.parametrize("dtype", TYPES32, ids=lambda t: t.__name__)
@pytest.mark.parametrize("n", [1, 1000, 4097, TILE + 1, 3 * TILE + 17, LARGE + 17, PLARGE + 17])
def test_typed32_pairs(n, dtype, desc):
    print("typed pairs %s desc=%d n=%d" % (dtype.__name__, desc, n), flush=True)
    check_typed(pins.typed_sample(rng(n), dtype, n), desc)


@pytest.mark.parametrize("desc", [False, True])
@pytest.mark.parametrize("dtype", TYPES32, ids=lambda t: t.__name__)
@pytest.mark.parametrize("n", [777, TILE + 1, KLARGE + 17, (1 << 27) + 3 * 32768 + 17])
def test_typed32_keys(n, dtype, desc):
    print("typed keys %s desc=%d n=%d" % (dtype.__name__, desc, n), flush=True)
    check_typed(pins.typed_sample(rng(n + 1), dtype, n), desc, pairs=False)


@pytest.mark.parametrize("dtype", TYPES32, ids=lambda t: t.__name__)
@pytest.mark.parametrize("b,e", [(0, 16), (16, 32), (3, 29), (31, 32), (24, 32)])
def test_typed32_bit_ranges(dtype, b, e):
    n = 3 * TILE + 999
    print("typed %s bits [%d,%d)" % (dtype.__name__, b, e), flush=True)
    keys = pins.typed_sample(rng(b * 40 + e), dtype, n)
    for desc in (False, True):
        check_typed(keys, desc, b, e)


def test_typed32_huge_pairs():
    n = HLARGE + 3 * 28672 + 17
    print("typed pairs i32 descending n=%d" % n, flush=True)
    check_typed(pins.typed_sample(rng(5), np.int32, n), True)


@pytest.mark.parametrize("desc", [False, True])
@pytest.mark.parametrize("dtype", TYPES64, ids=lambda t: t.__name__)
@pytest.mark.parametrize("n", [1, 63, 1000, T64, T64 + 1, 3 * T64 + 17, 256 * T64 + 5])
def test_typed64(n, dtype, desc):
    print("64-bit %s desc=%d n=%d" % (dtype.__name__, desc, n), flush=True)
    keys = pins.typed_sample(rng(n + 7), dtype, n)
    check_typed(keys, desc)
    check_typed(keys, desc, pairs=False)


@pytest.mark.parametrize("dtype", TYPES64, ids=lambda t: t.__name__)
@pytest.mark.parametrize("b,e", [(0, 32), (32, 64), (28, 36), (5, 59), (60, 64), (0, 8)])
def test_typed64_bit_ranges(dtype, b, e):
    n = 5 * T64 + 321
    print("64-bit %s bits [%d,%d)" % (dtype.__name__, b, e), flush=True)
    keys = pins.typed_sample(rng(b * 70 + e), dtype, n)
    for desc in (False, True):
        check_typed(keys, desc, b, e)


def test_u64_pairs_2p27():
    n = 1 << 27
    print("u64 pairs n=2^27: generate", flush=True)
    keys = rng(27).integers(0, 2**64, n, dtype=np.uint64)
    keys[: n // 4] &= np.uint64(0xFFFF00FFFFFF00FF)   # a clustered quarter
    vals = np.arange(n, dtype=np.uint32)
    print("u64 pairs n=2^27: gpu", flush=True)
    k, v = gpu_sort_typed(keys, vals)
    print("u64 pairs n=2^27: oracle", flush=True)
    rk, rv = oracle.sort_typed(keys, vals)
    assert np.array_equal(v, rv) and np.array_equal(k, rk)


@pytest.mark.parametrize("n", [1, 100, T64 + 1, 3 * T64 + 17, (1 << 20) + 17])
@pytest.mark.parametrize("with_vals", [True, False])
def test_two_keys(n, with_vals):
    print("two keys n=%d vals=%d" % (n, with_vals), flush=True)
    r = rng(n + 3)
    major = r.integers(0, 2**32, n, dtype=np.uint32)
    major[: n // 2] = r.integers(0, 7, n // 2, dtype=np.uint32)   # ties on the major key
    minor = r.integers(0, 2**32, n, dtype=np.uint32)
    minor[::3] = r.integers(0, 4, minor[::3].size, dtype=np.uint32)
    vals = np.arange(n, dtype=np.uint32) if with_vals else None
    got = gpu_sort_two_keys(major, minor, vals)
    # the exercise: stable by the minor key first, then stable by the major key
    ref = oracle.sort_two_keys(minor, major, vals)
    assert np.array_equal(got[0], ref[1]) and np.array_equal(got[1], ref[0])
    if with_vals:
        assert np.array_equal(got[2], ref[2])


@pytest.mark.parametrize("dtype", TYPES32 + TYPES64, ids=lambda t: t.__name__)
@pytest.mark.parametrize("n", [0, 5, 1000003])
def test_digit_counts_typed(dtype, n):
    print("digit counts %s n=%d" % (dtype.__name__, n), flush=True)
    keys = pins.typed_sample(rng(n + 11), dtype, n)
    width = keys.dtype.itemsize * 8
    for desc in (False, True):
        for (b, e) in [(0, width), (3, width - 5), (width - 8, width)]:
            got = gpu_digit_counts(keys, desc, b, e)
            ref = oracle.digit_histograms_typed(keys, b, e, desc)
            assert np.array_equal(got.astype(np.uint64), ref), (desc, b, e)


def test_digit_counts_of_the_workloads():
    """The upsweep's counts on the measured workloads' inputs."""
    print("digit counts: 2^28 uniform u32", flush=True)
    keys = workloads.uniform_u32(1 << 28)
    assert np.array_equal(gpu_digit_counts(keys).astype(np.uint64), oracle.digit_histograms(keys))
    print("digit counts: 2^26 Zipf u32, bits [0,16)", flush=True)
    z = workloads.zipf_u32(1 << 26)
    assert np.array_equal(gpu_digit_counts(z, False, 0, 16).astype(np.uint64),
                          oracle.digit_histograms(z, 0, 16))
    print("digit counts: 2^28 f32 with specials", flush=True)
    f = workloads.normal_specials_f32(1 << 28)
    assert np.array_equal(gpu_digit_counts(f).astype(np.uint64),
                          oracle.digit_histograms(f, 0, 32, transform_f32=True))
