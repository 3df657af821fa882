"""Seeded random sweep of the typed sort entry points, bit for bit against
the oracle.

Each case draws a size from one of three ranges in turn (up to one 16384-key
tile, log-uniform; the hybrid range up to 3 * 2^20; above it up to 6 * 2^20),
so the one-workgroup sort, the hybrid path and its multi-pass fallback, and
the small LSD shapes with both look-back forms are all reached, a key type
(every type equally often, and in every size range), a direction, a bit range (the full width half of the time) and a key
distribution (typed samples with extremes and specials, a narrow range that
crowds the top digit, a handful of values, an already sorted input), and
sorts keys only or keys with index values.

A second sweep draws prefix sums, selects and partitions: sizes log-uniform
up to 2^23 (one case in four between 2^20 and 2^24, so tiles run in several
rounds of the persistent grid), any of the six comparisons against a random
threshold on u32, i32 or f32 elements (floats from random bit patterns, so
NaNs, infinities and signed zeros occur), with or without index values.
"""
import numpy as np
import pytest

import oracle
import pins
from gpu_helpers import _raw, gpu_scan, gpu_select, gpu_sort_typed

pytestmark = pytest.mark.gpu

TYPES = [np.uint32, np.int32, np.float32, np.uint64, np.int64, np.float64]
CASES = 48
MAX_N = 6 << 20


def draw(case):
    r = np.random.default_rng(1000 + case)
    size_class = (case // len(TYPES)) % 3   # every type meets every size range
    if size_class == 0:      # up to one tile (log-uniform)
        n = int(np.exp(r.uniform(0.0, np.log(16384))))
    elif size_class == 1:    # the hybrid range of 4-byte keys
        n = int(r.integers(16385, (3 << 20) + 1))
    else:                    # above it, to 6 * 2^20
        n = int(r.integers((3 << 20) + 1, MAX_N + 1))
    dtype = TYPES[case % len(TYPES)]
    width = np.dtype(dtype).itemsize * 8
    if r.random() < 0.5:
        b, e = 0, width
    else:
        b = int(r.integers(0, width))
        e = int(r.integers(b + 1, width + 1))
    descending = bool(r.random() < 0.3)
    pairs = bool(r.random() < 0.6)
    kind = ["typed", "narrow", "few", "sorted"][int(r.integers(0, 4))]
    keys = pins.typed_sample(r, dtype, n)
    raw = keys.view(np.uint32 if width == 32 else np.uint64)
    if kind == "narrow":      # values below 2^20: one top digit holds every key
        raw &= raw.dtype.type(0xFFFFF)
    elif kind == "few":
        raw[:] = raw[:5][r.integers(0, 5, n)] if n >= 5 else raw
    elif kind == "sorted":
        raw.sort()
    return n, dtype, b, e, descending, pairs, kind, keys


@pytest.mark.parametrize("case", range(CASES))
def test_random_typed_sort(case):
    n, dtype, b, e, descending, pairs, kind, keys = draw(case)
    print("sweep case %d: %s n=%d bits=[%d,%d) %s %s %s" % (
        case, np.dtype(dtype).name, n, b, e, "desc" if descending else "asc",
        "pairs" if pairs else "keys", kind), flush=True)
    bits = (lambda a: a.view(np.uint32 if a.dtype.itemsize == 4 else np.uint64))
    if pairs:
        vals = np.arange(n, dtype=np.uint32)
        k, v = gpu_sort_typed(keys, vals, descending, b, e)
        rk, rv = oracle.sort_typed(keys, vals, b, e, descending)
        assert np.array_equal(bits(k), bits(rk)) and np.array_equal(v, rv)
    else:
        k = gpu_sort_typed(keys, None, descending, b, e)
        rk = oracle.sort_typed(keys, None, b, e, descending)
        assert np.array_equal(bits(k), bits(rk))


STREAM_CASES = 48
OPS = ["<", "<=", ">", ">=", "==", "!="]


@pytest.mark.parametrize("case", range(STREAM_CASES))
def test_random_scan_select_partition(case):
    r = np.random.default_rng(3000 + case)
    if case % 4:
        n = int(np.exp(r.uniform(0.0, np.log(1 << 23))))
    else:
        n = int(r.integers(1 << 20, 1 << 24))
    kind = case % 3
    if kind == 0:
        inclusive = bool(r.random() < 0.5)
        print("stream case %d: scan n=%d inclusive=%d" % (case, n, inclusive), flush=True)
        x = r.integers(0, 1 << 32, n, dtype=np.uint64).astype(np.uint32)
        assert np.array_equal(gpu_scan(x, inclusive), oracle.scan_u32(x, inclusive))
        return
    partition = kind == 2
    dtype = [np.uint32, np.int32, np.float32][int(r.integers(0, 3))]
    op = OPS[int(r.integers(0, len(OPS)))]
    x = (pins.random_float_patterns(r, n).view(np.float32) if dtype == np.float32
         else pins.typed_sample(r, dtype, n))
    t = {np.uint32: np.uint32(r.integers(0, 1 << 32, dtype=np.uint64)),
         np.int32: np.int32(r.integers(-2 ** 31, 2 ** 31 - 1)),
         np.float32: np.float32(r.standard_normal())}[dtype]
    vals = np.arange(n, dtype=np.uint32) if r.random() < 0.5 else None
    print("stream case %d: %s n=%d %s x %s %r vals=%d" % (
        case, "partition" if partition else "select", n, np.dtype(dtype).name, op, t,
        vals is not None), flush=True)
    o, v, c = gpu_select(x, op, t, vals, partition)
    ref = oracle.select(x, op, t, vals, partition)
    assert c == ref[-1]
    m = n if partition else c
    assert np.array_equal(_raw(o)[:m], _raw(ref[0])[:m])
    if vals is not None:
        assert np.array_equal(v[:m], ref[1][:m])
