"""Pins of the CPU oracle against facts fixed outside it.

Each ``pin_*`` function takes an ``oracle.Oracle`` and raises AssertionError
when the oracle disagrees with:

* the worked examples printed on the pages (``tests/golden/``),
* brute force: Python's ``sorted`` (guaranteed stable) on the ordering field,
  exhaustively over tiny arrays and on random small ones,
* an IEEE 754 totalOrder key built here from the sign and magnitude bits, and
  Python float comparisons for the non-NaN values,
* numpy library routines (stable ``argsort``, ``bincount``, boolean masks),
* invariants that define a stable sort (permutation, order, stability) and
  special cases that reduce to identities.

The same functions run against builds of the oracle with planted mistakes
(``test_oracle_mutants.py``) to show that every plausible slip is caught.
"""
import itertools
import math
import os
import struct

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def read_golden(name):
    fields = {}
    with open(os.path.join(GOLDEN, name), encoding="utf-8") as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            k, v = line.split(":", 1)
            fields[k.strip()] = v.split()
    return fields


def field_of(k, begin_bit, end_bit):
    width = end_bit - begin_bit
    if width == 0:
        return 0
    return (int(k) >> begin_bit) & ((1 << width) - 1)


def stable_reference(keys, begin_bit, end_bit):
    """Permutation that stably sorts `keys` by their field (Python's stable sort)."""
    ks = [int(k) for k in keys]
    return sorted(range(len(ks)), key=lambda i: field_of(ks[i], begin_bit, end_bit))


def total_order_key(bits):
    """IEEE 754 totalOrder of a binary32 pattern as a sortable tuple.

    Negative patterns order by decreasing magnitude bits, non-negative ones by
    increasing magnitude bits; every negative pattern precedes every
    non-negative one (so -NaN < -inf < ... < -0 < +0 < ... < +inf < +NaN).
    """
    bits = int(bits)
    mag = bits & 0x7FFFFFFF
    if bits >> 31:
        return (0, -mag)
    return (1, mag)


def f32_value(bits):
    return struct.unpack("<f", struct.pack("<I", int(bits)))[0]


def float_compare_key(bits):
    """Key from the float value itself, -0.0 before +0.0 (non-NaN only)."""
    x = f32_value(bits)
    assert not math.isnan(x)
    return (x, math.copysign(1.0, x))


def check_sorted_pairs(keys_in, keys_out, vals_out, begin_bit, end_bit):
    """Stable-sort invariants with values = original indices (vectorised)."""
    keys_in = np.asarray(keys_in, np.uint32)
    keys_out = np.asarray(keys_out, np.uint32)
    vals_out = np.asarray(vals_out, np.uint32)
    n = keys_in.size
    assert keys_out.size == n and vals_out.size == n
    if n == 0:
        return
    seen = np.zeros(n, np.int64)
    np.add.at(seen, vals_out.astype(np.int64), 1)
    assert np.all(seen == 1), "values are not a permutation of 0..n-1"
    assert np.array_equal(keys_out, keys_in[vals_out.astype(np.int64)]), "key/value association broken"
    width = end_bit - begin_bit
    mask = np.uint64((1 << width) - 1) if width else np.uint64(0)
    f = (keys_out.astype(np.uint64) >> np.uint64(begin_bit)) & mask
    assert np.all(f[1:] >= f[:-1]), "field not non-decreasing"
    eq = f[1:] == f[:-1]
    assert np.all(vals_out[1:][eq] > vals_out[:-1][eq]), "not stable"


# --- worked examples -------------------------------------------------------------

def pin_radix_golden(o):
    g = read_golden("radix_example.txt")
    keys = np.array([int(x) for x in g["keys_in"]], np.uint32)
    want_k = np.array([int(x) for x in g["keys_out"]], np.uint32)
    want_v = np.array([int(x) for x in g["vals_out"]], np.uint32)
    assert np.array_equal(o.sort_u32(keys), want_k)
    k, v = o.sort_u32(keys, np.arange(keys.size, dtype=np.uint32))
    assert np.array_equal(k, want_k) and np.array_equal(v, want_v)


def pin_compaction_golden(o):
    g = read_golden("compaction_example.txt")
    x = np.array([float(s) for s in g["in"]], np.float32)
    want = np.array([float(s) for s in g["out"]], np.float32)
    out, k = o.compact_positive_f32(x)
    assert k == int(g["count"][0])
    assert np.array_equal(out.view(np.uint32), want.view(np.uint32))


def pin_bitonic_golden(o):
    g = read_golden("bitonic_exercise.txt")
    keys = np.array([int(x) for x in g["keys_in"]], np.uint32)
    want = np.array([int(x) for x in g["keys_out"]], np.uint32)
    assert np.array_equal(o.bitonic_tile(keys, keys.size), want)
    assert np.array_equal(o.sort_u32(keys), want)


# --- brute force -------------------------------------------------------------------

EXHAUSTIVE_ALPHABET = [0x00000000, 0x000000FF, 0x00000100, 0x80000001, 0xFFFFFFFF]
EXHAUSTIVE_RANGES = [(0, 32), (0, 8), (8, 16), (4, 13), (0, 1), (31, 32), (7, 7), (1, 9)]


def pin_bruteforce_exhaustive(o, max_n=6, alphabet_size=4):
    alpha = EXHAUSTIVE_ALPHABET[:alphabet_size]
    for n in range(0, max_n + 1):
        for combo in itertools.product(alpha, repeat=n):
            keys = np.array(combo, np.uint32)
            vals = np.arange(n, dtype=np.uint32)
            for (b, e) in EXHAUSTIVE_RANGES:
                perm = stable_reference(keys, b, e)
                k, v = o.sort_u32(keys, vals, b, e)
                assert list(v) == perm, (combo, b, e)
                assert list(k) == [int(keys[i]) for i in perm]


def pin_bruteforce_random(o, cases=300, seed=1):
    rng = np.random.default_rng(seed)
    for c in range(cases):
        n = int(rng.integers(0, 257))
        kind = c % 3
        if kind == 0:
            keys = rng.integers(0, 2**32, n, dtype=np.uint32)
        elif kind == 1:
            keys = rng.integers(0, 6, n, dtype=np.uint32) * np.uint32(0x01010101)
        else:
            keys = (rng.integers(0, 2**32, n, dtype=np.uint32) & np.uint32(0x0F0F00F3))
        b = int(rng.integers(0, 33))
        e = int(rng.integers(b, 33))
        digit_bits = int(rng.choice([1, 3, 4, 8, 11, 16]))
        vals = np.arange(n, dtype=np.uint32)
        perm = stable_reference(keys, b, e)
        k, v = o.sort_u32(keys, vals, b, e, digit_bits)
        assert list(v) == perm, (c, n, b, e, digit_bits)
        assert np.array_equal(k, keys[np.array(perm, dtype=np.int64)] if n else keys)
        assert np.array_equal(o.sort_u32(keys, None, b, e, digit_bits), k)


# --- floats --------------------------------------------------------------------------

# IEEE 754 totalOrder ladder of binary32 patterns, smallest first.
FLOAT_LADDER = [
    0xFFC00000,  # -qNaN
    0xFF800000,  # -inf
    0xC0000000,  # -2.0
    0xBF800000,  # -1.0
    0x80800000,  # -min normal
    0x806CE3EE,  # -1e-38 (subnormal)
    0x80000001,  # -min subnormal
    0x80000000,  # -0.0
    0x00000000,  # +0.0
    0x00000001,  # +min subnormal
    0x006CE3EE,  # +1e-38 (subnormal)
    0x00800000,  # +min normal
    0x3F800000,  # +1.0
    0x40000000,  # +2.0
    0x7F800000,  # +inf
    0x7FC00000,  # +qNaN
]


def random_float_patterns(rng, n):
    cls = rng.integers(0, 6, n)
    bits = rng.integers(0, 2**32, n, dtype=np.uint32)
    sign = (rng.integers(0, 2, n, dtype=np.uint32) << np.uint32(31)).astype(np.uint32)
    out = bits.copy()
    sub = (bits & np.uint32(0x007FFFFF)) | sign
    out[cls == 1] = sub[cls == 1]                                   # subnormals / zeros
    out[cls == 2] = (sign | np.uint32(0))[cls == 2]                 # signed zeros
    out[cls == 3] = (sign | np.uint32(0x7F800000))[cls == 3]        # infinities
    out[cls == 4] = np.array(FLOAT_LADDER, np.uint32)[rng.integers(0, len(FLOAT_LADDER), n)][cls == 4]
    return out


def pin_float_order(o, cases=200, seed=2):
    ladder = np.array(FLOAT_LADDER, np.uint32)
    rng = np.random.default_rng(seed)
    for _ in range(20):
        perm = rng.permutation(ladder.size)
        got = o.sort_f32(ladder[perm].view(np.float32)).view(np.uint32)
        assert np.array_equal(got, ladder)
    for c in range(cases):
        n = int(rng.integers(0, 129))
        bits = random_float_patterns(rng, n)
        vals = np.arange(n, dtype=np.uint32)
        perm = sorted(range(n), key=lambda i: total_order_key(bits[i]))
        k, v = o.sort_f32(bits.view(np.float32), vals)
        assert list(v) == perm, c
        assert np.array_equal(k.view(np.uint32), bits[np.array(perm, np.int64)] if n else bits)
        finite = [i for i in range(n) if not math.isnan(f32_value(bits[i]))]
        sub = bits[np.array(finite, np.int64)] if finite else np.zeros(0, np.uint32)
        perm2 = sorted(range(sub.size), key=lambda i: float_compare_key(sub[i]))
        k2, v2 = o.sort_f32(sub.view(np.float32), np.arange(sub.size, dtype=np.uint32))
        assert list(v2) == perm2


def pin_float_transform_sampled(o, n=1 << 20, seed=3):
    """Transform order agrees with float comparison on random non-NaN pairs."""
    rng = np.random.default_rng(seed)
    a = random_float_patterns(rng, n)
    b = random_float_patterns(rng, n)
    fa, fb = a.view(np.float32), b.view(np.float32)
    ok = ~(np.isnan(fa) | np.isnan(fb))
    a, b, fa, fb = a[ok], b[ok], fa[ok], fb[ok]
    oa, ob = o.f32_to_order(a), o.f32_to_order(b)
    sa = np.signbit(fa)
    sb = np.signbit(fb)
    # float order with -0 < +0: compare values, then sign as tie-break
    less = (fa < fb) | ((fa == fb) & sa & ~sb)
    equal = (a == b)
    assert np.array_equal(oa < ob, less)
    assert np.array_equal(oa == ob, equal)


def pin_float_transform_roundtrip_exhaustive(o, chunk=1 << 24):
    """The transform is a bijection on all 2^32 patterns and round-trips."""
    base = np.arange(chunk, dtype=np.uint32)
    one = np.uint32(1)
    for s in range(0, 1 << 32, chunk):
        bits = base + np.uint32(s)
        ordr = o.f32_to_order(bits)
        back = o.order_to_f32(ordr)
        assert np.array_equal(back, bits), hex(s)
        # within one sign half the transform is monotone in the pattern:
        # increasing for non-negative patterns, decreasing for negative ones
        if s < (1 << 31):
            assert np.all(ordr[1:] - ordr[:-1] == one), hex(s)
        else:
            assert np.all(ordr[:-1] - ordr[1:] == one), hex(s)
    assert o.f32_to_order(np.array([0x7FFFFFFF], np.uint32))[0] == 0xFFFFFFFF
    assert o.f32_to_order(np.array([0xFFFFFFFF], np.uint32))[0] == 0x00000000


# --- large-input invariants and identities ---------------------------------------

def pin_invariants_large(o, n=1 << 20, seed=4):
    rng = np.random.default_rng(seed)
    for keys, (b, e) in [
        (rng.integers(0, 2**32, n, dtype=np.uint32), (0, 32)),
        (rng.integers(0, 1000, n, dtype=np.uint32), (0, 32)),
        (rng.integers(0, 2**32, n, dtype=np.uint32), (4, 13)),
        (rng.integers(0, 2**16, n, dtype=np.uint32), (0, 16)),
    ]:
        vals = np.arange(n, dtype=np.uint32)
        k, v = o.sort_u32(keys, vals, b, e)
        check_sorted_pairs(keys, k, v, b, e)
        f = (keys.astype(np.uint64) >> np.uint64(b)) & np.uint64((1 << (e - b)) - 1)
        ref = np.argsort(f, kind="stable").astype(np.uint32)
        assert np.array_equal(v, ref)


def pin_digit_width_invariance(o, n=1 << 16, seed=5):
    rng = np.random.default_rng(seed)
    keys = rng.integers(0, 2**32, n, dtype=np.uint32)
    keys[rng.integers(0, n, n // 4)] = np.uint32(0xFFFFFFFF)
    vals = np.arange(n, dtype=np.uint32)
    for (b, e) in [(0, 32), (3, 29), (0, 16), (16, 32), (5, 6)]:
        ref = o.sort_u32(keys, vals, b, e, 8)
        for bits in (1, 2, 4, 5, 11, 16):
            got = o.sort_u32(keys, vals, b, e, bits)
            assert np.array_equal(got[0], ref[0]) and np.array_equal(got[1], ref[1]), (b, e, bits)


def pin_special_cases(o, seed=6):
    rng = np.random.default_rng(seed)
    empty = np.zeros(0, np.uint32)
    k, v = o.sort_u32(empty, empty)
    assert k.size == 0 and v.size == 0
    one = np.array([0xDEADBEEF], np.uint32)
    assert np.array_equal(o.sort_u32(one), one)
    n = 5000
    keys = rng.integers(0, 2**32, n, dtype=np.uint32)
    ident = np.arange(n, dtype=np.uint32)
    for b in (0, 7, 32):                       # empty bit range: identity
        k, v = o.sort_u32(keys, ident, b, b)
        assert np.array_equal(k, keys) and np.array_equal(v, ident)
    same = np.full(n, 0x12345678, np.uint32)   # all equal: identity permutation
    k, v = o.sort_u32(same, ident)
    assert np.array_equal(v, ident)
    allmax = np.full(n, 0xFFFFFFFF, np.uint32)
    k, v = o.sort_u32(allmax, ident)
    assert np.array_equal(v, ident) and np.array_equal(k, allmax)
    distinct = np.unique(keys)
    k, v = o.sort_u32(distinct, np.arange(distinct.size, dtype=np.uint32))
    assert np.array_equal(v, np.arange(distinct.size, dtype=np.uint32))
    rev = distinct[::-1].copy()
    k, v = o.sort_u32(rev, np.arange(rev.size, dtype=np.uint32))
    assert np.array_equal(v, np.arange(rev.size, dtype=np.uint32)[::-1])
    assert np.array_equal(k, distinct)


def pin_histograms(o, n=1 << 18, seed=7):
    rng = np.random.default_rng(seed)
    keys = rng.integers(0, 2**32, n, dtype=np.uint32)
    keys[: n // 8] = rng.integers(0, 3, n // 8, dtype=np.uint32)
    for (b, e) in [(0, 32), (0, 16), (4, 13), (31, 32), (9, 9)]:
        h = o.digit_histograms(keys, b, e)
        passes = (e - b + 7) // 8
        assert h.shape == (passes, 256)
        for p in range(passes):
            s = b + 8 * p
            w = min(8, e - s)
            d = (keys.astype(np.uint64) >> np.uint64(s)) & np.uint64((1 << w) - 1)
            ref = np.bincount(d.astype(np.int64), minlength=256)
            assert np.array_equal(h[p], ref.astype(np.uint64)), (b, e, p)
    # float keys: counts of the transform's digits, and they match the
    # run lengths of the sorted output's digits
    x = rng.standard_normal(n).astype(np.float32)
    hf = o.digit_histograms(x, 0, 32, transform_f32=True)
    sk = o.sort_f32(x)
    ordr = o.f32_to_order(sk)
    for p in range(4):
        d = (ordr >> np.uint32(8 * p)) & np.uint32(255)
        assert np.array_equal(hf[p], np.bincount(d.astype(np.int64), minlength=256).astype(np.uint64))
    top = (ordr >> np.uint32(24)).astype(np.int64)
    assert np.all(np.diff(top) >= 0)


def pin_compaction(o, seed=8):
    rng = np.random.default_rng(seed)
    specials = np.array([0x00000000, 0x80000000, 0x00000001, 0x80000001, 0x006CE3EE,
                         0x806CE3EE, 0x7F800000, 0xFF800000, 0x7FC00000, 0xFFC00000,
                         0x3F800000, 0xBF800000], np.uint32).view(np.float32)
    cases = [np.zeros(0, np.float32), specials, np.ones(1000, np.float32),
             -np.ones(1000, np.float32), np.zeros(777, np.float32)]
    for n in (1, 2, 63, 64, 65, 4095, 4096, 4097, 100003):
        x = rng.standard_normal(n).astype(np.float32)
        x[rng.integers(0, n, n // 10 + 1)] = 0.0
        cases.append(x)
        cases.append(np.concatenate([x, specials]))
    for x in cases:
        out, k = o.compact_positive_f32(x)
        keep = x > np.float32(0)
        assert k == int(keep.sum())
        assert np.array_equal(out[:k].view(np.uint32), x[keep].view(np.uint32))
        assert np.all(out[k:].view(np.uint32) == 0)
    # positive subnormals are kept (denormals honoured)
    out, k = o.compact_positive_f32(np.array([0x00000001], np.uint32).view(np.float32))
    assert k == 1 and out.view(np.uint32)[0] == 1


def pin_bitonic_tile(o, seed=9):
    rng = np.random.default_rng(seed)
    for n, tile, (b, e) in [(1024, 1024, (0, 32)), (1000, 1024, (0, 32)), (3000, 1024, (0, 32)),
                            (4099, 256, (0, 32)), (513, 1, (0, 32)), (700, 100, (4, 13)),
                            (2048, 1000, (0, 8)), (0, 64, (0, 32))]:
        keys = rng.integers(0, 2**32, n, dtype=np.uint32)
        if n:
            keys[rng.integers(0, n, n // 5)] = np.uint32(0xFFFFFFFF)
        got = o.bitonic_tile(keys, tile, b, e)
        width = e - b
        for s in range(0, n, tile):
            seg = keys[s:s + tile]
            f = (seg.astype(np.uint64) >> np.uint64(b)) & np.uint64((1 << width) - 1)
            assert np.array_equal(got[s:s + tile], seg[np.argsort(f, kind="stable")]), (n, tile, s)


# --- key types, 64-bit keys, descending order, multi-key ---------------------------

INT_TYPES = (np.uint32, np.int32, np.uint64, np.int64)
FLOAT_TYPES = (np.float32, np.float64)

# IEEE 754 totalOrder ladder of binary64 patterns, smallest first.
F64_LADDER = [
    0xFFF8000000000000,  # -qNaN
    0xFFF0000000000000,  # -inf
    0xC000000000000000,  # -2.0
    0xBFF0000000000000,  # -1.0
    0x8010000000000000,  # -min normal
    0x8000000000000001,  # -min subnormal
    0x8000000000000000,  # -0.0
    0x0000000000000000,  # +0.0
    0x0000000000000001,  # +min subnormal
    0x0010000000000000,  # +min normal
    0x3FF0000000000000,  # +1.0
    0x4000000000000000,  # +2.0
    0x7FF0000000000000,  # +inf
    0x7FF8000000000000,  # +qNaN
]


def total_order_key_bits(bits, width):
    """IEEE 754 totalOrder of a binary32/binary64 pattern as a sortable tuple."""
    bits = int(bits)
    sign = bits >> (width - 1)
    mag = bits & ((1 << (width - 1)) - 1)
    return (0, -mag) if sign else (1, mag)


def typed_sample(rng, dtype, n):
    """Keys of `dtype` with duplicates, extremes and (for floats) specials."""
    if dtype in (np.uint32, np.int32):
        raw = rng.integers(0, 2**32, n, dtype=np.uint32)
        pool = np.array([0, 1, 0x7FFFFFFF, 0x80000000, 0x80000001, 0xFFFFFFFF, 0x12345678],
                        np.uint32)
        pick = rng.integers(0, 3, n) == 0
        raw[pick] = pool[rng.integers(0, pool.size, int(pick.sum()))]
        return raw.view(dtype)
    if dtype == np.float32:
        return random_float_patterns(rng, n).view(np.float32)
    raw = rng.integers(0, 2**64, n, dtype=np.uint64)
    if dtype == np.float64:
        cls = rng.integers(0, 4, n)
        ladder = np.array(F64_LADDER, np.uint64)
        raw[cls == 1] = ladder[rng.integers(0, ladder.size, n)][cls == 1]
        raw[cls == 2] = raw[cls == 2] & np.uint64(0x800FFFFFFFFFFFFF)   # subnormals, zeros
        return raw.view(np.float64)
    pool = np.array([0, 1, 0x7FFFFFFFFFFFFFFF, 0x8000000000000000, 0xFFFFFFFFFFFFFFFF,
                     0x00000000FFFFFFFF, 0x0000000100000000, 0xFFFFFFFF00000000], np.uint64)
    pick = rng.integers(0, 3, n) == 0
    raw[pick] = pool[rng.integers(0, pool.size, int(pick.sum()))]
    return raw.view(dtype)


def value_key(x, dtype):
    """Sort key from the value: Python ints, or totalOrder for floats."""
    if dtype in INT_TYPES:
        return int(x)
    width = np.dtype(dtype).itemsize * 8
    bits = np.array([x], dtype).view(np.uint32 if width == 32 else np.uint64)[0]
    return total_order_key_bits(bits, width)


def order_pattern_np(keys, descending=False):
    """Order patterns of typed keys, written with numpy bit operations (an
    XOR form of the offsets and transforms the oracle states arithmetically)."""
    dt = keys.dtype.type
    if dt in (np.uint32, np.int32, np.float32):
        u = keys.view(np.uint32).copy()
        top = np.uint32(0x80000000)
        allb = np.uint32(0xFFFFFFFF)
    else:
        u = keys.view(np.uint64).copy()
        top = np.uint64(1 << 63)
        allb = np.uint64(0xFFFFFFFFFFFFFFFF)
    if dt in (np.int32, np.int64):
        u ^= top
    elif dt in (np.float32, np.float64):
        neg = (u & top) != 0
        u = np.where(neg, u ^ allb, u | top)
    if descending:
        u ^= allb
    return u


def pin_typed_bruteforce(o, cases=240, seed=10):
    """Full-range typed sorts against Python's stable sorted on the values."""
    rng = np.random.default_rng(seed)
    types = INT_TYPES + FLOAT_TYPES
    for c in range(cases):
        dt = types[c % len(types)]
        desc = (c // len(types)) % 2 == 1
        n = int(rng.integers(0, 97))
        keys = typed_sample(rng, dt, n)
        vals = np.arange(n, dtype=np.uint32)
        ref = sorted(range(n), key=lambda i: value_key(keys[i], dt), reverse=desc)
        k, v = o.sort_typed(keys, vals, descending=desc)
        assert list(v) == ref, (dt, desc, c)
        width = np.dtype(dt).itemsize * 8
        raw = np.uint32 if width == 32 else np.uint64
        assert np.array_equal(k.view(raw), keys.view(raw)[np.array(ref, np.int64)] if n else
                              keys.view(raw)), (dt, desc, c)
        assert np.array_equal(o.sort_typed(keys, None, descending=desc).view(raw), k.view(raw))
        if dt in FLOAT_TYPES:
            # non-NaN values by float comparison, -0.0 before +0.0 (reversed when descending)
            fin = np.array([i for i in range(n) if not math.isnan(float(keys[i]))], np.int64)
            sub = keys[fin] if fin.size else keys[:0]
            key = lambda i: (float(sub[i]), math.copysign(1.0, float(sub[i])))
            ref2 = sorted(range(sub.size), key=key, reverse=desc)
            _, v2 = o.sort_typed(sub, np.arange(sub.size, dtype=np.uint32), descending=desc)
            assert list(v2) == ref2, (dt, desc, c)


def pin_typed_bit_ranges(o, n=1 << 14, seed=11):
    """Partial bit ranges select bits of the order pattern: the permutation is
    numpy's stable argsort of that field."""
    rng = np.random.default_rng(seed)
    for dt in INT_TYPES + FLOAT_TYPES:
        width = np.dtype(dt).itemsize * 8
        keys = typed_sample(rng, dt, n)
        vals = np.arange(n, dtype=np.uint32)
        for desc in (False, True):
            pat = order_pattern_np(keys, desc).astype(np.uint64)
            for _ in range(4):
                b = int(rng.integers(0, width + 1))
                e = int(rng.integers(b, width + 1))
                mask = np.uint64((1 << (e - b)) - 1) if e - b < 64 else np.uint64(0xFFFFFFFFFFFFFFFF)
                f = (pat >> np.uint64(b)) & mask
                ref = np.argsort(f, kind="stable")
                digit_bits = int(rng.choice([3, 8, 11]))
                _, v = o.sort_typed(keys, vals, b, e, desc, digit_bits)
                assert np.array_equal(v, ref.astype(np.uint32)), (dt, desc, b, e)


def pin_u64_lsd(o, seed=12):
    """64-bit LSD sort: exhaustive tiny arrays over an alphabet that differs in
    both words, and numpy's stable argsort on random fields."""
    alpha = [0x0000000000000000, 0x00000000FFFFFFFF, 0x0000000100000000, 0xFFFFFFFF00000001]
    for n in range(0, 6):
        for combo in itertools.product(alpha, repeat=n):
            keys = np.array(combo, np.uint64)
            vals = np.arange(n, dtype=np.uint32)
            for (b, e) in [(0, 64), (0, 32), (32, 64), (28, 36), (31, 33), (5, 5)]:
                ref = sorted(range(n), key=lambda i: (int(keys[i]) >> b) & ((1 << (e - b)) - 1))
                k, v = o.sort_u64(keys, vals, b, e)
                assert list(v) == ref, (combo, b, e)
    rng = np.random.default_rng(seed)
    n = 1 << 16
    keys = rng.integers(0, 2**64, n, dtype=np.uint64)
    keys[: n // 4] &= np.uint64(0xFFFF0000FFFF00FF)
    vals = np.arange(n, dtype=np.uint32)
    for (b, e, bits) in [(0, 64, 8), (0, 64, 16), (3, 61, 5), (30, 40, 8), (0, 33, 11)]:
        f = (keys >> np.uint64(b)) & np.uint64((1 << (e - b)) - 1 if e - b < 64 else 2**64 - 1)
        k, v = o.sort_u64(keys, vals, b, e, bits)
        assert np.array_equal(v, np.argsort(f, kind="stable").astype(np.uint32)), (b, e, bits)
        assert np.array_equal(k, keys[v])


def pin_two_keys(o, seed=13):
    """Multi-key: brute force on tiny inputs and numpy's lexsort (a stable
    sort on the last key, then the one before) on larger ones."""
    rng = np.random.default_rng(seed)
    for c in range(150):
        n = int(rng.integers(0, 40))
        first = rng.integers(0, 4, n, dtype=np.uint32) * np.uint32(0x40000001)
        second = rng.integers(0, 3, n, dtype=np.uint32) << np.uint32(30)
        vals = np.arange(n, dtype=np.uint32)
        ref = sorted(range(n), key=lambda i: (int(second[i]), int(first[i])))
        f, s2, v = o.sort_two_keys(first, second, vals)
        assert list(v) == ref, c
        assert np.array_equal(f, first[v]) and np.array_equal(s2, second[v])
    n = 1 << 16
    first = rng.integers(0, 2**32, n, dtype=np.uint32)
    first[: n // 2] &= np.uint32(0xF)
    second = rng.integers(0, 50, n, dtype=np.uint32)
    vals = np.arange(n, dtype=np.uint32)
    f, s2, v = o.sort_two_keys(first, second, vals)
    assert np.array_equal(v, np.lexsort((first, second)).astype(np.uint32))
    f2, s3 = o.sort_two_keys(first, second)
    assert np.array_equal(f2, f) and np.array_equal(s3, s2)


def pin_histograms_typed(o, n=1 << 15, seed=14):
    """Typed digit counts equal numpy's bincount of the order pattern's digits,
    and the top-digit counts of signed keys equal a count by value ranges."""
    rng = np.random.default_rng(seed)
    for dt in INT_TYPES + FLOAT_TYPES:
        width = np.dtype(dt).itemsize * 8
        keys = typed_sample(rng, dt, n)
        for desc in (False, True):
            pat = order_pattern_np(keys, desc).astype(np.uint64)
            for (b, e) in [(0, width), (4, width - 3), (width - 8, width)]:
                h = o.digit_histograms_typed(keys, b, e, desc)
                for p in range(h.shape[0]):
                    s = b + 8 * p
                    w = min(8, e - s)
                    d = (pat >> np.uint64(s)) & np.uint64((1 << w) - 1)
                    ref = np.bincount(d.astype(np.int64), minlength=256).astype(np.uint64)
                    assert np.array_equal(h[p], ref), (dt, desc, b, e, p)
    # signed keys: the top 8 bits of the pattern count the keys in the value
    # ranges [-2^31 + k 2^24, -2^31 + (k + 1) 2^24)
    x = rng.integers(-2**31, 2**31, n, dtype=np.int64).astype(np.int32)
    h = o.digit_histograms_typed(x, 24, 32)
    by_range = np.bincount(((x.astype(np.int64) + 2**31) // 2**24), minlength=256)
    assert np.array_equal(h[0], by_range.astype(np.uint64))


# --- scan and select --------------------------------------------------------------

def pin_scan(o, seed=15):
    """Prefix sums against numpy's cumsum (taken in 64 bits, then reduced
    modulo 2^32) and closed forms."""
    rng = np.random.default_rng(seed)
    for n in (0, 1, 2, 63, 64, 65, 1000, 1 << 16):
        for hi in (3, 2**20, 2**32):
            x = rng.integers(0, hi, n, dtype=np.uint64).astype(np.uint32)
            inc = (np.cumsum(x.astype(np.uint64)) & np.uint64(0xFFFFFFFF)).astype(np.uint32)
            exc = np.concatenate([np.zeros(min(n, 1), np.uint32), inc[:-1]]) if n else inc
            assert np.array_equal(o.scan_u32(x, inclusive=True), inc), (n, hi)
            assert np.array_equal(o.scan_u32(x), exc), (n, hi)
    n = 100000
    assert np.array_equal(o.scan_u32(np.ones(n, np.uint32)), np.arange(n, dtype=np.uint32))
    i = np.arange(n, dtype=np.uint64)
    tri = ((i * (i - 1) // 2) & np.uint64(0xFFFFFFFF)).astype(np.uint32)   # sum of 0 .. i-1
    assert np.array_equal(o.scan_u32(np.arange(n, dtype=np.uint32)), tri)


SELECT_OPS = ["<", "<=", ">", ">=", "==", "!="]


def _np_compare(x, op, t):
    return {"<": x < t, "<=": x <= t, ">": x > t, ">=": x >= t, "==": x == t, "!=": x != t}[op]


def pin_select(o, seed=16):
    """Select and partition against numpy boolean masks (IEEE comparisons for
    floats, signed or unsigned for integers), the pages' worked compaction
    example, and brute force with Python comparisons."""
    g = read_golden("compaction_example.txt")
    x = np.array([float(v) for v in g["in"]], np.float32)
    kept, k = o.select(x, ">", 0.0)
    assert k == int(g["count"][0])
    want = np.array([float(v) for v in g["out"]], np.float32)[:k]
    assert np.array_equal(kept[:k].view(np.uint32), want.view(np.uint32))
    part, k = o.select(x, ">", 0.0, partition=True)
    assert np.array_equal(part.view(np.uint32),
                          np.concatenate([x[x > 0], x[~(x > 0)]]).view(np.uint32))
    rng = np.random.default_rng(seed)
    specials = np.array(FLOAT_LADDER, np.uint32).view(np.float32)
    for dt in (np.uint32, np.int32, np.float32):
        for n in (0, 1, 100, 4099, 70000):
            if dt == np.float32:
                x = random_float_patterns(rng, n).view(np.float32)
                t_choices = list(specials) + [np.float32(0.5)]
            else:
                x = typed_sample(rng, dt, n)
                t_choices = [dt(0), dt(7), np.array([0x80000000], np.uint32).view(dt)[0]]
                if n:
                    t_choices.append(x[n // 2])
            vals = np.arange(n, dtype=np.uint32)
            for op in SELECT_OPS:
                t = t_choices[int(rng.integers(0, len(t_choices)))]
                with np.errstate(invalid="ignore"):
                    mask = _np_compare(x, op, t)
                out, vo, k = o.select(x, op, t, vals)
                assert k == int(mask.sum()), (dt, n, op, t)
                raw = x.view(np.uint32)
                assert np.array_equal(out.view(np.uint32)[:k], raw[mask]), (dt, n, op)
                assert np.array_equal(vo[:k], vals[mask])
                out, vo, k = o.select(x, op, t, vals, partition=True)
                assert np.array_equal(out.view(np.uint32),
                                      np.concatenate([raw[mask], raw[~mask]])), (dt, n, op)
                assert np.array_equal(vo, np.concatenate([vals[mask], vals[~mask]]))
    # brute force with Python comparisons on tiny inputs
    ops = {"<": lambda a, b: a < b, "<=": lambda a, b: a <= b, ">": lambda a, b: a > b,
           ">=": lambda a, b: a >= b, "==": lambda a, b: a == b, "!=": lambda a, b: a != b}
    alphabet = [-1.5, -0.0, 0.0, 1e-40, 2.0, float("nan"), float("inf")]
    for combo in itertools.product(alphabet, repeat=3):
        x = np.array(combo, np.float32)
        for op, f in ops.items():
            for t in (0.0, 2.0, float("nan")):
                keep = [i for i in range(3) if f(float(x[i]), t)]
                out, k = o.select(x, op, t, partition=True)
                order = keep + [i for i in range(3) if i not in keep]
                assert k == len(keep) and np.array_equal(out.view(np.uint32),
                                                         x.view(np.uint32)[order]), (combo, op, t)


QUICK_PINS = [pin_radix_golden, pin_compaction_golden, pin_bitonic_golden,
              pin_bruteforce_exhaustive, pin_bruteforce_random, pin_float_order,
              pin_float_transform_sampled, pin_invariants_large, pin_digit_width_invariance,
              pin_special_cases, pin_histograms, pin_compaction, pin_bitonic_tile,
              pin_typed_bruteforce, pin_typed_bit_ranges, pin_u64_lsd, pin_two_keys,
              pin_histograms_typed, pin_scan, pin_select]
