"""Bit-exact parity of the HIP library with the CPU oracle (needs an MI355X).

Every comparison is on raw bits with tolerance 0: a sort only permutes its
inputs.  Sizes span several tiles and a ragged tail; the named workloads run
at their full sizes, compared element by element with the oracle where it
finishes in seconds and otherwise through the properties that define a
stable sort uniquely (permutation with key/value association, non-decreasing
field, strictly increasing original index among equal fields).
"""
import numpy as np
import pytest

import oracle
import pins
import workloads
from gpu_helpers import (gpu_bitonic, gpu_compact, gpu_sort_keys_u32, gpu_sort_pairs_f32,
                         gpu_sort_pairs_u32, temp_for)

pytestmark = pytest.mark.gpu

# Sort paths: up to TILE keys one workgroup sorts in LDS (tile shapes of 1024,
# 4096 and 16384 keys); above, the one-sweep passes use TILE-key tiles.  LARGE
# is the first size at which every CU gets a tile; pair sorts switch to
# PTILE-key tiles at PLARGE and keys-only sorts to 512-thread blocks of 32
# keys each at KLARGE.
TILE = 16384
STILE = 4096
LARGE = 256 * TILE
KLARGE = 512 * TILE  # keys-only sorts switch to 512 x 32 tiles (two blocks per CU) here
PTILE = 24576  # keys per tile of a pair sort from PLARGE on
PLARGE = 256 * PTILE
HTILE = 28672  # keys per tile of a pair sort from HLARGE on
HLARGE = 1 << 26
CTILE = 32768  # floats per tile of the compaction
SIZES = [1, 2, 63, 64, 65, 1000, 1024, 1025, STILE, STILE + 1, TILE - 1, TILE, TILE + 1,
         3 * TILE + 17, (1 << 20) + 17, LARGE - 1, LARGE, LARGE + 17, PLARGE - 1, PLARGE,
         PLARGE + 2 * PTILE + 17]
RANGES = [(0, 32), (0, 16), (8, 24), (4, 13), (0, 1), (31, 32), (7, 7), (0, 8), (24, 32)]


def rng(seed):
    return np.random.default_rng(seed)


def check_pairs(keys, b, e):
    vals = np.arange(keys.size, dtype=np.uint32)
    k, v = gpu_sort_pairs_u32(keys, vals, b, e)
    rk, rv = oracle.sort_u32(keys, vals, b, e)
    assert np.array_equal(v, rv), ("values", keys.size, b, e)
    assert np.array_equal(k, rk), ("keys", keys.size, b, e)


@pytest.mark.parametrize("n", SIZES)
def test_pairs_u32_sizes_full_range(n):
    print("pairs u32 n=%d" % n, flush=True)
    check_pairs(rng(n).integers(0, 2**32, n, dtype=np.uint32), 0, 32)


@pytest.mark.parametrize("b,e", RANGES)
@pytest.mark.parametrize("n", [65, 3000, TILE + 1, 5 * TILE - 3, LARGE + 2 * TILE + 5,
                               PLARGE + 3 * PTILE + 5])
def test_pairs_u32_bit_ranges(n, b, e):
    print("pairs u32 n=%d bits=[%d,%d)" % (n, b, e), flush=True)
    check_pairs(rng(n + b * 33 + e).integers(0, 2**32, n, dtype=np.uint32), b, e)


DISTRIBUTIONS = ["all_equal", "all_max", "single_digit", "few_values", "sorted", "reversed", "zipf",
                 "top_byte_only", "card24", "card300"]


def dist_keys(kind, n):
    r = rng(11)
    if kind == "all_equal":
        return np.full(n, 0x12345678, np.uint32)
    if kind == "all_max":
        return np.full(n, 0xFFFFFFFF, np.uint32)
    if kind == "single_digit":
        return (r.integers(0, 2**32, n, dtype=np.uint32) & np.uint32(0xFFFF00FF)) | np.uint32(0x5A00)
    if kind == "few_values":
        return r.integers(0, 5, n, dtype=np.uint32) * np.uint32(0x01000001)
    if kind == "sorted":
        return np.sort(r.integers(0, 2**32, n, dtype=np.uint32))
    if kind == "reversed":
        return np.sort(r.integers(0, 2**32, n, dtype=np.uint32))[::-1].copy()
    if kind == "zipf":
        return workloads.zipf_u32(n, seed=3)
    if kind in ("card24", "card300"):
        # few distinct full-width keys: after the first pass equal keys form runs in every tile,
        # so tiles switch between the atomic and the ballot rank
        distinct = r.integers(0, 2**32, 24 if kind == "card24" else 300, dtype=np.uint32)
        return distinct[r.integers(0, distinct.size, n)]
    return r.integers(0, 256, n, dtype=np.uint32) << np.uint32(24)


# LARGE - 17: 256 tiles of 16384 keys, the largest LSD sort whose passes use
# the wide look-back; LARGE + 1234: 257 tiles, the walk
@pytest.mark.parametrize("kind", DISTRIBUTIONS)
@pytest.mark.parametrize("n", [2000, 3 * TILE + 1234, LARGE - 17, LARGE + 1234, PLARGE + 1234])
def test_pairs_u32_distributions(kind, n):
    keys = dist_keys(kind, n)
    print("pairs u32 distribution=%s n=%d" % (kind, n), flush=True)
    for (b, e) in [(0, 32), (0, 16), (16, 32)]:
        check_pairs(keys, b, e)


@pytest.mark.parametrize("b,e", [(0, 32), (3, 29)])
def test_keys_u32_huge_tiles(b, e):
    """Keys-only sorts from 2^27 keys use one 1024 x 32 block per CU (32768-key tiles)."""
    n = (1 << 27) + 3 * 32768 + 17
    print("keys u32 huge tiles n=%d bits=[%d,%d)" % (n, b, e), flush=True)
    keys = rng(n + b).integers(0, 2**32, n, dtype=np.uint32)
    keys[: n // 4] &= np.uint32(0xFF00FFFF)
    assert np.array_equal(gpu_sort_keys_u32(keys, b, e), oracle.sort_u32(keys, None, b, e))


@pytest.mark.parametrize("n", [HLARGE - 1, HLARGE + 3 * HTILE + 17])
def test_pairs_u32_huge_tiles(n):
    """Either side of the switch to 28672-key pair tiles, with a partial last tile."""
    print("pairs u32 huge tiles n=%d" % n, flush=True)
    keys = rng(n).integers(0, 2**32, n, dtype=np.uint32)
    keys[: n // 4] &= np.uint32(0xFFFF00FF)   # a quarter with a common middle byte: clustered tiles
    check_pairs(keys, 0, 32)


@pytest.mark.parametrize("kind", DISTRIBUTIONS)
@pytest.mark.parametrize("n", [3 * TILE + 1234, KLARGE + 1234])
def test_keys_u32_distributions(kind, n):
    """Skewed inputs through both keys-only pass shapes (the first full-range pass of the
    large shape ranks equal keys of a row in any order)."""
    keys = dist_keys(kind, n)
    print("keys u32 distribution=%s n=%d" % (kind, n), flush=True)
    for (b, e) in [(0, 32), (0, 16), (16, 32)]:
        assert np.array_equal(gpu_sort_keys_u32(keys, b, e), oracle.sort_u32(keys, None, b, e)), (b, e)


@pytest.mark.parametrize("n", [1, 64, 1000, 4000, TILE, TILE + 1, 3 * TILE + 17, (1 << 20) + 17,
                               LARGE + 17, KLARGE - 1, KLARGE, KLARGE + 2 * TILE + 17])
@pytest.mark.parametrize("b,e", [(0, 32), (4, 13), (8, 24)])
def test_keys_u32(n, b, e):
    print("keys u32 n=%d bits=[%d,%d)" % (n, b, e), flush=True)
    keys = rng(n * 7 + b).integers(0, 2**32, n, dtype=np.uint32)
    keys[: n // 3] &= np.uint32(0xFF0F0F0F)
    k = gpu_sort_keys_u32(keys, b, e)
    assert np.array_equal(k, oracle.sort_u32(keys, None, b, e))


@pytest.mark.parametrize("n", [1, 65, 1000, 4000, TILE, TILE + 1, 3 * TILE + 17, (1 << 20) + 17,
                               LARGE + 17, PLARGE + 17])
@pytest.mark.parametrize("b,e", [(0, 32), (0, 16), (16, 32), (3, 29), (31, 32)])
def test_pairs_f32(n, b, e):
    print("pairs f32 n=%d bits=[%d,%d)" % (n, b, e), flush=True)
    r = rng(n + 17 * b + e)
    bits = pins.random_float_patterns(r, n)
    vals = np.arange(n, dtype=np.uint32)
    k, v = gpu_sort_pairs_f32(bits, vals, b, e)
    rk, rv = oracle.sort_f32(bits.view(np.float32), vals, b, e)
    assert np.array_equal(v, rv)
    assert np.array_equal(k.view(np.uint32), rk.view(np.uint32))


def test_pairs_f32_specials_ladder():
    ladder = np.array(pins.FLOAT_LADDER, np.uint32)
    keys = np.tile(ladder, 2000)
    keys = keys[rng(5).permutation(keys.size)]
    vals = np.arange(keys.size, dtype=np.uint32)
    k, v = gpu_sort_pairs_f32(keys, vals)
    rk, rv = oracle.sort_f32(keys.view(np.float32), vals)
    assert np.array_equal(v, rv) and np.array_equal(k.view(np.uint32), rk.view(np.uint32))


@pytest.mark.parametrize("n", [1, 3, 4, 5, 63, 64, 65, 1000, CTILE - 1, CTILE, CTILE + 1,
                               3 * CTILE + 5, (1 << 20) + 3])
def test_compaction_sizes(n):
    print("compact n=%d" % n, flush=True)
    x = workloads.signed_mix_f32(n, seed=n)
    o, c = gpu_compact(x)
    ro, rc = oracle.compact_positive_f32(x)
    assert c == rc
    assert np.array_equal(o.view(np.uint32), ro.view(np.uint32))


@pytest.mark.parametrize("kind", ["all_positive", "none_positive", "specials", "zeros"])
def test_compaction_cases(kind):
    n = 2 * CTILE + 77
    r = rng(21)
    if kind == "all_positive":
        x = np.abs(r.standard_normal(n).astype(np.float32)) + np.float32(0.5)
    elif kind == "none_positive":
        x = -np.abs(r.standard_normal(n).astype(np.float32))
    elif kind == "zeros":
        x = np.zeros(n, np.float32)
        x[::3] = np.float32(-0.0)
    else:
        x = np.array(pins.FLOAT_LADDER * (n // len(pins.FLOAT_LADDER) + 1), np.uint32)[:n]
        x = x[r.permutation(n)].view(np.float32)
    o, c = gpu_compact(x)
    ro, rc = oracle.compact_positive_f32(x)
    assert c == rc
    assert np.array_equal(o.view(np.uint32), ro.view(np.uint32))


@pytest.mark.parametrize("tile", [1, 2, 3, 64, 100, 255, 512, 1000, 1024])
@pytest.mark.parametrize("n", [1, 1023, 1024, 1025, 5000])
def test_bitonic_tiles(tile, n):
    keys = rng(tile + n).integers(0, 2**32, n, dtype=np.uint32)
    keys[::7] = np.uint32(0xFFFFFFFF)
    assert np.array_equal(gpu_bitonic(keys, tile), oracle.bitonic_tile(keys, tile))


@pytest.mark.parametrize("b,e", [(0, 8), (4, 13), (24, 32), (5, 5)])
def test_bitonic_bit_ranges(b, e):
    keys = rng(b + e).integers(0, 2**32, 4000, dtype=np.uint32)
    assert np.array_equal(gpu_bitonic(keys, 1000, b, e), oracle.bitonic_tile(keys, 1000, b, e))


@pytest.mark.parametrize("n", [4 * TILE + 99, LARGE + 99, PLARGE + 99])
def test_back_to_back_calls_share_temp(n):
    """Stale counters or tile states from an earlier call must not leak."""
    print("back-to-back n=%d" % n, flush=True)
    need = 0
    import sorting_lsd_radix_amd as rs
    need = rs.rs_sort_pairs_u32(None, None, None, None, n, 0, 32, None, 0)
    temp = temp_for(need)
    for seed in range(4):
        keys = rng(100 + seed).integers(0, 2**(8 * (seed + 1)) if seed < 3 else 2**32, n,
                                         dtype=np.uint64).astype(np.uint32)
        vals = np.arange(n, dtype=np.uint32)
        k, v = gpu_sort_pairs_u32(keys, vals, 0, 32, temp=temp)
        rk, rv = oracle.sort_u32(keys, vals)
        assert np.array_equal(k, rk) and np.array_equal(v, rv), seed
        o, c = gpu_compact(workloads.signed_mix_f32(n, seed=seed), temp=temp)
        ro, rc = oracle.compact_positive_f32(workloads.signed_mix_f32(n, seed=seed))
        assert c == rc and np.array_equal(o.view(np.uint32), ro.view(np.uint32))


# --- the named workloads, at their full sizes ------------------------------------------

def test_workload_tile_1024_keys():
    """1024 uniform keys: both the bitonic tile and the 4-pass radix sort (in one workgroup)."""
    keys = workloads.tile_keys()
    ref = oracle.sort_u32(keys)
    assert np.array_equal(gpu_bitonic(keys, 1024), ref)
    assert np.array_equal(oracle.bitonic_tile(keys, 1024), ref)
    assert np.array_equal(gpu_sort_keys_u32(keys), ref)


def test_workload_pairs_2p20():
    keys, vals = workloads.pairs_small()
    k, v = gpu_sort_pairs_u32(keys, vals)
    rk, rv = oracle.sort_u32(keys, vals)
    assert np.array_equal(k, rk) and np.array_equal(v, rv)


def test_workload_zipf_2p26_bits_0_16():
    print("zipf 2^26 generate", flush=True)
    keys, vals = workloads.pairs_zipf()
    k, v = gpu_sort_pairs_u32(keys, vals, 0, 16)
    print("zipf 2^26 oracle", flush=True)
    rk, rv = oracle.sort_u32(keys, vals, 0, 16)
    assert np.array_equal(k, rk) and np.array_equal(v, rv)


def test_workload_compaction_2p28():
    print("compaction 2^28 generate", flush=True)
    x = workloads.compact_input()
    o, c = gpu_compact(x)
    assert c == workloads.signed_mix_expected_count(x.size) == 120_795_955
    ro, rc = oracle.compact_positive_f32(x)
    assert c == rc
    assert np.array_equal(o.view(np.uint32), ro.view(np.uint32))


def check_stable_sort_by_order(keys_bits_in, order_out, keys_out_bits, vals_out):
    """Properties that pin a stable sort uniquely, given the sort order of the output."""
    n = keys_bits_in.size
    seen = np.zeros(n, np.uint8)
    seen[vals_out] = 1
    assert seen.all(), "values are not a permutation"
    del seen
    assert np.array_equal(keys_out_bits, keys_bits_in[vals_out]), "key/value association"
    d = order_out[1:] >= order_out[:-1]
    assert d.all(), "not sorted"
    eq = order_out[1:] == order_out[:-1]
    assert (vals_out[1:][eq] > vals_out[:-1][eq]).all(), "not stable"


def test_workload_float_pairs_2p28():
    print("float pairs 2^28 generate", flush=True)
    keys, vals = workloads.float_pairs()
    bits = keys.view(np.uint32)
    k, v = gpu_sort_pairs_f32(bits, vals)
    kb = k.view(np.uint32)
    print("float pairs 2^28 check", flush=True)
    check_stable_sort_by_order(bits, oracle.f32_to_order(kb), kb, v)
    # the four injected specials sit in order: -1e-38 < -0.0 < +0.0 < +1e-38
    m = keys.size // 256
    for pattern in (workloads.SUBNORMAL_NEG_BITS, 0x80000000, 0x00000000,
                    workloads.SUBNORMAL_POS_BITS):
        assert int((kb == np.uint32(pattern)).sum()) >= m
    print("float pairs 2^28 oracle", flush=True)
    rk, rv = oracle.sort_f32(keys, vals)
    assert np.array_equal(v, rv), "values differ from the oracle"
    assert np.array_equal(kb, rk.view(np.uint32)), "keys differ from the oracle"


def test_workload_headline_pairs_and_keys_2p28():
    """2^28 uniform pairs and the keys-only sort of the same keys, both
    compared element by element with the oracle."""
    print("headline 2^28 generate", flush=True)
    keys, vals = workloads.headline_pairs()
    k, v = gpu_sort_pairs_u32(keys, vals)
    print("headline 2^28 check", flush=True)
    check_stable_sort_by_order(keys, k, k, v)
    print("headline 2^28 oracle (pairs)", flush=True)
    rk, rv = oracle.sort_u32(keys, vals)
    assert np.array_equal(v, rv), "values differ from the oracle"
    assert np.array_equal(k, rk), "keys differ from the oracle"
    del v, rv, k
    print("headline 2^28 keys only", flush=True)
    ko = gpu_sort_keys_u32(keys)
    print("headline 2^28 oracle (keys)", flush=True)
    assert np.array_equal(ko, oracle.sort_u32(keys)), "keys-only sort differs from the oracle"
    assert np.array_equal(ko, rk)
