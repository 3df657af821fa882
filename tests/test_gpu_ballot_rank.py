"""Parity of the build with the ballot rank forced on every path.

The default library ranks keys with LDS atomic adds whose same-address lanes
gfx950 serves in lane order (observed behaviour, checked by
test_gpu_hw_probe.py).  librs_ballot.so is the same source built with
RS_FORCE_BALLOT_RANK: every one-sweep tile and the one-workgroup sort then
rank with eight ballots and mbcnt, which is stable by construction.  This
runs a parity subset that reaches every pass shape and the tile sort through
that build, bit for bit against the oracle.
"""
import os

import numpy as np
import pytest

import oracle
import pins
import sorting_lsd_radix_amd as rs
from sorting_lsd_radix_amd import build as rs_build
from gpu_helpers import gpu_sort_keys_u32, gpu_sort_pairs_f32, gpu_sort_pairs_u32
from test_gpu_parity import HLARGE, HTILE, KLARGE, LARGE, PLARGE, TILE, dist_keys

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def ballot_library():
    assert os.path.exists(rs_build.BALLOT_LIB_PATH), "build librs_ballot.so first"
    prev = rs.use_library(rs_build.BALLOT_LIB_PATH)
    yield
    rs.use_library(prev)


def rng(seed):
    return np.random.default_rng(seed)


@pytest.mark.parametrize("n", [1000, 4097, TILE, 3 * TILE + 17, LARGE + 17, PLARGE + 17,
                               HLARGE + 3 * HTILE + 17])
@pytest.mark.parametrize("b,e", [(0, 32), (4, 13)])
def test_ballot_pairs_u32(n, b, e):
    print("ballot build: pairs u32 n=%d bits=[%d,%d)" % (n, b, e), flush=True)
    keys = rng(n + b).integers(0, 2**32, n, dtype=np.uint32)
    vals = np.arange(n, dtype=np.uint32)
    k, v = gpu_sort_pairs_u32(keys, vals, b, e)
    rk, rv = oracle.sort_u32(keys, vals, b, e)
    assert np.array_equal(v, rv) and np.array_equal(k, rk)


@pytest.mark.parametrize("n", [1000, TILE + 1, KLARGE + 17, (1 << 27) + 3 * 32768 + 17])
def test_ballot_keys_u32(n):
    print("ballot build: keys u32 n=%d" % n, flush=True)
    keys = rng(n).integers(0, 2**32, n, dtype=np.uint32)
    keys[: n // 3] &= np.uint32(0xFF0F0F0F)
    for (b, e) in [(0, 32), (3, 29)]:
        assert np.array_equal(gpu_sort_keys_u32(keys, b, e), oracle.sort_u32(keys, None, b, e))


@pytest.mark.parametrize("n", [100000, PLARGE + 1234])
@pytest.mark.parametrize("kind", ["card24", "zipf", "all_equal", "few_values"])
def test_ballot_distributions(kind, n):
    print("ballot build: pairs distribution=%s n=%d" % (kind, n), flush=True)
    keys = dist_keys(kind, n)
    vals = np.arange(n, dtype=np.uint32)
    k, v = gpu_sort_pairs_u32(keys, vals)
    rk, rv = oracle.sort_u32(keys, vals)
    assert np.array_equal(v, rv) and np.array_equal(k, rk)


@pytest.mark.parametrize("n", [777, LARGE + 17])
def test_ballot_pairs_f32(n):
    print("ballot build: pairs f32 n=%d" % n, flush=True)
    bits = pins.random_float_patterns(rng(n), n)
    vals = np.arange(n, dtype=np.uint32)
    k, v = gpu_sort_pairs_f32(bits, vals)
    rk, rv = oracle.sort_f32(bits.view(np.float32), vals)
    assert np.array_equal(v, rv) and np.array_equal(k.view(np.uint32), rk.view(np.uint32))
