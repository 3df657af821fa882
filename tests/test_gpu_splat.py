"""Tile/depth keys of a splat renderer through the 64-bit sort (synthetic only).

Each splat emits one entry per screen tile its bounding square touches:
key = tile id * 2^32 + depth bits, value = splat index (workloads.splat_pairs).
Sorting the keys on bits [0, 32 + tile bits) groups the entries by tile and
orders each tile's entries by depth, stably.  The output is compared with
the oracle element by element, and each tile's run is checked to be the
tile's entries in depth order.
"""
import numpy as np
import pytest

import oracle
import workloads
from gpu_helpers import gpu_sort_typed

pytestmark = pytest.mark.gpu

END_BIT = 32 + workloads.SPLAT_TILE_BITS


@pytest.mark.parametrize("gaussians", [1, 1000, 1 << 16, 1 << 20])
def test_splat_keys(gaussians):
    print("splat keys: %d splats" % gaussians, flush=True)
    keys, vals = workloads.splat_pairs(gaussians, seed=gaussians)
    k, v = gpu_sort_typed(keys, vals, False, 0, END_BIT)
    rk, rv = oracle.sort_typed(keys, vals, 0, END_BIT)
    assert np.array_equal(k, rk) and np.array_equal(v, rv)
    tile = (k >> np.uint64(32)).astype(np.int64)
    assert np.all(np.diff(tile) >= 0)
    same = tile[1:] == tile[:-1]
    depth = (k & np.uint64(0xFFFFFFFF)).astype(np.uint32).view(np.float32)
    assert np.all(depth[1:][same] >= depth[:-1][same])
