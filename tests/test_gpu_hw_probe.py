"""GPU check of the hardware property the stable rank of the sort relies on.

Every one-sweep pass kernel (keys only and key-value, every tile shape and
key type, the hybrid sort's top-digit pass and its multi-pass fallback
included) ranks a key with one LDS atomic add (`ds_add_rtn_u32`) on its
wave's digit counter while the digits of the pass are spread out, and the
one-workgroup sort of up to 16384 keys and the hybrid sort's per-bucket sort
always do.  That rank is the stable
one only if the lanes of one instruction that hit the same counter are
served in lane order: observed gfx950 behaviour, not a documented guarantee.
This test runs a probe kernel (tests/hw_probe/lds_lane_order.hip) that
compares every atomic result with the lane-order rank, for uniform,
clustered, all-equal, skewed and same-bank digit patterns.  The library can
be built with the ballot rank forced on every path (RS_FORCE_BALLOT_RANK),
which does not depend on this property.
"""
import ctypes
import os

import pytest

pytestmark = pytest.mark.gpu

LIB = os.path.join(os.path.dirname(os.path.abspath(__file__)), "hw_probe", "liblds_probe.so")
MODES = {0: "uniform", 1: "8 values", 2: "all equal", 3: "80% one digit", 4: "same-bank digits"}


@pytest.mark.parametrize("mode", sorted(MODES))
def test_lds_atomic_add_serves_lanes_in_order(mode):
    assert os.path.exists(LIB), "build the probe first (__graft_entry__.build())"
    lib = ctypes.CDLL(LIB)
    lib.probe_lds_lane_order.restype = ctypes.c_longlong
    lib.probe_lds_lane_order.argtypes = [ctypes.c_int] * 4
    print("lds lane-order probe mode=%d (%s)" % (mode, MODES[mode]), flush=True)
    bad = lib.probe_lds_lane_order(mode, 4, 512, 64)
    assert bad == 0, "%d lanes out of lane order (mode %s)" % (bad, MODES[mode])
