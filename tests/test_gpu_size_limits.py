"""The top of the accepted size range, on the GPU, element by element.

n = 2^30 - 1 is the largest size the library accepts.  For pair sorts the
last 28672-key tile then reaches past 2^30 keys, where a pad's byte offset
would wrap round 2^32 unless clamped; n = 2^29 + 2^20 + 17 makes every
entry point address bytes past 2^31 (signed 32-bit overflow of a byte
offset) with a ragged last tile.  Every output is compared with the oracle
bit for bit.  These runs use up to ~24 GiB of device memory and ~40 GiB of
host memory.
"""
import gc

import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_helpers import (gpu_bitonic, gpu_compact, gpu_sort_keys_u32, gpu_sort_pairs_f32,
                         gpu_sort_pairs_u32)

pytestmark = pytest.mark.gpu

N_MAX = (1 << 30) - 1
N_MID = (1 << 29) + (1 << 20) + 17


def release():
    gc.collect()
    torch.cuda.empty_cache()


def say(msg):
    print(msg, flush=True)


@pytest.mark.parametrize("n", [N_MAX, N_MID])
def test_pairs_u32_at_size_limit(n):
    say("pairs u32 n=%d: generate" % n)
    keys = workloads.uniform_u32(n, seed=31)
    vals = workloads.index_values(n)
    say("pairs u32 n=%d: gpu" % n)
    k, v = gpu_sort_pairs_u32(keys, vals)
    release()
    say("pairs u32 n=%d: oracle" % n)
    rk, rv = oracle.sort_u32(keys, vals)
    del keys, vals
    assert np.array_equal(v, rv), "values"
    assert np.array_equal(k, rk), "keys"


@pytest.mark.parametrize("n", [N_MAX, N_MID])
def test_keys_u32_at_size_limit(n):
    say("keys u32 n=%d: generate" % n)
    keys = workloads.uniform_u32(n, seed=32)
    say("keys u32 n=%d: gpu" % n)
    k = gpu_sort_keys_u32(keys)
    release()
    say("keys u32 n=%d: oracle" % n)
    assert np.array_equal(k, oracle.sort_u32(keys))


@pytest.mark.parametrize("n", [N_MAX, N_MID])
def test_pairs_f32_at_size_limit(n):
    say("pairs f32 n=%d: generate" % n)
    keys = workloads.normal_specials_f32(n, seed=33)
    vals = workloads.index_values(n)
    say("pairs f32 n=%d: gpu" % n)
    k, v = gpu_sort_pairs_f32(keys.view(np.uint32), vals)
    release()
    say("pairs f32 n=%d: oracle" % n)
    rk, rv = oracle.sort_f32(keys, vals)
    del keys, vals
    assert np.array_equal(v, rv), "values"
    assert np.array_equal(k.view(np.uint32), rk.view(np.uint32)), "keys"


def test_compaction_past_2p31_bytes():
    n = N_MID
    say("compaction n=%d: generate" % n)
    x = workloads.signed_mix_f32(n, seed=34)
    say("compaction n=%d: gpu" % n)
    o, c = gpu_compact(x)
    release()
    say("compaction n=%d: oracle" % n)
    ro, rc = oracle.compact_positive_f32(x)
    assert c == rc
    assert np.array_equal(o.view(np.uint32), ro.view(np.uint32))


def test_bitonic_tiles_past_2p31_bytes():
    n = N_MID
    say("bitonic tiles n=%d: generate" % n)
    keys = workloads.uniform_u32(n, seed=35)
    say("bitonic tiles n=%d: gpu" % n)
    k = gpu_bitonic(keys, 1000)
    release()
    say("bitonic tiles n=%d: oracle" % n)
    assert np.array_equal(k, oracle.bitonic_tile(keys, 1000))
