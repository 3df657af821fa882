"""Shared helpers of the GPU parity tests: device transfer and call wrappers.

Every call goes through the C ABI via the package's ``rs_*`` bindings with
explicitly allocated outputs that are pre-filled with 0xDEADBEEF, so a
missed output element shows up as a mismatch.  Inputs are re-read after the
call to check that the library left them untouched.
"""
import numpy as np
import torch

import sorting_lsd_radix_amd as rs

POISON = -559038737  # 0xDEADBEEF as int32
DEV = torch.device("cuda:0")


def to_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def poisoned(n, dtype=torch.uint32):
    t = torch.full((max(n, 0),), POISON, dtype=torch.int32, device=DEV)
    return t.view(dtype)


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def temp_for(nbytes):
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=DEV)


def gpu_sort_pairs_u32(keys, vals, b=0, e=32, temp=None):
    n = keys.size
    tk, tv = to_dev(keys), to_dev(vals)
    ko, vo = poisoned(n), poisoned(n)
    need = rs.rs_sort_pairs_u32(None, None, None, None, n, b, e, None, 0)
    temp = temp_for(need) if temp is None else temp
    rs.rs_sort_pairs_u32(tk, ko, tv, vo, n, b, e, temp, temp.numel())
    k, v = host(ko), host(vo)
    assert np.array_equal(host(tk), keys) and np.array_equal(host(tv), vals), "input modified"
    return k, v


def gpu_sort_keys_u32(keys, b=0, e=32, temp=None):
    n = keys.size
    tk = to_dev(keys)
    ko = poisoned(n)
    need = rs.rs_sort_keys_u32(None, None, n, b, e, None, 0)
    temp = temp_for(need) if temp is None else temp
    rs.rs_sort_keys_u32(tk, ko, n, b, e, temp, temp.numel())
    k = host(ko)
    assert np.array_equal(host(tk), keys), "input modified"
    return k


def gpu_sort_pairs_f32(keys, vals, b=0, e=32, temp=None):
    n = keys.size
    tk, tv = to_dev(keys.view(np.float32)), to_dev(vals)
    ko, vo = poisoned(n, torch.float32), poisoned(n)
    need = rs.rs_sort_pairs_f32(None, None, None, None, n, b, e, None, 0)
    temp = temp_for(need) if temp is None else temp
    rs.rs_sort_pairs_f32(tk, ko, tv, vo, n, b, e, temp, temp.numel())
    k, v = host(ko), host(vo)
    assert np.array_equal(host(tk).view(np.uint32), keys.view(np.uint32)), "input modified"
    return k, v


def gpu_compact(x, temp=None):
    n = x.size
    tx = to_dev(x)
    out = poisoned(n, torch.float32)
    cnt = poisoned(1)
    need = rs.rs_compact_positive_f32(None, None, None, n, None, 0)
    temp = temp_for(need) if temp is None else temp
    rs.rs_compact_positive_f32(tx, out, cnt, n, temp, temp.numel())
    o, c = host(out), int(host(cnt)[0])
    assert np.array_equal(host(tx).view(np.uint32), x.view(np.uint32)), "input modified"
    return o, c


def gpu_bitonic(keys, tile, b=0, e=32):
    n = keys.size
    tk = to_dev(keys)
    ko = poisoned(n)
    rs.rs_bitonic_tile(tk, ko, n, tile, b, e)
    k = host(ko)
    assert np.array_equal(host(tk), keys), "input modified"
    return k
