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


_TORCH_OF = {np.uint32: torch.uint32, np.int32: torch.int32, np.float32: torch.float32,
             np.uint64: torch.uint64, np.int64: torch.int64, np.float64: torch.float64}
_KEY_TYPE = {np.uint32: rs.RS_KEY_U32, np.int32: rs.RS_KEY_I32, np.float32: rs.RS_KEY_F32,
             np.uint64: rs.RS_KEY_U64, np.int64: rs.RS_KEY_I64, np.float64: rs.RS_KEY_F64}


def _raw(a):
    """Bit patterns of a typed array (unsigned view of the same width)."""
    return a.view(np.uint32 if a.dtype.itemsize == 4 else np.uint64)


def poisoned_like(keys):
    """A device array of the keys' type filled with 0xDE bytes."""
    t = torch.full((max(keys.size, 0) * keys.dtype.itemsize,), 0xDE, dtype=torch.uint8, device=DEV)
    return t.view(_TORCH_OF[keys.dtype.type])


def gpu_sort_typed(keys, vals=None, descending=False, b=0, e=None, temp=None):
    """rs_sort_keys / rs_sort_pairs on a typed numpy array; returns keys or (keys, vals)."""
    n = keys.size
    kt = _KEY_TYPE[keys.dtype.type]
    e = keys.dtype.itemsize * 8 if e is None else e
    tk = to_dev(keys)
    ko = poisoned_like(keys)
    if vals is None:
        need = rs.rs_sort_keys(kt, descending, None, None, n, b, e, None, 0)
        temp = temp_for(need) if temp is None else temp
        rs.rs_sort_keys(kt, descending, tk, ko, n, b, e, temp, temp.numel())
        k = host(ko)
        assert np.array_equal(_raw(host(tk)), _raw(keys)), "input modified"
        return k
    tv = to_dev(vals)
    vo = poisoned(n)
    need = rs.rs_sort_pairs(kt, descending, None, None, None, None, n, b, e, None, 0)
    temp = temp_for(need) if temp is None else temp
    rs.rs_sort_pairs(kt, descending, tk, ko, tv, vo, n, b, e, temp, temp.numel())
    k, v = host(ko), host(vo)
    assert np.array_equal(_raw(host(tk)), _raw(keys)) and np.array_equal(host(tv), vals), \
        "input modified"
    return k, v


def gpu_sort_two_keys(major, minor, vals=None, temp=None):
    """rs_sort_two_keys_u32; returns (major, minor) or (major, minor, vals)."""
    n = major.size
    tm, tn = to_dev(major), to_dev(minor)
    mo, no = poisoned(n), poisoned(n)
    tv = to_dev(vals) if vals is not None else None
    vo = poisoned(n) if vals is not None else None
    need = rs.rs_sort_two_keys_u32(None, None, None, None, None, None, n, None, 0)
    temp = temp_for(need) if temp is None else temp
    rs.rs_sort_two_keys_u32(tm, tn, mo, no, tv, vo, n, temp, temp.numel())
    out = (host(mo), host(no)) if vals is None else (host(mo), host(no), host(vo))
    assert np.array_equal(host(tm), major) and np.array_equal(host(tn), minor), "input modified"
    return out


def gpu_digit_counts(keys, descending=False, b=0, e=None):
    """rs_digit_counts on a typed numpy array: uint32 [passes, 256]."""
    kt = _KEY_TYPE[keys.dtype.type]
    e = keys.dtype.itemsize * 8 if e is None else e
    passes = (e - b + 7) // 8
    tk = to_dev(keys)
    counts = poisoned(max(passes, 1) * 256)
    rs.rs_digit_counts(kt, descending, tk, keys.size, b, e, counts)
    return host(counts)[: passes * 256].reshape(passes, 256)


def gpu_scan(x, inclusive=False, inplace=False):
    """rs_exclusive_scan_u32 / rs_inclusive_scan_u32 through the C ABI."""
    n = x.size
    fn = rs.rs_inclusive_scan_u32 if inclusive else rs.rs_exclusive_scan_u32
    tx = to_dev(x)
    out = tx if inplace else poisoned(n)
    need = fn(None, None, n, None, 0)
    temp = temp_for(need)
    fn(tx, out, n, temp, temp.numel())
    o = host(out)
    if not inplace:
        assert np.array_equal(host(tx), x), "input modified"
    return o


def gpu_select(x, op, threshold, vals=None, partition=False):
    """rs_select / rs_partition through the C ABI; returns (out, vals_out or None, count).
    Without partition only out[:count] is defined (the rest keeps the poison)."""
    n = x.size
    kt = _KEY_TYPE[x.dtype.type]
    bits = int(np.array([threshold], x.dtype).view(np.uint32)[0])
    fn = rs.rs_partition if partition else rs.rs_select
    tx = to_dev(x)
    out = poisoned_like(x)
    tv = to_dev(vals) if vals is not None else None
    vo = poisoned(n) if vals is not None else None
    cnt = poisoned(1)
    need = fn(kt, rs._OPS[op], bits, None, None, tv, vo, None, n, None, 0)
    temp = temp_for(need)
    fn(kt, rs._OPS[op], bits, tx, out, tv, vo, cnt, n, temp, temp.numel())
    o, c = host(out), int(host(cnt)[0])
    v = host(vo) if vals is not None else None
    assert np.array_equal(_raw(host(tx)), _raw(x)), "input modified"
    return o, v, c
