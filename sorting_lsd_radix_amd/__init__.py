"""Python binding of the gfx950 stable LSD radix sort library (``librs.so``).

The functions named ``rs_*`` mirror the C ABI in ``include/rs.h`` one for one:
they only turn tensors or integers into device pointers and sizes, call the
library and raise :class:`RsError` on a status other than ``RS_OK``.  Every
step of the computation runs in the library's HIP kernels.  The convenience
wrappers below them (``sort_keys_u32`` ...) allocate outputs and temporary
storage with torch on the tensors' device and launch on torch's current
stream; torch provides memory and streams only.

Loading fails with an error when ``librs.so`` has not been built; there is no
fallback implementation.  ``use_library(path)`` binds the functions to another
build of the same sources (the tests use it for the build with the ballot rank
forced on every path, ``librs_ballot.so``).
"""
import ctypes
import os

__all__ = [
    "RsError", "RS_OK", "RS_ERR_INVALID_VALUE", "RS_ERR_UNSUPPORTED_SIZE",
    "RS_ERR_TEMP_TOO_SMALL", "RS_ERR_OVERLAP", "RS_ERR_MISALIGNED", "RS_ERR_HIP",
    "RS_KEY_U32", "RS_KEY_I32", "RS_KEY_F32", "RS_KEY_U64", "RS_KEY_I64", "RS_KEY_F64",
    "rs_sort_keys_u32", "rs_sort_pairs_u32", "rs_sort_pairs_f32", "rs_sort_keys", "rs_sort_pairs",
    "rs_sort_two_keys_u32", "rs_digit_counts", "rs_compact_positive_f32",
    "rs_compact_positive_f32_noalloc", "rs_exclusive_scan_u32", "rs_inclusive_scan_u32",
    "rs_select", "rs_partition", "RS_OP_LT", "RS_OP_LE", "RS_OP_GT", "RS_OP_GE", "RS_OP_EQ",
    "RS_OP_NE", "rs_bitonic_tile", "rs_status_string", "rs_timing_enable", "rs_timing_collect",
    "exclusive_scan_u32", "inclusive_scan_u32", "select", "partition",
    "sort_keys_u32", "sort_pairs_u32", "sort_pairs_f32", "sort_keys", "sort_pairs",
    "sort_two_keys_u32", "digit_counts", "compact_positive_f32", "bitonic_tile",
    "library_path", "use_library", "EXPORTED_SYMBOLS", "KERNEL_NAMES",
]

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_PKG, "librs.so")

RS_OK = 0
RS_ERR_INVALID_VALUE = 1
RS_ERR_UNSUPPORTED_SIZE = 2
RS_ERR_TEMP_TOO_SMALL = 3
RS_ERR_OVERLAP = 4
RS_ERR_MISALIGNED = 5
RS_ERR_HIP = 6

RS_KEY_U32 = 0
RS_KEY_I32 = 1
RS_KEY_F32 = 2
RS_KEY_U64 = 3
RS_KEY_I64 = 4
RS_KEY_F64 = 5

RS_KERNEL_UPSWEEP = 0
RS_KERNEL_ONESWEEP = 1
RS_KERNEL_SORT_INIT = 2
RS_KERNEL_COMPACT_INIT = 3
RS_KERNEL_COMPACT = 4
RS_KERNEL_BITONIC = 5
RS_KERNEL_COPY = 6
RS_KERNEL_TILE_SORT = 7
RS_KERNEL_BUCKET_SORT = 8
KERNEL_NAMES = {0: "upsweep", 1: "onesweep", 2: "sort_init", 3: "compact_init",
                4: "compact", 5: "bitonic", 6: "copy", 7: "tile_sort", 8: "bucket_sort",
                9: "scan_init", 10: "scan", 11: "select_init", 12: "select_count", 13: "select"}

RS_OP_LT, RS_OP_LE, RS_OP_GT, RS_OP_GE, RS_OP_EQ, RS_OP_NE = range(6)
_OPS = {"<": RS_OP_LT, "<=": RS_OP_LE, ">": RS_OP_GT, ">=": RS_OP_GE, "==": RS_OP_EQ,
        "!=": RS_OP_NE}

EXPORTED_SYMBOLS = ["rs_sort_keys_u32", "rs_sort_pairs_u32", "rs_sort_pairs_f32",
                    "rs_sort_keys", "rs_sort_pairs", "rs_sort_two_keys_u32", "rs_digit_counts",
                    "rs_compact_positive_f32", "rs_compact_positive_f32_noalloc",
                    "rs_exclusive_scan_u32", "rs_inclusive_scan_u32", "rs_select", "rs_partition",
                    "rs_bitonic_tile", "rs_status_string",
                    "rs_timing_enable", "rs_timing_collect"]

_lib = None
_lib_path = _LIB_PATH


class RsError(RuntimeError):
    def __init__(self, status, what):
        self.status = status
        super().__init__("%s: %s" % (what, rs_status_string(status)))


def library_path():
    return _lib_path


def use_library(path=None):
    """Bind every function to the library at `path` (None: the default
    librs.so); returns the previous path."""
    global _lib, _lib_path
    prev = _lib_path
    _lib_path = _LIB_PATH if path is None else os.path.abspath(path)
    _lib = None
    return prev


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_lib_path):
        raise RuntimeError("%s is not built; run "
                           "`python -m sorting_lsd_radix_amd.build` or "
                           "`python -c 'import __graft_entry__ as g; g.build()'`" % _lib_path)
    lib = ctypes.CDLL(_lib_path)
    vp, u64, i32, u32 = ctypes.c_void_p, ctypes.c_uint64, ctypes.c_int, ctypes.c_uint32
    szp = ctypes.POINTER(ctypes.c_size_t)
    lib.rs_sort_keys_u32.argtypes = [vp, vp, u64, i32, i32, vp, szp, vp]
    lib.rs_sort_pairs_u32.argtypes = [vp, vp, vp, vp, u64, i32, i32, vp, szp, vp]
    lib.rs_sort_pairs_f32.argtypes = [vp, vp, vp, vp, u64, i32, i32, vp, szp, vp]
    lib.rs_sort_keys.argtypes = [i32, i32, vp, vp, u64, i32, i32, vp, szp, vp]
    lib.rs_sort_pairs.argtypes = [i32, i32, vp, vp, vp, vp, u64, i32, i32, vp, szp, vp]
    lib.rs_sort_two_keys_u32.argtypes = [vp, vp, vp, vp, vp, vp, u64, vp, szp, vp]
    lib.rs_digit_counts.argtypes = [i32, i32, vp, u64, i32, i32, vp, vp]
    lib.rs_compact_positive_f32.argtypes = [vp, vp, vp, u64, vp, szp, vp]
    lib.rs_compact_positive_f32_noalloc.argtypes = [vp, vp, vp, u64, vp]
    lib.rs_compact_positive_f32_noalloc.restype = i32
    for f in (lib.rs_exclusive_scan_u32, lib.rs_inclusive_scan_u32):
        f.argtypes = [vp, vp, u64, vp, szp, vp]
        f.restype = i32
    for f in (lib.rs_select, lib.rs_partition):
        f.argtypes = [i32, i32, u32, vp, vp, vp, vp, vp, u64, vp, szp, vp]
        f.restype = i32
    lib.rs_bitonic_tile.argtypes = [vp, vp, u64, u32, i32, i32, vp]
    for f in (lib.rs_sort_keys_u32, lib.rs_sort_pairs_u32, lib.rs_sort_pairs_f32, lib.rs_sort_keys,
              lib.rs_sort_pairs, lib.rs_sort_two_keys_u32, lib.rs_digit_counts,
              lib.rs_compact_positive_f32, lib.rs_bitonic_tile):
        f.restype = i32
    lib.rs_status_string.argtypes = [i32]
    lib.rs_status_string.restype = ctypes.c_char_p
    lib.rs_timing_enable.argtypes = [i32]
    lib.rs_timing_enable.restype = i32
    lib.rs_timing_collect.argtypes = [ctypes.POINTER(ctypes.c_int), ctypes.POINTER(ctypes.c_float),
                                      i32]
    lib.rs_timing_collect.restype = i32
    _lib = lib
    return lib


# --- argument marshalling ------------------------------------------------------------

def _ptr(x):
    """Device pointer of a tensor, or an integer address, or None."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _call(what, status):
    if status != RS_OK:
        raise RsError(status, what)


def rs_status_string(status):
    return _load().rs_status_string(int(status)).decode()


def _sort_call(fn, what, args, n, begin_bit, end_bit, d_temp, temp_bytes, stream):
    size = ctypes.c_size_t(0 if temp_bytes is None else int(temp_bytes))
    st = fn(*[_ptr(a) for a in args], int(n), int(begin_bit), int(end_bit), _ptr(d_temp),
            ctypes.byref(size), _stream(stream) if d_temp is not None else None)
    _call(what, st)
    return size.value if d_temp is None else None


def rs_sort_keys_u32(keys_in, keys_out, n, begin_bit, end_bit, d_temp, temp_bytes, stream=None):
    """C: rs_sort_keys_u32.  With d_temp None, returns the temp size."""
    return _sort_call(_load().rs_sort_keys_u32, "rs_sort_keys_u32", (keys_in, keys_out), n,
                      begin_bit, end_bit, d_temp, temp_bytes, stream)


def rs_sort_pairs_u32(keys_in, keys_out, vals_in, vals_out, n, begin_bit, end_bit, d_temp,
                      temp_bytes, stream=None):
    """C: rs_sort_pairs_u32.  With d_temp None, returns the temp size."""
    return _sort_call(_load().rs_sort_pairs_u32, "rs_sort_pairs_u32",
                      (keys_in, keys_out, vals_in, vals_out), n, begin_bit, end_bit, d_temp,
                      temp_bytes, stream)


def rs_sort_pairs_f32(keys_in, keys_out, vals_in, vals_out, n, begin_bit, end_bit, d_temp,
                      temp_bytes, stream=None):
    """C: rs_sort_pairs_f32.  With d_temp None, returns the temp size."""
    return _sort_call(_load().rs_sort_pairs_f32, "rs_sort_pairs_f32",
                      (keys_in, keys_out, vals_in, vals_out), n, begin_bit, end_bit, d_temp,
                      temp_bytes, stream)


def rs_sort_keys(key_type, descending, keys_in, keys_out, n, begin_bit, end_bit, d_temp,
                 temp_bytes, stream=None):
    """C: rs_sort_keys.  With d_temp None, returns the temp size."""
    size = ctypes.c_size_t(0 if temp_bytes is None else int(temp_bytes))
    st = _load().rs_sort_keys(int(key_type), int(bool(descending)), _ptr(keys_in), _ptr(keys_out),
                              int(n), int(begin_bit), int(end_bit), _ptr(d_temp),
                              ctypes.byref(size), _stream(stream) if d_temp is not None else None)
    _call("rs_sort_keys", st)
    return size.value if d_temp is None else None


def rs_sort_pairs(key_type, descending, keys_in, keys_out, vals_in, vals_out, n, begin_bit,
                  end_bit, d_temp, temp_bytes, stream=None):
    """C: rs_sort_pairs.  With d_temp None, returns the temp size."""
    size = ctypes.c_size_t(0 if temp_bytes is None else int(temp_bytes))
    st = _load().rs_sort_pairs(int(key_type), int(bool(descending)), _ptr(keys_in), _ptr(keys_out),
                               _ptr(vals_in), _ptr(vals_out), int(n), int(begin_bit), int(end_bit),
                               _ptr(d_temp), ctypes.byref(size),
                               _stream(stream) if d_temp is not None else None)
    _call("rs_sort_pairs", st)
    return size.value if d_temp is None else None


def rs_sort_two_keys_u32(major_in, minor_in, major_out, minor_out, vals_in, vals_out, n, d_temp,
                         temp_bytes, stream=None):
    """C: rs_sort_two_keys_u32.  With d_temp None, returns the temp size."""
    size = ctypes.c_size_t(0 if temp_bytes is None else int(temp_bytes))
    st = _load().rs_sort_two_keys_u32(_ptr(major_in), _ptr(minor_in), _ptr(major_out),
                                      _ptr(minor_out), _ptr(vals_in), _ptr(vals_out), int(n),
                                      _ptr(d_temp), ctypes.byref(size),
                                      _stream(stream) if d_temp is not None else None)
    _call("rs_sort_two_keys_u32", st)
    return size.value if d_temp is None else None


def rs_digit_counts(key_type, descending, keys, n, begin_bit, end_bit, d_counts, stream=None):
    """C: rs_digit_counts."""
    st = _load().rs_digit_counts(int(key_type), int(bool(descending)), _ptr(keys), int(n),
                                 int(begin_bit), int(end_bit), _ptr(d_counts), _stream(stream))
    _call("rs_digit_counts", st)


def rs_compact_positive_f32(x_in, x_out, d_count, n, d_temp, temp_bytes, stream=None):
    """C: rs_compact_positive_f32.  With d_temp None, returns the temp size."""
    size = ctypes.c_size_t(0 if temp_bytes is None else int(temp_bytes))
    st = _load().rs_compact_positive_f32(_ptr(x_in), _ptr(x_out), _ptr(d_count), int(n),
                                         _ptr(d_temp), ctypes.byref(size),
                                         _stream(stream) if d_temp is not None else None)
    _call("rs_compact_positive_f32", st)
    return size.value if d_temp is None else None


def rs_compact_positive_f32_noalloc(x_in, x_out, d_count, n, stream=None):
    """C: rs_compact_positive_f32_noalloc (the library's static scratch, no temp)."""
    st = _load().rs_compact_positive_f32_noalloc(_ptr(x_in), _ptr(x_out), _ptr(d_count), int(n),
                                                 _stream(stream))
    _call("rs_compact_positive_f32_noalloc", st)


def _scan_call(fn, what, x_in, x_out, n, d_temp, temp_bytes, stream):
    size = ctypes.c_size_t(0 if temp_bytes is None else int(temp_bytes))
    st = fn(_ptr(x_in), _ptr(x_out), int(n), _ptr(d_temp), ctypes.byref(size),
            _stream(stream) if d_temp is not None else None)
    _call(what, st)
    return size.value if d_temp is None else None


def rs_exclusive_scan_u32(x_in, x_out, n, d_temp, temp_bytes, stream=None):
    """C: rs_exclusive_scan_u32.  With d_temp None, returns the temp size."""
    return _scan_call(_load().rs_exclusive_scan_u32, "rs_exclusive_scan_u32", x_in, x_out, n,
                      d_temp, temp_bytes, stream)


def rs_inclusive_scan_u32(x_in, x_out, n, d_temp, temp_bytes, stream=None):
    """C: rs_inclusive_scan_u32.  With d_temp None, returns the temp size."""
    return _scan_call(_load().rs_inclusive_scan_u32, "rs_inclusive_scan_u32", x_in, x_out, n,
                      d_temp, temp_bytes, stream)


def _select_call(fn, what, key_type, op, threshold_bits, x_in, x_out, vals_in, vals_out, d_count,
                 n, d_temp, temp_bytes, stream):
    size = ctypes.c_size_t(0 if temp_bytes is None else int(temp_bytes))
    st = fn(int(key_type), int(op), int(threshold_bits) & 0xFFFFFFFF, _ptr(x_in), _ptr(x_out),
            _ptr(vals_in), _ptr(vals_out), _ptr(d_count), int(n), _ptr(d_temp), ctypes.byref(size),
            _stream(stream) if d_temp is not None else None)
    _call(what, st)
    return size.value if d_temp is None else None


def rs_select(key_type, op, threshold_bits, x_in, x_out, vals_in, vals_out, d_count, n, d_temp,
              temp_bytes, stream=None):
    """C: rs_select.  With d_temp None, returns the temp size."""
    return _select_call(_load().rs_select, "rs_select", key_type, op, threshold_bits, x_in, x_out,
                        vals_in, vals_out, d_count, n, d_temp, temp_bytes, stream)


def rs_partition(key_type, op, threshold_bits, x_in, x_out, vals_in, vals_out, d_count, n, d_temp,
                 temp_bytes, stream=None):
    """C: rs_partition.  With d_temp None, returns the temp size."""
    return _select_call(_load().rs_partition, "rs_partition", key_type, op, threshold_bits, x_in,
                        x_out, vals_in, vals_out, d_count, n, d_temp, temp_bytes, stream)


def rs_bitonic_tile(keys_in, keys_out, n, tile, begin_bit, end_bit, stream=None):
    """C: rs_bitonic_tile."""
    st = _load().rs_bitonic_tile(_ptr(keys_in), _ptr(keys_out), int(n), int(tile),
                                 int(begin_bit), int(end_bit), _stream(stream))
    _call("rs_bitonic_tile", st)


def rs_timing_enable(enable):
    _call("rs_timing_enable", _load().rs_timing_enable(1 if enable else 0))


def rs_timing_collect():
    """[(kernel name, milliseconds), ...] of the launches recorded so far."""
    lib = _load()
    held = lib.rs_timing_collect(None, None, 0)
    if held < 0:
        raise RsError(RS_ERR_HIP, "rs_timing_collect")
    ids = (ctypes.c_int * max(held, 1))()
    ms = (ctypes.c_float * max(held, 1))()
    got = lib.rs_timing_collect(ids, ms, held)
    if got < 0:
        raise RsError(RS_ERR_HIP, "rs_timing_collect")
    return [(KERNEL_NAMES.get(ids[i], str(ids[i])), float(ms[i])) for i in range(min(got, held))]


# --- convenience wrappers (torch allocates; the library computes) -------------------

def _temp(nbytes, device):
    import torch
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


def _check_tensor(t, dtype, name):
    if not t.is_cuda or t.dtype != dtype or not t.is_contiguous():
        raise TypeError("%s must be a contiguous CUDA tensor of %s" % (name, dtype))


def sort_keys_u32(keys, begin_bit=0, end_bit=32, out=None, temp=None, stream=None):
    """Stable sort of a uint32 tensor by bits [begin_bit, end_bit); returns the sorted keys."""
    import torch
    _check_tensor(keys, torch.uint32, "keys")
    n = keys.numel()
    out = torch.empty_like(keys) if out is None else out
    need = rs_sort_keys_u32(None, None, n, begin_bit, end_bit, None, 0)
    temp = _temp(need, keys.device) if temp is None else temp
    rs_sort_keys_u32(keys, out, n, begin_bit, end_bit, temp, temp.numel(), stream)
    return out


def sort_pairs_u32(keys, vals, begin_bit=0, end_bit=32, keys_out=None, vals_out=None, temp=None,
                   stream=None):
    """Stable sort of uint32 (key, value) tensors; returns (keys_out, vals_out)."""
    import torch
    _check_tensor(keys, torch.uint32, "keys")
    _check_tensor(vals, torch.uint32, "vals")
    n = keys.numel()
    keys_out = torch.empty_like(keys) if keys_out is None else keys_out
    vals_out = torch.empty_like(vals) if vals_out is None else vals_out
    need = rs_sort_pairs_u32(None, None, None, None, n, begin_bit, end_bit, None, 0)
    temp = _temp(need, keys.device) if temp is None else temp
    rs_sort_pairs_u32(keys, keys_out, vals, vals_out, n, begin_bit, end_bit, temp, temp.numel(),
                      stream)
    return keys_out, vals_out


def sort_pairs_f32(keys, vals, begin_bit=0, end_bit=32, keys_out=None, vals_out=None, temp=None,
                   stream=None):
    """Stable IEEE-total-order sort of float32 keys with uint32 values."""
    import torch
    _check_tensor(keys, torch.float32, "keys")
    _check_tensor(vals, torch.uint32, "vals")
    n = keys.numel()
    keys_out = torch.empty_like(keys) if keys_out is None else keys_out
    vals_out = torch.empty_like(vals) if vals_out is None else vals_out
    need = rs_sort_pairs_f32(None, None, None, None, n, begin_bit, end_bit, None, 0)
    temp = _temp(need, keys.device) if temp is None else temp
    rs_sort_pairs_f32(keys, keys_out, vals, vals_out, n, begin_bit, end_bit, temp, temp.numel(),
                      stream)
    return keys_out, vals_out


def _key_type(t):
    import torch
    table = {torch.uint32: RS_KEY_U32, torch.int32: RS_KEY_I32, torch.float32: RS_KEY_F32,
             torch.uint64: RS_KEY_U64, torch.int64: RS_KEY_I64, torch.float64: RS_KEY_F64}
    if not t.is_cuda or not t.is_contiguous() or t.dtype not in table:
        raise TypeError("keys must be a contiguous CUDA tensor of uint32, int32, float32, "
                        "uint64, int64 or float64")
    return table[t.dtype], t.element_size() * 8


def sort_keys(keys, descending=False, begin_bit=0, end_bit=None, out=None, temp=None, stream=None):
    """Stable sort of a typed key tensor (ascending or descending); returns the sorted keys."""
    kt, width = _key_type(keys)
    end_bit = width if end_bit is None else end_bit
    n = keys.numel()
    out = keys.new_empty(keys.shape) if out is None else out
    need = rs_sort_keys(kt, descending, None, None, n, begin_bit, end_bit, None, 0)
    temp = _temp(need, keys.device) if temp is None else temp
    rs_sort_keys(kt, descending, keys, out, n, begin_bit, end_bit, temp, temp.numel(), stream)
    return out


def sort_pairs(keys, vals, descending=False, begin_bit=0, end_bit=None, keys_out=None,
               vals_out=None, temp=None, stream=None):
    """Stable sort of typed keys with uint32 values; returns (keys_out, vals_out)."""
    import torch
    kt, width = _key_type(keys)
    _check_tensor(vals, torch.uint32, "vals")
    end_bit = width if end_bit is None else end_bit
    n = keys.numel()
    keys_out = keys.new_empty(keys.shape) if keys_out is None else keys_out
    vals_out = torch.empty_like(vals) if vals_out is None else vals_out
    need = rs_sort_pairs(kt, descending, None, None, None, None, n, begin_bit, end_bit, None, 0)
    temp = _temp(need, keys.device) if temp is None else temp
    rs_sort_pairs(kt, descending, keys, keys_out, vals, vals_out, n, begin_bit, end_bit, temp,
                  temp.numel(), stream)
    return keys_out, vals_out


def sort_two_keys_u32(major, minor, vals=None, temp=None, stream=None):
    """Stable sort by (major, minor) uint32 keys; returns (major, minor) or (major, minor, vals)."""
    import torch
    _check_tensor(major, torch.uint32, "major")
    _check_tensor(minor, torch.uint32, "minor")
    n = major.numel()
    mo, no = torch.empty_like(major), torch.empty_like(minor)
    vo = None
    if vals is not None:
        _check_tensor(vals, torch.uint32, "vals")
        vo = torch.empty_like(vals)
    need = rs_sort_two_keys_u32(None, None, None, None, None, None, n, None, 0)
    temp = _temp(need, major.device) if temp is None else temp
    rs_sort_two_keys_u32(major, minor, mo, no, vals, vo, n, temp, temp.numel(), stream)
    return (mo, no) if vals is None else (mo, no, vo)


def digit_counts(keys, descending=False, begin_bit=0, end_bit=None, stream=None):
    """Per-pass 8-bit digit counts of a typed key tensor: uint32 tensor [passes, 256]."""
    import torch
    kt, width = _key_type(keys)
    end_bit = width if end_bit is None else end_bit
    passes = (end_bit - begin_bit + 7) // 8
    counts = torch.zeros((max(passes, 1), 256), dtype=torch.uint32, device=keys.device)
    rs_digit_counts(kt, descending, keys, keys.numel(), begin_bit, end_bit, counts, stream)
    return counts[:passes]


def _scan_tensor(fn, x, out, temp, stream):
    import torch
    _check_tensor(x, torch.uint32, "x")
    out = torch.empty_like(x) if out is None else out
    need = fn(None, None, x.numel(), None, 0)
    temp = _temp(need, x.device) if temp is None else temp
    fn(x, out, x.numel(), temp, temp.numel(), stream)
    return out


def exclusive_scan_u32(x, out=None, temp=None, stream=None):
    """Exclusive prefix sums of a uint32 tensor, modulo 2^32."""
    return _scan_tensor(rs_exclusive_scan_u32, x, out, temp, stream)


def inclusive_scan_u32(x, out=None, temp=None, stream=None):
    """Inclusive prefix sums of a uint32 tensor, modulo 2^32."""
    return _scan_tensor(rs_inclusive_scan_u32, x, out, temp, stream)


def _threshold_bits(x, threshold):
    import numpy as np
    dt = {RS_KEY_U32: np.uint32, RS_KEY_I32: np.int32, RS_KEY_F32: np.float32}
    kt, _ = _key_type(x)
    if kt not in dt:
        raise TypeError("select and partition take uint32, int32 or float32 elements")
    return kt, int(np.array([threshold], dt[kt]).view(np.uint32)[0])


def _select_tensor(fn, x, op, threshold, vals, temp, stream):
    import torch
    kt, bits = _threshold_bits(x, threshold)
    out = torch.empty_like(x)
    vo = None
    if vals is not None:
        _check_tensor(vals, torch.uint32, "vals")
        vo = torch.empty_like(vals)
    count = torch.empty(1, dtype=torch.uint32, device=x.device)
    need = fn(kt, _OPS[op], bits, None, None, vals, vo, None, x.numel(), None, 0)
    temp = _temp(need, x.device) if temp is None else temp
    fn(kt, _OPS[op], bits, x, out, vals, vo, count, x.numel(), temp, temp.numel(), stream)
    return (out, count) if vals is None else (out, vo, count)


def select(x, op, threshold, vals=None, temp=None, stream=None):
    """Elements with `x op threshold` (op in <, <=, >, >=, ==, !=) in order at the front of
    the output; returns (out, count) or (out, vals_out, count); count is a 1-element tensor."""
    return _select_tensor(rs_select, x, op, threshold, vals, temp, stream)


def partition(x, op, threshold, vals=None, temp=None, stream=None):
    """Stable partition: kept elements in order, then the rest in order."""
    return _select_tensor(rs_partition, x, op, threshold, vals, temp, stream)


def compact_positive_f32(x, out=None, count=None, temp=None, stream=None):
    """(out, count): x > 0 kept in order at the front, +0.0 after; count is a 1-element tensor."""
    import torch
    _check_tensor(x, torch.float32, "x")
    n = x.numel()
    out = torch.empty_like(x) if out is None else out
    count = torch.empty(1, dtype=torch.uint32, device=x.device) if count is None else count
    need = rs_compact_positive_f32(None, None, None, n, None, 0)
    temp = _temp(need, x.device) if temp is None else temp
    rs_compact_positive_f32(x, out, count, n, temp, temp.numel(), stream)
    return out, count


def bitonic_tile(keys, tile, begin_bit=0, end_bit=32, out=None, stream=None):
    """Each run of `tile` (<= 1024) keys sorted on its own, stably."""
    import torch
    _check_tensor(keys, torch.uint32, "keys")
    out = torch.empty_like(keys) if out is None else out
    rs_bitonic_tile(keys, out, keys.numel(), tile, begin_bit, end_bit, stream)
    return out
