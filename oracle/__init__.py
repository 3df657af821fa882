"""CPU oracle for the stable LSD radix sort, compaction and bitonic tile.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg may import this package; the library under
``sorting_lsd_radix_amd`` never does.  The arithmetic lives in ``oracle.c``
(plain C, built with gcc -O2, single-threaded); this module only marshals
numpy arrays into it.  See ``oracle.c`` for the passages each function
follows.

``Oracle(path)`` binds the same functions to another build of the C source;
the tests use it to check that planted mistakes make the pins fail.
"""
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "oracle.c")
LIB_PATH = os.path.join(_HERE, "liboracle.so")
GCC_FLAGS = ["-O2", "-std=c99", "-fPIC", "-shared", "-Wall", "-Wextra", "-fno-fast-math"]


def compile_source(src, out):
    """Compile a C source of the oracle into a shared library at `out`."""
    subprocess.run(["gcc"] + GCC_FLAGS + ["-o", out + ".tmp", src], check=True)
    os.replace(out + ".tmp", out)
    return out


def build(force=True):
    """Compile oracle.c into liboracle.so (every call when force is true)."""
    if force or not os.path.exists(LIB_PATH):
        compile_source(SOURCE, LIB_PATH)
    return LIB_PATH


_U32P = ctypes.POINTER(ctypes.c_uint32)
_U64P = ctypes.POINTER(ctypes.c_uint64)
_F32P = ctypes.POINTER(ctypes.c_float)


def _ptr(a, ctype):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def _u32(a):
    a = np.ascontiguousarray(a)
    if a.dtype != np.uint32:
        raise TypeError("expected uint32 array, got %s" % a.dtype)
    return a


def _f32_bits(a):
    a = np.ascontiguousarray(a)
    if a.dtype == np.float32:
        return a.view(np.uint32)
    return _u32(a)


def _check(rc, what):
    if rc < 0:
        raise ValueError("%s failed with code %d" % (what, rc))
    return rc


class Oracle:
    """The oracle's functions bound to one build of the C source."""

    def __init__(self, path=None):
        if path is None:
            if not os.path.exists(LIB_PATH):
                build(force=False)
            path = LIB_PATH
        lib = ctypes.CDLL(path)
        u64 = ctypes.c_uint64
        i32 = ctypes.c_int
        lib.oracle_lsd_sort_u32.argtypes = [_U32P, _U32P, _U32P, _U32P, u64, i32, i32, i32]
        lib.oracle_lsd_sort_u32.restype = i32
        lib.oracle_sort_pairs_f32.argtypes = [_U32P, _U32P, _U32P, _U32P, u64, i32, i32, i32]
        lib.oracle_sort_pairs_f32.restype = i32
        lib.oracle_digit_histograms.argtypes = [_U32P, u64, i32, i32, i32, _U64P]
        lib.oracle_digit_histograms.restype = i32
        lib.oracle_compact_positive_f32.argtypes = [_F32P, _F32P, u64]
        lib.oracle_compact_positive_f32.restype = u64
        lib.oracle_bitonic_tile.argtypes = [_U32P, _U32P, u64, u64, i32, i32]
        lib.oracle_bitonic_tile.restype = i32
        lib.oracle_f32_to_order.argtypes = [_U32P, _U32P, u64]
        lib.oracle_f32_to_order.restype = None
        lib.oracle_order_to_f32.argtypes = [_U32P, _U32P, u64]
        lib.oracle_order_to_f32.restype = None
        vp = ctypes.c_void_p
        lib.oracle_lsd_sort_u64.argtypes = [_U64P, _U32P, _U64P, _U32P, u64, i32, i32, i32]
        lib.oracle_lsd_sort_u64.restype = i32
        lib.oracle_sort_typed.argtypes = [i32, i32, vp, _U32P, vp, _U32P, u64, i32, i32, i32]
        lib.oracle_sort_typed.restype = i32
        lib.oracle_digit_histograms_typed.argtypes = [i32, i32, vp, u64, i32, i32, _U64P]
        lib.oracle_digit_histograms_typed.restype = i32
        lib.oracle_sort_two_keys.argtypes = [_U32P, _U32P, _U32P, _U32P, _U32P, _U32P, u64]
        lib.oracle_sort_two_keys.restype = i32
        lib.oracle_scan_u32.argtypes = [_U32P, _U32P, u64, i32]
        lib.oracle_scan_u32.restype = None
        lib.oracle_select.argtypes = [i32, i32, ctypes.c_uint32, _U32P, _U32P, _U32P, _U32P, u64,
                                      i32]
        lib.oracle_select.restype = ctypes.c_int64
        self.lib = lib
        self.path = path

    def sort_u32(self, keys, vals=None, begin_bit=0, end_bit=32, digit_bits=8):
        """Stable LSD radix sort by bits [begin_bit, end_bit); keys or (keys, vals)."""
        keys = _u32(keys)
        n = keys.size
        k_out = np.empty(n, np.uint32)
        if vals is None:
            _check(self.lib.oracle_lsd_sort_u32(_ptr(keys, ctypes.c_uint32), None,
                                                _ptr(k_out, ctypes.c_uint32), None, n,
                                                begin_bit, end_bit, digit_bits),
                   "oracle_lsd_sort_u32")
            return k_out
        vals = _u32(vals)
        if vals.size != n:
            raise ValueError("keys and vals differ in length")
        v_out = np.empty(n, np.uint32)
        _check(self.lib.oracle_lsd_sort_u32(_ptr(keys, ctypes.c_uint32),
                                            _ptr(vals, ctypes.c_uint32),
                                            _ptr(k_out, ctypes.c_uint32),
                                            _ptr(v_out, ctypes.c_uint32),
                                            n, begin_bit, end_bit, digit_bits),
               "oracle_lsd_sort_u32")
        return k_out, v_out

    def sort_f32(self, keys, vals=None, begin_bit=0, end_bit=32, digit_bits=8):
        """Stable sort of float32 keys by the order-preserving transform."""
        bits = _f32_bits(keys)
        n = bits.size
        k_out = np.empty(n, np.uint32)
        v_out = None
        vp = None
        if vals is not None:
            vals = _u32(vals)
            if vals.size != n:
                raise ValueError("keys and vals differ in length")
            v_out = np.empty(n, np.uint32)
            vp = _ptr(vals, ctypes.c_uint32)
        _check(self.lib.oracle_sort_pairs_f32(_ptr(bits, ctypes.c_uint32), vp,
                                              _ptr(k_out, ctypes.c_uint32),
                                              _ptr(v_out, ctypes.c_uint32),
                                              n, begin_bit, end_bit, digit_bits),
               "oracle_sort_pairs_f32")
        if vals is None:
            return k_out.view(np.float32)
        return k_out.view(np.float32), v_out

    def digit_histograms(self, keys, begin_bit=0, end_bit=32, transform_f32=False):
        """counts[p, d] for every 8-bit pass p over [begin_bit, end_bit) (uint64)."""
        bits = _f32_bits(keys) if transform_f32 else _u32(keys)
        passes = (end_bit - begin_bit + 7) // 8
        out = np.zeros(max(passes, 1) * 256, np.uint64)
        p = _check(self.lib.oracle_digit_histograms(_ptr(bits, ctypes.c_uint32), bits.size,
                                                    begin_bit, end_bit,
                                                    int(bool(transform_f32)),
                                                    _ptr(out, ctypes.c_uint64)),
                   "oracle_digit_histograms")
        return out[: p * 256].reshape(p, 256)

    def compact_positive_f32(self, x):
        """(out, count): x > 0 kept in order at the front, +0.0 after."""
        x = np.ascontiguousarray(x, dtype=np.float32)
        out = np.empty_like(x)
        k = self.lib.oracle_compact_positive_f32(_ptr(x, ctypes.c_float),
                                                 _ptr(out, ctypes.c_float), x.size)
        return out, int(k)

    def bitonic_tile(self, keys, tile, begin_bit=0, end_bit=32):
        """Each consecutive run of `tile` keys sorted on its own, stably."""
        keys = _u32(keys)
        out = np.empty_like(keys)
        _check(self.lib.oracle_bitonic_tile(_ptr(keys, ctypes.c_uint32),
                                            _ptr(out, ctypes.c_uint32),
                                            keys.size, tile, begin_bit, end_bit),
               "oracle_bitonic_tile")
        return out

    def f32_to_order(self, bits):
        """Order-preserving transform of float32 bit patterns (uint32 -> uint32)."""
        bits = _f32_bits(bits)
        out = np.empty(bits.size, np.uint32)
        self.lib.oracle_f32_to_order(_ptr(bits, ctypes.c_uint32), _ptr(out, ctypes.c_uint32),
                                     bits.size)
        return out

    def order_to_f32(self, order):
        """Inverse of f32_to_order (uint32 -> uint32 bit patterns)."""
        order = _u32(order)
        out = np.empty(order.size, np.uint32)
        self.lib.oracle_order_to_f32(_ptr(order, ctypes.c_uint32), _ptr(out, ctypes.c_uint32),
                                     order.size)
        return out


    # ---- key types, 64-bit keys, multi-key --------------------------------------

    def sort_u64(self, keys, vals=None, begin_bit=0, end_bit=64, digit_bits=8):
        """Stable LSD radix sort of uint64 keys by bits [begin_bit, end_bit)."""
        keys = np.ascontiguousarray(keys)
        if keys.dtype != np.uint64:
            raise TypeError("expected uint64 keys, got %s" % keys.dtype)
        n = keys.size
        k_out = np.empty(n, np.uint64)
        v_out = None
        vp = None
        if vals is not None:
            vals = _u32(vals)
            if vals.size != n:
                raise ValueError("keys and vals differ in length")
            v_out = np.empty(n, np.uint32)
            vp = _ptr(vals, ctypes.c_uint32)
        _check(self.lib.oracle_lsd_sort_u64(_ptr(keys, ctypes.c_uint64), vp,
                                            _ptr(k_out, ctypes.c_uint64),
                                            _ptr(v_out, ctypes.c_uint32),
                                            n, begin_bit, end_bit, digit_bits),
               "oracle_lsd_sort_u64")
        return k_out if vals is None else (k_out, v_out)

    def sort_typed(self, keys, vals=None, begin_bit=0, end_bit=None, descending=False,
                   digit_bits=8):
        """Stable sort of a uint32/int32/float32/uint64/int64/float64 array by
        bits [begin_bit, end_bit) of its order pattern (end_bit defaults to the
        key width), ascending or descending; returns keys or (keys, vals)."""
        keys = np.ascontiguousarray(keys)
        key_type = KEY_TYPES[keys.dtype.type]
        width = keys.dtype.itemsize * 8
        end_bit = width if end_bit is None else end_bit
        n = keys.size
        k_out = np.empty_like(keys)
        v_out = None
        vp = None
        if vals is not None:
            vals = _u32(vals)
            if vals.size != n:
                raise ValueError("keys and vals differ in length")
            v_out = np.empty(n, np.uint32)
            vp = _ptr(vals, ctypes.c_uint32)
        _check(self.lib.oracle_sort_typed(key_type, int(bool(descending)), keys.ctypes.data, vp,
                                          k_out.ctypes.data, _ptr(v_out, ctypes.c_uint32), n,
                                          begin_bit, end_bit, digit_bits),
               "oracle_sort_typed")
        return k_out if vals is None else (k_out, v_out)

    def digit_histograms_typed(self, keys, begin_bit=0, end_bit=None, descending=False):
        """counts[p, d] of the order patterns of typed keys (uint64)."""
        keys = np.ascontiguousarray(keys)
        key_type = KEY_TYPES[keys.dtype.type]
        end_bit = keys.dtype.itemsize * 8 if end_bit is None else end_bit
        passes = (end_bit - begin_bit + 7) // 8
        out = np.zeros(max(passes, 1) * 256, np.uint64)
        p = _check(self.lib.oracle_digit_histograms_typed(key_type, int(bool(descending)),
                                                          keys.ctypes.data, keys.size, begin_bit,
                                                          end_bit, _ptr(out, ctypes.c_uint64)),
                   "oracle_digit_histograms_typed")
        return out[: p * 256].reshape(p, 256)

    def sort_two_keys(self, first, second, vals=None):
        """Stable sort by `first`, then stable sort of that by `second` (the
        multi-key exercise); returns (first, second) or (first, second, vals)
        permuted."""
        first, second = _u32(first), _u32(second)
        n = first.size
        if second.size != n:
            raise ValueError("keys differ in length")
        f_out = np.empty(n, np.uint32)
        s_out = np.empty(n, np.uint32)
        v_out = None
        if vals is not None:
            vals = _u32(vals)
            if vals.size != n:
                raise ValueError("keys and vals differ in length")
            v_out = np.empty(n, np.uint32)
        _check(self.lib.oracle_sort_two_keys(_ptr(first, ctypes.c_uint32),
                                             _ptr(second, ctypes.c_uint32),
                                             _ptr(vals, ctypes.c_uint32),
                                             _ptr(f_out, ctypes.c_uint32),
                                             _ptr(s_out, ctypes.c_uint32),
                                             _ptr(v_out, ctypes.c_uint32), n),
               "oracle_sort_two_keys")
        return (f_out, s_out) if vals is None else (f_out, s_out, v_out)


    # ---- scan and select -----------------------------------------------------------

    def scan_u32(self, x, inclusive=False):
        """Prefix sums of a uint32 array modulo 2^32 (exclusive by default)."""
        x = _u32(x)
        out = np.empty_like(x)
        self.lib.oracle_scan_u32(_ptr(x, ctypes.c_uint32), _ptr(out, ctypes.c_uint32), x.size,
                                 int(bool(inclusive)))
        return out

    def select(self, x, op, threshold, vals=None, partition=False):
        """Elements of a uint32/int32/float32 array with `x OP threshold` (OP in
        OPS), in input order; with partition the rejected ones follow in input
        order.  Returns (out, count) or (out, vals_out, count); without
        partition only out[:count] is defined (the rest is zero here)."""
        x = np.ascontiguousarray(x)
        key_type = KEY_TYPES[x.dtype.type]
        if key_type > 2:
            raise TypeError("select takes 4-byte elements")
        bits = x.view(np.uint32)
        tbits = int(np.array([threshold], x.dtype).view(np.uint32)[0])
        out = np.zeros(x.size, np.uint32)
        v_out = None
        if vals is not None:
            vals = _u32(vals)
            if vals.size != x.size:
                raise ValueError("values differ in length")
            v_out = np.zeros(x.size, np.uint32)
        k = _check(self.lib.oracle_select(key_type, OPS[op], tbits, _ptr(bits, ctypes.c_uint32),
                                          _ptr(vals, ctypes.c_uint32), _ptr(out, ctypes.c_uint32),
                                          _ptr(v_out, ctypes.c_uint32), x.size,
                                          int(bool(partition))), "oracle_select")
        out = out.view(x.dtype)
        return (out, int(k)) if vals is None else (out, v_out, int(k))


# comparison operators of select (the library uses the same numbering)
OPS = {"<": 0, "<=": 1, ">": 2, ">=": 3, "==": 4, "!=": 5}

# numpy scalar type -> key type code of oracle_sort_typed (the library uses
# the same numbering)
KEY_TYPES = {np.uint32: 0, np.int32: 1, np.float32: 2, np.uint64: 3, np.int64: 4, np.float64: 5}

_default = None


def default():
    """The oracle built from oracle.c in this directory."""
    global _default
    if _default is None:
        _default = Oracle()
    return _default


def sort_u32(*a, **k):
    return default().sort_u32(*a, **k)


def sort_f32(*a, **k):
    return default().sort_f32(*a, **k)


def digit_histograms(*a, **k):
    return default().digit_histograms(*a, **k)


def compact_positive_f32(*a, **k):
    return default().compact_positive_f32(*a, **k)


def bitonic_tile(*a, **k):
    return default().bitonic_tile(*a, **k)


def f32_to_order(*a, **k):
    return default().f32_to_order(*a, **k)


def order_to_f32(*a, **k):
    return default().order_to_f32(*a, **k)


def sort_u64(*a, **k):
    return default().sort_u64(*a, **k)


def sort_typed(*a, **k):
    return default().sort_typed(*a, **k)


def digit_histograms_typed(*a, **k):
    return default().digit_histograms_typed(*a, **k)


def sort_two_keys(*a, **k):
    return default().sort_two_keys(*a, **k)


def scan_u32(*a, **k):
    return default().scan_u32(*a, **k)


def select(*a, **k):
    return default().select(*a, **k)
