"""The C-ABI library loads and exports what include/rs.h declares (CPU only).

Only host-side paths run here: symbol lookup, the temp-size query and the
argument checks, all of which return before anything touches a GPU.
"""
import ctypes
import os
import re

import pytest

import sorting_lsd_radix_amd as rs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "rs.h")


def declared_functions():
    text = open(HEADER, encoding="utf-8").read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(rs_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(rs.library_path()):
        from sorting_lsd_radix_amd import build
        build.build()
    return ctypes.CDLL(rs.library_path())


def test_header_declares_the_entry_points():
    names = declared_functions()
    for f in ["rs_sort_keys_u32", "rs_sort_pairs_u32", "rs_sort_pairs_f32",
              "rs_compact_positive_f32", "rs_bitonic_tile", "rs_status_string"]:
        assert f in names
    assert set(names) == set(rs.EXPORTED_SYMBOLS)


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_status_strings():
    for code in range(7):
        assert rs.rs_status_string(code).startswith("RS_")
    assert rs.rs_status_string(99) == "unknown rs_status"


def test_temp_query_depends_only_on_n():
    q1 = rs.rs_sort_pairs_u32(None, None, None, None, 1 << 20, 0, 32, None, 0)
    q2 = rs.rs_sort_pairs_u32(None, None, None, None, 1 << 20, 0, 8, None, 0)
    assert q1 == q2 and q1 > 2 * 4 * (1 << 20)
    k1 = rs.rs_sort_keys_u32(None, None, 1 << 20, 0, 32, None, 0)
    assert 4 * (1 << 20) < k1 < q1
    f1 = rs.rs_sort_pairs_f32(None, None, None, None, 1 << 20, 0, 32, None, 0)
    assert f1 == q1
    c = rs.rs_compact_positive_f32(None, None, None, 1 << 20, None, 0)
    assert 0 < c < (1 << 20)
    assert rs.rs_sort_keys_u32(None, None, 0, 0, 32, None, 0) > 0


@pytest.mark.parametrize("b,e", [(-1, 32), (0, 33), (9, 8)])
def test_bad_bit_range_rejected_before_launch(b, e):
    with pytest.raises(rs.RsError) as ei:
        rs.rs_sort_keys_u32(None, None, 16, b, e, None, 0)
    assert ei.value.status == rs.RS_ERR_INVALID_VALUE
    with pytest.raises(rs.RsError) as ei:
        rs.rs_bitonic_tile(0x1000, 0x2000, 16, 16, b, e, stream=0)
    assert ei.value.status == rs.RS_ERR_INVALID_VALUE


def test_size_limit():
    with pytest.raises(rs.RsError) as ei:
        rs.rs_sort_keys_u32(None, None, 1 << 30, 0, 32, None, 0)
    assert ei.value.status == rs.RS_ERR_UNSUPPORTED_SIZE
    with pytest.raises(rs.RsError) as ei:
        rs.rs_compact_positive_f32(None, None, None, 1 << 30, None, 0)
    assert ei.value.status == rs.RS_ERR_UNSUPPORTED_SIZE


# Fake, never-dereferenced addresses: every case below fails a host check first.
A, B, C, D, T = 0x10000000, 0x20000000, 0x30000000, 0x40000000, 0x50000000


def _pairs(*args, **kw):
    return rs.rs_sort_pairs_u32(*args, **kw)


@pytest.mark.parametrize("args,status", [
    ((None, B, C, D, 64, 0, 32, T, 1 << 30), rs.RS_ERR_INVALID_VALUE),
    ((A, B, None, D, 64, 0, 32, T, 1 << 30), rs.RS_ERR_INVALID_VALUE),
    ((A + 4, B, C, D, 64, 0, 32, T, 1 << 30), rs.RS_ERR_MISALIGNED),
    ((A, B, C, D + 8, 64, 0, 32, T, 1 << 30), rs.RS_ERR_MISALIGNED),
    ((A, B, C, D, 64, 0, 32, T + 4, 1 << 30), rs.RS_ERR_MISALIGNED),
    ((A, B, C, D, 64, 0, 32, T, 16), rs.RS_ERR_TEMP_TOO_SMALL),
    ((A, A + 128, C, D, 64, 0, 32, T, 1 << 30), rs.RS_ERR_OVERLAP),
    ((A, B, C, A, 64, 0, 32, T, 1 << 30), rs.RS_ERR_OVERLAP),
    ((A, B, C, D, 64, 0, 32, A + 64, 1 << 30), rs.RS_ERR_OVERLAP),
])
def test_pairs_argument_errors(args, status):
    with pytest.raises(rs.RsError) as ei:
        _pairs(*args, stream=0)
    assert ei.value.status == status


def test_compaction_argument_errors():
    cases = [
        ((A, B, None, 64, T, 1 << 20), rs.RS_ERR_INVALID_VALUE),
        ((None, B, C, 64, T, 1 << 20), rs.RS_ERR_INVALID_VALUE),
        ((A, B, C + 2, 64, T, 1 << 20), rs.RS_ERR_MISALIGNED),
        ((A + 4, B, C, 64, T, 1 << 20), rs.RS_ERR_MISALIGNED),
        ((A, B, C, 64, T, 8), rs.RS_ERR_TEMP_TOO_SMALL),
        ((A, A + 16, C, 64, T, 1 << 20), rs.RS_ERR_OVERLAP),
        ((A, B, B + 8, 64, T, 1 << 20), rs.RS_ERR_OVERLAP),
    ]
    for args, status in cases:
        with pytest.raises(rs.RsError) as ei:
            rs.rs_compact_positive_f32(*args, stream=0)
        assert ei.value.status == status, args


def test_bitonic_argument_errors():
    for tile in (0, 1025):
        with pytest.raises(rs.RsError) as ei:
            rs.rs_bitonic_tile(A, B, 64, tile, 0, 32, stream=0)
        assert ei.value.status == rs.RS_ERR_INVALID_VALUE
    with pytest.raises(rs.RsError) as ei:
        rs.rs_bitonic_tile(A, A + 16, 64, 64, 0, 32, stream=0)
    assert ei.value.status == rs.RS_ERR_OVERLAP
    with pytest.raises(rs.RsError) as ei:
        rs.rs_bitonic_tile(A + 4, B, 64, 64, 0, 32, stream=0)
    assert ei.value.status == rs.RS_ERR_MISALIGNED


def test_empty_input_is_ok_without_launch():
    # n == 0 returns RS_OK before any launch (keys/pairs/bitonic)
    rs.rs_sort_keys_u32(None, None, 0, 0, 32, T, 1 << 20, stream=0)
    rs.rs_sort_pairs_u32(None, None, None, None, 0, 0, 32, T, 1 << 20, stream=0)
    rs.rs_bitonic_tile(None, None, 0, 16, 0, 32, stream=0)


# --- typed keys, two-key sorts, digit counts ------------------------------------------

def test_typed_key_checks():
    for bad_type in (-1, 6, 99):
        with pytest.raises(rs.RsError) as ei:
            rs.rs_sort_keys(bad_type, 0, None, None, 16, 0, 32, None, 0)
        assert ei.value.status == rs.RS_ERR_INVALID_VALUE
    for kt in (rs.RS_KEY_U32, rs.RS_KEY_I32, rs.RS_KEY_F32):
        assert rs.rs_sort_keys(kt, 1, None, None, 1000, 0, 32, None, 0) > 0
        with pytest.raises(rs.RsError) as ei:
            rs.rs_sort_pairs(kt, 0, None, None, None, None, 1000, 0, 33, None, 0)
        assert ei.value.status == rs.RS_ERR_INVALID_VALUE
    for kt in (rs.RS_KEY_U64, rs.RS_KEY_I64, rs.RS_KEY_F64):
        assert rs.rs_sort_pairs(kt, 0, None, None, None, None, 1000, 0, 64, None, 0) > 0
        with pytest.raises(rs.RsError) as ei:
            rs.rs_sort_keys(kt, 0, None, None, 1000, 0, 65, None, 0)
        assert ei.value.status == rs.RS_ERR_INVALID_VALUE
        with pytest.raises(rs.RsError) as ei:
            rs.rs_sort_keys(kt, 0, None, None, 1 << 29, 0, 64, None, 0)
        assert ei.value.status == rs.RS_ERR_UNSUPPORTED_SIZE
        assert rs.rs_sort_keys(kt, 0, None, None, (1 << 29) - 1, 0, 64, None, 0) > 8 * ((1 << 29) - 1)


def test_typed_temp_query_depends_only_on_n_and_width():
    n = 1 << 20
    u32 = rs.rs_sort_pairs(rs.RS_KEY_U32, 0, None, None, None, None, n, 0, 32, None, 0)
    assert u32 == rs.rs_sort_pairs_u32(None, None, None, None, n, 0, 32, None, 0)
    assert u32 == rs.rs_sort_pairs(rs.RS_KEY_F32, 1, None, None, None, None, n, 3, 9, None, 0)
    u64 = rs.rs_sort_pairs(rs.RS_KEY_U64, 0, None, None, None, None, n, 0, 64, None, 0)
    assert u64 == rs.rs_sort_pairs(rs.RS_KEY_F64, 1, None, None, None, None, n, 7, 40, None, 0)
    assert u64 > 8 * n + 4 * n
    keys64 = rs.rs_sort_keys(rs.RS_KEY_I64, 0, None, None, n, 0, 64, None, 0)
    assert 8 * n < keys64 < u64


def test_two_key_checks():
    q = rs.rs_sort_two_keys_u32(None, None, None, None, None, None, 1 << 20, None, 0)
    assert q > 2 * 8 * (1 << 20)   # two 8-byte key buffers in temp
    with pytest.raises(rs.RsError) as ei:
        rs.rs_sort_two_keys_u32(None, None, None, None, None, None, 1 << 29, None, 0)
    assert ei.value.status == rs.RS_ERR_UNSUPPORTED_SIZE
    with pytest.raises(rs.RsError) as ei:   # values in without values out
        rs.rs_sort_two_keys_u32(A, B, C, D, T, None, 64, T + (1 << 24), 1 << 24, stream=0)
    assert ei.value.status == rs.RS_ERR_INVALID_VALUE
    with pytest.raises(rs.RsError) as ei:   # major out overlaps minor in
        rs.rs_sort_two_keys_u32(A, B, B + 64, D, None, None, 64, T, 1 << 24, stream=0)
    assert ei.value.status == rs.RS_ERR_OVERLAP


def test_digit_count_checks():
    with pytest.raises(rs.RsError) as ei:
        rs.rs_digit_counts(rs.RS_KEY_U32, 0, A, 64, 0, 32, C + 2, stream=0)
    assert ei.value.status == rs.RS_ERR_MISALIGNED
    with pytest.raises(rs.RsError) as ei:
        rs.rs_digit_counts(rs.RS_KEY_U32, 0, A + 4, 64, 0, 32, C, stream=0)
    assert ei.value.status == rs.RS_ERR_MISALIGNED
    with pytest.raises(rs.RsError) as ei:
        rs.rs_digit_counts(rs.RS_KEY_U64, 0, A, 64, 0, 65, C, stream=0)
    assert ei.value.status == rs.RS_ERR_INVALID_VALUE
    with pytest.raises(rs.RsError) as ei:
        rs.rs_digit_counts(rs.RS_KEY_U32, 0, A, 64, 0, 32, None, stream=0)
    assert ei.value.status == rs.RS_ERR_INVALID_VALUE
    with pytest.raises(rs.RsError) as ei:   # counts inside the keys
        rs.rs_digit_counts(rs.RS_KEY_U32, 0, A, 1 << 20, 0, 32, A + 1024, stream=0)
    assert ei.value.status == rs.RS_ERR_OVERLAP
    # an empty bit range counts nothing and launches nothing
    rs.rs_digit_counts(rs.RS_KEY_U32, 0, A, 64, 9, 9, C, stream=0)


def test_scan_and_select_checks():
    assert rs.rs_exclusive_scan_u32(None, None, 1 << 20, None, 0) > 0
    with pytest.raises(rs.RsError) as ei:
        rs.rs_inclusive_scan_u32(None, None, 1 << 30, None, 0)
    assert ei.value.status == rs.RS_ERR_UNSUPPORTED_SIZE
    with pytest.raises(rs.RsError) as ei:   # partial overlap of in and out
        rs.rs_exclusive_scan_u32(A, A + 16, 64, T, 1 << 20, stream=0)
    assert ei.value.status == rs.RS_ERR_OVERLAP
    with pytest.raises(rs.RsError) as ei:
        rs.rs_exclusive_scan_u32(A + 4, B, 64, T, 1 << 20, stream=0)
    assert ei.value.status == rs.RS_ERR_MISALIGNED
    for bad in [(rs.RS_KEY_U64, rs.RS_OP_GT), (rs.RS_KEY_F32, 6), (rs.RS_KEY_F32, -1)]:
        with pytest.raises(rs.RsError) as ei:
            rs.rs_select(bad[0], bad[1], 0, None, None, None, None, None, 64, None, 0)
        assert ei.value.status == rs.RS_ERR_INVALID_VALUE
    with pytest.raises(rs.RsError) as ei:   # values in without values out
        rs.rs_partition(rs.RS_KEY_F32, rs.RS_OP_GT, 0, A, B, C, None, D, 64, T, 1 << 20, stream=0)
    assert ei.value.status == rs.RS_ERR_INVALID_VALUE
    with pytest.raises(rs.RsError) as ei:   # output overlaps the values
        rs.rs_partition(rs.RS_KEY_F32, rs.RS_OP_GT, 0, A, C + 64, C, D, D + (1 << 20), 64, T,
                        1 << 20, stream=0)
    assert ei.value.status == rs.RS_ERR_OVERLAP
    q1 = rs.rs_select(rs.RS_KEY_I32, rs.RS_OP_EQ, 5, None, None, None, None, None, 1 << 20, None, 0)
    q2 = rs.rs_partition(rs.RS_KEY_U32, rs.RS_OP_NE, 9, None, None, None, None, None, 1 << 20,
                         None, 0)
    assert q1 == q2 > 0
