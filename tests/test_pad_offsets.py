"""Pad stores of the last, partial tile never land inside the output (CPU only).

A one-sweep pass pads a partial last tile with keys that rank after every
real key of the last digit, so their destinations are n, n + 1, ...,
tiles * TILE - 1.  The scatter stores them through a buffer descriptor of n
elements, which drops every store whose byte offset is at least 4 n.  The
byte offset is a 32-bit quantity: for a tile that reaches past 2^30 keys,
dst * 4 wraps round 2^32 and would land at the start of the buffer, so the
kernel clamps dst to n before scaling.  This test replays, for every n in
the top window of the accepted sizes, the tile count the library chooses
(read back from its temp-size query, which sizes two look-back state arrays
of tiles x 256 words) and the pad-offset arithmetic of the scatter.
"""
import numpy as np

import sorting_lsd_radix_amd as rs

MAX_N = 1 << 30
WINDOW = 2 * 28672
FIXED = 4 * 256 * 4 + 4 * 64 * 4 + 64 * 4   # digit counts + tile counters of four passes + multi-pass counters


def align256(x):
    return (x + 255) // 256 * 256


def tiles_from_query(n, pairs):
    if pairs:
        temp = rs.rs_sort_pairs_u32(None, None, None, None, n, 0, 32, None, 0)
    else:
        temp = rs.rs_sort_keys_u32(None, None, n, 0, 32, None, 0)
    states = temp - FIXED - (2 if pairs else 1) * align256(4 * n)
    assert states % 2 == 0
    per_array = states // 2
    assert per_array % 1024 == 0, (n, temp)
    return per_array // 1024


def pad_offsets(n, tiles, tile_keys, clamp):
    """Byte offsets (mod 2^32) of the pad stores of the last tile."""
    dst = np.arange(n, tiles * tile_keys, dtype=np.uint64)
    if clamp:
        dst = np.minimum(dst, np.uint64(n))
    return (dst * np.uint64(4)) & np.uint64(0xFFFFFFFF)


def test_pad_stores_fall_outside_the_output_near_the_size_limit():
    wrapped_before_fix = 0
    for pairs, tile_keys in ((True, 28672), (False, 32768)):
        for n in range(MAX_N - WINDOW, MAX_N):
            tiles = tiles_from_query(n, pairs)
            assert tiles == -(-n // tile_keys), (pairs, n, tiles)
            if tiles * tile_keys == n:
                continue   # a full last tile has no pads
            off = pad_offsets(n, tiles, tile_keys, clamp=True)
            assert np.all(off >= np.uint64(4 * n)), (pairs, n)
            raw = pad_offsets(n, tiles, tile_keys, clamp=False)
            if np.any(raw < np.uint64(4 * n)):
                wrapped_before_fix += 1
    # without the clamp, exactly the pair sorts whose last tile reaches past
    # 2^30 keys would have stored pads into the output's first elements
    assert wrapped_before_fix == 4095


def test_sizes_past_the_limit_are_refused():
    for n in (MAX_N, MAX_N + 1):
        try:
            rs.rs_sort_pairs_u32(None, None, None, None, n, 0, 32, None, 0)
        except rs.RsError as e:
            assert e.status == rs.RS_ERR_UNSUPPORTED_SIZE
        else:
            raise AssertionError("n = %d accepted" % n)
