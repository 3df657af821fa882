"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module holds only random-number recipes (numpy PCG64, ``default_rng``);
none of the sort or compaction arithmetic lives here, so the CPU oracle and
the HIP library can both be fed from it without sharing any method code.

The pages' own workloads are a JSON file of keys that is not available, C
``rand()`` integers and an N of about 10^8 for compaction; the recipes below
stand in for them.  Every generator takes ``n`` so that tests can draw the
same distribution at sizes the oracle finishes in seconds.

Recipes (seed 0 unless stated):

* ``uniform_u32(n)``: ``rng.integers(0, 2**32, n, dtype=uint32)``.
* ``zipf_u32(n)``: truncated Zipf, exponent 1.2, over 65536 values by inverse
  CDF: ``p_k ~ k**-1.2`` for k = 1..65536, ``key = min(searchsorted(cdf, u,
  'right'), 65535)`` with ``u = rng.random()``; key 0 is the most frequent.
* ``signed_mix_f32(n)``: ``floor(0.45 n)`` positive values ``|N(0,1)|`` (exact
  zeros replaced by 1.0), as many negative ``-|N(0,1)|`` (exact zeros replaced
  by 1.0 before the sign, so no -0.0), the rest +0.0; concatenated in that
  order, then shuffled with ``rng.permutation``.
* ``normal_specials_f32(n)``: ``N(0,1)`` float32, then four disjoint index sets
  of ``n // 256`` each, taken in order from one ``rng.permutation(n)``, are set
  to -0.0, +0.0, +1e-38 (bits 0x006CE3EE, subnormal) and -1e-38 (0x806CE3EE).
* values for key-value sorts: ``arange(n, dtype=uint32)`` (original index).
* ``splat_pairs(gaussians)``: screen-space splats for a tile renderer (the
  pages introduce radix sort as the sorting step of a Gaussian-splatting
  renderer; the key layout below is this build's synthetic stand-in, no
  scene is used).  A 1920 x 1080 screen in 16 x 16-pixel tiles (120 x 68 =
  8160 tiles, 13 bits of tile id).  Each splat has a centre drawn uniformly
  over the screen (70 %) or from 8 Gaussian clusters of sigma 80 pixels
  (30 %, clipped to the screen), a radius of 2 + 30 * u^3 pixels (u uniform,
  so most splats are small) and a depth uniform in [0.2, 100).  It emits one
  entry per tile its bounding square touches: key = tile id * 2^32 + the
  bit pattern of the float depth (positive floats order as their patterns),
  value = the splat's index.  Sorting the keys on bits [0, 32 + 13) groups
  the entries by tile and orders each tile front to back.
"""
import numpy as np

SEED = 0

# The workloads the measurements are quoted on (sizes in elements).
N_TILE = 1024            # keys-only tile: bitonic tile and 4-pass radix
N_PAIRS_SMALL = 1 << 20  # uniform key-value pairs
N_ZIPF = 1 << 26         # Zipf(1.2) key-value pairs over bits [0, 16)
N_COMPACT = 1 << 28      # float compaction
N_FLOAT_PAIRS = 1 << 28  # float key-value pairs with injected specials
N_HEADLINE = 1 << 28     # uniform u32 keys / key-value pairs

SUBNORMAL_POS_BITS = 0x006CE3EE  # +1e-38f
SUBNORMAL_NEG_BITS = 0x806CE3EE  # -1e-38f


def rng_for(seed=SEED):
    return np.random.default_rng(seed)


def uniform_u32(n, seed=SEED):
    return rng_for(seed).integers(0, 2**32, n, dtype=np.uint32)


def index_values(n):
    return np.arange(n, dtype=np.uint32)


def zipf_u32(n, seed=SEED, exponent=1.2, support=65536, chunk=1 << 24):
    rng = rng_for(seed)
    k = np.arange(1, support + 1, dtype=np.float64)
    p = k ** (-exponent)
    cdf = np.cumsum(p) / p.sum()
    out = np.empty(n, np.uint32)
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        u = rng.random(e - s)
        idx = np.searchsorted(cdf, u, side="right")
        np.minimum(idx, support - 1, out=idx)
        out[s:e] = idx.astype(np.uint32)
    return out


def signed_mix_f32(n, seed=SEED):
    rng = rng_for(seed)
    n_pos = int(np.floor(0.45 * n))
    n_neg = n_pos
    n_zero = n - n_pos - n_neg
    pos = np.abs(rng.standard_normal(n_pos, dtype=np.float32))
    pos[pos == 0] = np.float32(1.0)
    neg = np.abs(rng.standard_normal(n_neg, dtype=np.float32))
    neg[neg == 0] = np.float32(1.0)
    np.negative(neg, out=neg)
    zeros = np.zeros(n_zero, np.float32)
    x = np.concatenate([pos, neg, zeros])
    del pos, neg, zeros
    return rng.permutation(x)


def signed_mix_expected_count(n):
    """Positive count of ``signed_mix_f32(n)`` by construction."""
    return int(np.floor(0.45 * n))


def normal_specials_f32(n, seed=SEED):
    rng = rng_for(seed)
    x = rng.standard_normal(n, dtype=np.float32)
    m = n // 256
    if m > 0:
        idx = rng.permutation(n)
        bits = x.view(np.uint32)
        bits[idx[0:m]] = np.uint32(0x80000000)          # -0.0
        bits[idx[m:2 * m]] = np.uint32(0x00000000)      # +0.0
        bits[idx[2 * m:3 * m]] = np.uint32(SUBNORMAL_POS_BITS)
        bits[idx[3 * m:4 * m]] = np.uint32(SUBNORMAL_NEG_BITS)
    return x


# --- the named workloads -------------------------------------------------------

def tile_keys(seed=SEED):
    """1024 uniform u32 keys (keys-only, bitonic tile and 4-pass radix)."""
    return uniform_u32(N_TILE, seed)


def pairs_small(n=N_PAIRS_SMALL, seed=SEED):
    """Uniform u32 keys with index values, full 32 bits."""
    return uniform_u32(n, seed), index_values(n)


def pairs_zipf(n=N_ZIPF, seed=SEED):
    """Zipf(1.2) keys over 65536 values with index values, bits [0, 16)."""
    return zipf_u32(n, seed), index_values(n)


def compact_input(n=N_COMPACT, seed=SEED):
    return signed_mix_f32(n, seed)


def float_pairs(n=N_FLOAT_PAIRS, seed=SEED):
    """N(0,1) float keys with injected +-0 and +-1e-38, index values."""
    return normal_specials_f32(n, seed), index_values(n)


def headline_pairs(n=N_HEADLINE, seed=SEED):
    return uniform_u32(n, seed), index_values(n)


# --- tile/depth keys of a splat renderer ------------------------------------------------

SPLAT_W, SPLAT_H, SPLAT_TILE = 1920, 1080, 16
SPLAT_TILES_X = (SPLAT_W + SPLAT_TILE - 1) // SPLAT_TILE
SPLAT_TILES_Y = (SPLAT_H + SPLAT_TILE - 1) // SPLAT_TILE
SPLAT_TILE_BITS = int(np.ceil(np.log2(SPLAT_TILES_X * SPLAT_TILES_Y)))


def splat_pairs(gaussians, seed=SEED):
    """(keys uint64, values uint32) for `gaussians` splats (see the module notes)."""
    rng = rng_for(seed)
    cx = rng.random(gaussians) * SPLAT_W
    cy = rng.random(gaussians) * SPLAT_H
    clustered = rng.random(gaussians) < 0.3
    centres = rng.random((8, 2)) * np.array([SPLAT_W, SPLAT_H])
    which = rng.integers(0, 8, gaussians)
    jitter = rng.standard_normal((gaussians, 2)) * 80.0
    cx = np.where(clustered, np.clip(centres[which, 0] + jitter[:, 0], 0, SPLAT_W - 1), cx)
    cy = np.where(clustered, np.clip(centres[which, 1] + jitter[:, 1], 0, SPLAT_H - 1), cy)
    radius = 2.0 + 30.0 * rng.random(gaussians) ** 3
    depth = (0.2 + rng.random(gaussians) * 99.8).astype(np.float32)
    tx0 = np.clip(((cx - radius) // SPLAT_TILE).astype(np.int64), 0, SPLAT_TILES_X - 1)
    tx1 = np.clip(((cx + radius) // SPLAT_TILE).astype(np.int64), 0, SPLAT_TILES_X - 1)
    ty0 = np.clip(((cy - radius) // SPLAT_TILE).astype(np.int64), 0, SPLAT_TILES_Y - 1)
    ty1 = np.clip(((cy + radius) // SPLAT_TILE).astype(np.int64), 0, SPLAT_TILES_Y - 1)
    wx = tx1 - tx0 + 1
    wy = ty1 - ty0 + 1
    count = wx * wy
    owner = np.repeat(np.arange(gaussians, dtype=np.int64), count)
    local = np.arange(owner.size, dtype=np.int64) - np.repeat(np.cumsum(count) - count, count)
    tx = tx0[owner] + local % wx[owner]
    ty = ty0[owner] + local // wx[owner]
    tile = (ty * SPLAT_TILES_X + tx).astype(np.uint64)
    keys = (tile << np.uint64(32)) | depth.view(np.uint32)[owner].astype(np.uint64)
    return keys, owner.astype(np.uint32)
