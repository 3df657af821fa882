"""Planted mistakes in the oracle must make at least one pin fail.

Each mutant is a copy of ``oracle/oracle.c`` with one textual change (a
dropped step, a wrong index, an inclusive scan, a wrong sign transform ...),
built with gcc into a temporary directory and run against the quick pins.
The real oracle is untouched; this only shows that the pins are strong
enough to catch plausible slips.  CPU only.
"""
import os
import subprocess
import sys

import pytest

import oracle
import pins

TESTS = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(TESTS)

MUTANTS = [
    ("inclusive scan instead of exclusive",
     "cnt[d] = sum;\n        sum += c;", "sum += c;\n        cnt[d] = sum;"),
    ("scatter in reverse input order (unstable)",
     "for (j = 0; j < n; ++j) {\n        uint32_t dg", "for (j = n; j-- > 0;) {\n        uint32_t dg"),
    ("values not moved with their keys",
     "dst_vals[slot] = src_vals[j];", "dst_vals[slot] = src_vals[slot];"),
    ("last digit not narrowed to the bit range",
     "if (width > digit_bits)\n            width = digit_bits;\n        counting_sort_pass",
     "width = digit_bits;\n        counting_sort_pass"),
    ("digit shift off by one",
     "return (key >> shift) & mask;", "return (key >> (shift + 1)) & mask;"),
    ("pass loop stops one digit early",
     "for (shift = begin_bit; shift < end_bit; shift += digit_bits)",
     "for (shift = begin_bit; shift + digit_bits < end_bit; shift += digit_bits)"),
    ("negative floats not inverted",
     "return (u & 0x80000000u) ? ~u : (u | 0x80000000u);",
     "return (u & 0x80000000u) ? u : (u | 0x80000000u);"),
    ("sign bit of non-negative floats not set",
     "return (u & 0x80000000u) ? ~u : (u | 0x80000000u);",
     "return (u & 0x80000000u) ? ~u : u;"),
    ("inverse transform wrong for negatives",
     "return (o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o;",
     "return (o & 0x80000000u) ? (o & 0x7FFFFFFFu) : (o ^ 0x80000000u);"),
    ("compaction keeps zeros",
     "if (x > 0.0f) {", "if (x >= 0.0f) {"),
    ("compaction tail not zero-filled",
     "out[i] = 0.0f;", "out[i] = in[i];"),
    ("compaction skips the first element",
     "for (i = 0; i < n; ++i) {\n        float x", "for (i = 1; i < n; ++i) {\n        float x"),
    ("histogram ignores the float transform",
     "uint32_t k = transform_f32 ? f32_to_order(keys[i]) : keys[i];", "uint32_t k = keys[i];"),
    ("histogram pass digit not narrowed",
     "if (width > 8)\n            width = 8;\n        for (i = 0; i < n; ++i) {",
     "width = 8;\n        for (i = 0; i < n; ++i) {"),
    ("bitonic tile sorts across tile boundaries",
     "uint64_t len = (n - s < tile) ? (n - s) : tile;", "uint64_t len = n - s;"),
    ("signed 32-bit keys not offset",
     "p = (uint64_t)((int64_t)((const int32_t *)keys)[i] + ((int64_t)1 << 31));",
     "p = (uint32_t)((const int32_t *)keys)[i];"),
    ("signed 64-bit keys not offset",
     "p = ((const uint64_t *)keys)[i] + ((uint64_t)1 << 63);", "p = ((const uint64_t *)keys)[i];"),
    ("negative doubles not inverted",
     "p = (p & top) ? ~p : (p | top);", "p = (p & top) ? p : (p | top);"),
    ("descending order not complemented",
     "p = all - p;", "p = p + 0 * all;"),
    ("descending complement of 64-bit keys on 32 bits",
     "uint64_t all = (w == 64) ? ~(uint64_t)0 : (uint64_t)0xFFFFFFFFu;",
     "uint64_t all = (uint64_t)0xFFFFFFFFu;"),
    ("64-bit sort skips the digits of the high word",
     "        counting_sort_pass64(ka, va, kb, vb, n, shift, width, cnt);",
     "        if (shift >= 32)\n            continue;\n        counting_sort_pass64(ka, va, kb, vb, n, shift, width, cnt);"),
    ("64-bit digit taken from the low word only",
     "return (key >> shift) & low_bits;", "return ((uint32_t)key >> (shift & 31)) & low_bits;"),
    ("64-bit sort: last digit not narrowed",
     "int width = (end_bit - shift < digit_bits) ? end_bit - shift : digit_bits;",
     "int width = digit_bits;"),
    ("64-bit sort: pass loop stops one digit early",
     "for (shift = begin_bit; end_bit > shift; shift += digit_bits)",
     "for (shift = begin_bit; end_bit > shift + digit_bits; shift += digit_bits)"),
    ("64-bit pass: inclusive scan",
     "cnt[d] = running;\n        running += here;", "running += here;\n        cnt[d] = running;"),
    ("64-bit pass: values not moved with their keys",
     "dst_vals[at] = src_vals[j];", "dst_vals[at] = src_vals[at];"),
    ("64-bit pass: scatter in reverse input order",
     "for (j = 0; j < n; ++j) {\n        uint64_t dg", "for (j = n; j-- > 0;) {\n        uint64_t dg"),
    ("two-key sort: first step sorts by the second key",
     "rc = oracle_lsd_sort_u32(first, idx, tmp_keys, perm1, n, 0, 32, 8);",
     "rc = oracle_lsd_sort_u32(second, idx, tmp_keys, perm1, n, 0, 32, 8);"),
    ("two-key sort: second step forgets the first step's order",
     "rc = oracle_lsd_sort_u32(second_by1, perm1, tmp_keys, perm, n, 0, 32, 8);",
     "rc = oracle_lsd_sort_u32(second, idx, tmp_keys, perm, n, 0, 32, 8);"),
    ("exclusive scan adds the element first",
     "out[i] = running;\n            running += x;", "running += x;\n            out[i] = running;"),
    ("scan sums in the wrong direction",
     "            running += x;\n            out[i] = running;", "            running -= x;\n            out[i] = running;"),
    ("signed select compares as unsigned",
     "return compare_i32(a, b, op);", "return compare_u32((uint32_t)a, (uint32_t)b, op);"),
    ("float select compares bit patterns",
     "return compare_f32(a, b, op);", "return compare_u32(u, threshold_bits, op);"),
    ("partition puts the rejected elements in reverse order",
     "for (i = 0; i < n; ++i) {\n            if (!selected(", "for (i = n; i-- > 0;) {\n            if (!selected("),
    ("partition leaves the values of rejected elements behind",
     "vals_out[k + r] = vals[i];", "vals_out[k + r] = vals[k + r];"),
    ("typed histogram ignores descending order",
     "uint64_t pat = order_pattern(key_type, descending, keys, i);",
     "uint64_t pat = order_pattern(key_type, 0, keys, i);"),
]


_RUNNER = r"""
import sys
sys.path[:0] = [sys.argv[1], sys.argv[2]]
import oracle, pins
m = oracle.Oracle(sys.argv[3])
caught = []
for pin in pins.QUICK_PINS:
    try:
        pin(m)
    except (AssertionError, ValueError, IndexError):
        caught.append(pin.__name__)
print("CAUGHT", " ".join(caught))
"""


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, name, old, new):
    src = open(oracle.SOURCE, encoding="utf-8").read()
    assert src.count(old) == 1, "mutation anchor not unique in oracle.c: %r" % old
    path = os.path.join(str(tmp_path), "mutant.c")
    with open(path, "w", encoding="utf-8") as f:
        f.write(src.replace(old, new))
    lib = oracle.compile_source(path, os.path.join(str(tmp_path), "libmutant.so"))
    # A mutant may write out of bounds and abort; run it in its own process.
    r = subprocess.run([sys.executable, "-c", _RUNNER, ROOT, TESTS, lib],
                       capture_output=True, text=True, timeout=600)
    if r.returncode != 0:
        return  # the planted mistake crashed the oracle: caught
    line = [ln for ln in r.stdout.splitlines() if ln.startswith("CAUGHT")][-1]
    assert line.split()[1:], "no pin caught the mutant: " + name
