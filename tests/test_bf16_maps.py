"""Host-side check of the bf16 row kernel's compile-time tables and order keys
(draft_tree_verification_build_amd/csrc/bf16_maps.h, plain C++17, compiled here with g++).

- Every exp table entry against the C library's exp (Python's math.exp) within 1 ulp, for
  each bf16 value 2^-16 <= |v| < 2^8, and the 1.0 and 0.0 pairs after them.
- The 16-bit order key over all 65536 patterns: monotone in the value (NaNs aside), -0 and
  +0 equal, every key in 1..0xFFFF, and its inverse giving back the pattern (-0 gives +0)."""
from __future__ import annotations

import math
import os
import shutil
import struct
import subprocess

import numpy as np
import pytest

CSRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                    "draft_tree_verification_build_amd", "csrc")

PROGRAM = r"""
#include <cstdio>
#include "bf16_maps.h"
int main() {
  printf("%u %u %d\n", dtv::kExpBf16Lo, dtv::kExpBf16Mags, dtv::kExpBf16Entries);
  for (int i = 0; i < dtv::kExpBf16Entries; ++i) printf("%a\n", dtv::kExpBf16Tab.v[i]);
  for (unsigned b = 0; b < 65536; ++b) printf("%u %u\n", dtv::bf16_order_key(b), dtv::bf16_key_bits(dtv::bf16_order_key(b)));
  return 0;
}
"""


@pytest.fixture(scope="module")
def dump(tmp_path_factory):
    if shutil.which("g++") is None:
        pytest.skip("g++ not available")
    d = tmp_path_factory.mktemp("bf16maps")
    src, exe = d / "maps.cpp", d / "maps"
    src.write_text(PROGRAM)
    subprocess.run(["g++", "-std=c++17", "-O1", "-I", CSRC, str(src), "-o", str(exe)], check=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.split("\n")
    lo, mags, entries = (int(x) for x in out[0].split())
    tab = np.array([float.fromhex(x) for x in out[1:1 + entries]])
    keys = np.array([[int(v) for v in line.split()] for line in out[1 + entries:1 + entries + 65536]])
    return lo, mags, tab, keys


def bf16_value(bits: int) -> float:
    return struct.unpack(">f", struct.pack(">I", bits << 16))[0]


def test_exp_table_within_one_ulp(dump):
    lo, mags, tab, _ = dump
    assert bf16_value(lo) == 2.0 ** -16 and bf16_value(lo + mags) == 256.0
    assert tab.size == 2 * mags + 4
    worst = 0.0
    for r in range(mags):
        v = bf16_value(lo + r)
        for s, x in ((0, v), (1, -v)):
            e = math.exp(x)
            worst = max(worst, abs(tab[2 * r + s] - e) / math.ulp(e))
    assert worst <= 1.0, worst
    assert list(tab[2 * mags:]) == [1.0, 1.0, 0.0, 0.0]


def test_order_keys(dump):
    _, _, _, keys = dump
    k, back = keys[:, 0], keys[:, 1]
    assert k.min() >= 1 and k.max() <= 0xFFFF
    vals = np.array([bf16_value(b) for b in range(65536)])
    ok = ~np.isnan(vals)
    order = np.argsort(vals[ok], kind="stable")
    kv = k[ok][order]
    assert np.all(np.diff(kv) >= 0)
    # equal keys only for equal values (-0 and +0)
    same = np.diff(kv) == 0
    assert np.all(np.diff(vals[ok][order])[same] == 0)
    assert k[0x8000] == k[0x0000]
    expect = np.arange(65536)
    expect[0x8000] = 0x0000
    np.testing.assert_array_equal(back, expect)
