"""The split and merge kernels divide by the head count, the block size, the
split count and the group size with FastDiv (launch.h): a multiplier and a
shift computed on the host, floor(n / d) = (mulhi(m, n) + n) >> l for
0 <= n < 2^31 (Granlund and Montgomery, "Division by invariant integers using
multiplication", section 4).  This test compiles the header's host code and
checks its constants against exact integer division: every divisor up to
4096 and a spread of larger ones (powers of two, their neighbours, random),
each at the dividends where rounding is closest (multiples of d and their
neighbours, the top of the range) and at random ones."""
import os
import subprocess

import numpy as np
import pytest

from fp8_kv_cache_append_amd import build

pytestmark = pytest.mark.skipif(not os.path.exists(build.HIPCC), reason="hipcc not installed")

SRC = r"""
#include "launch.h"
#include <cstdio>
int main() {
  int d;
  while (std::scanf("%d", &d) == 1) {
    const fp8kv::FastDiv f = fp8kv::FastDiv::of(d);
    std::printf("%u %u %d\n", f.m, f.l, f.d);
  }
  return 0;
}
"""


def _divisors(rng):
    ds = set(range(1, 4097))
    for k in range(31):
        ds.update({2 ** k, 2 ** k + 1, max(1, 2 ** k - 1)})
    ds.update(int(x) for x in rng.integers(1, 2 ** 31 - 1, size=2000))
    return sorted(d for d in ds if 1 <= d < 2 ** 31)


def test_fastdiv_constants_divide_exactly(tmp_path):
    src = tmp_path / "fastdiv.cpp"
    src.write_text(SRC)
    exe = tmp_path / "fastdiv"
    subprocess.run([build.HIPCC, "-x", "hip", "--offload-arch=gfx950", "-O2", "-std=c++17",
                    "-I", build.CSRC, str(src), "-o", str(exe)], check=True, capture_output=True)
    rng = np.random.default_rng(7)
    ds = _divisors(rng)
    out = subprocess.run([str(exe)], input="\n".join(map(str, ds)) + "\n", check=True,
                         capture_output=True, text=True).stdout.split("\n")
    top = 2 ** 31 - 1
    for d, line in zip(ds, out):
        m, l, dd = (int(x) for x in line.split())
        assert dd == d and 0 <= m < 2 ** 32 and 0 <= l <= 31
        ns = np.concatenate([
            np.array([0, 1, top, top - 1, top // d * d, top // d * d - 1], np.int64),
            (np.arange(1, 64, dtype=np.int64)[:, None] * d + np.array([-1, 0, 1])).ravel(),
            rng.integers(0, 2 ** 31, size=64, dtype=np.int64)])
        ns = ns[(ns >= 0) & (ns <= top)].astype(object)     # exact Python integers
        got = [(((m * n) >> 32) + n) >> l for n in ns]
        assert got == [n // d for n in ns], d
