"""The append's quotients x / scale (device.h, e4m3_codes4) come from one
correctly rounded reciprocal y = RN(1 / scale) per row and quotient_rn:
q = RN(x y), r = x - scale q (exact, one fma), RN(q + r y) with the sign of x.
By Markstein's theorem on the fma-corrected reciprocal this is the correctly
rounded quotient when nothing underflows.  The e4m3 code depends on the fp32
quotient only through RN(x / scale), so the rule the kernel relies on is:
wherever RN(x / scale) has magnitude 2^-11 or more, quotient_rn equals it bit
for bit; below that both have magnitude under 2^-10 and the sign of x, i.e.
both encode to the same signed zero.

This test compiles the header's quotient_rn for the host (IEEE fp32 mul and
fma, as on the GPU) and checks the rule against host division for scales
amax / 448 across the range the kernel sends to this path ([2^-53, FLT_MAX]:
powers of two, significands of all ones, random), at random x in
[-amax, amax], at x whose quotient lies within a few ulps of every e4m3
rounding midpoint and of the saturation bound 448, and at every fp32 x in a
window of quotients around 1 and around 2^-11.  It also checks storage_scale,
the scale RN(amax / 448) from the constant RN(1 / 448) and quotient_rn,
against the division."""
import os
import subprocess

import pytest

from fp8_kv_cache_append_amd import build

pytestmark = pytest.mark.skipif(not os.path.exists(build.HIPCC), reason="hipcc not installed")

SRC = r"""
#include "device.h"
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
static float f_of(uint32_t u) { float f; std::memcpy(&f, &u, 4); return f; }
static uint32_t u_of(float f) { uint32_t u; std::memcpy(&u, &f, 4); return u; }
static uint64_t state = 0x9e3779b97f4a7c15ull;
static uint64_t next() { state ^= state << 13; state ^= state >> 7; state ^= state << 17; return state; }
static long checked = 0, failed = 0;
static void check(float x, float s, float y) {
  const float ref = x / s, got = fp8kv::quotient_rn(x, s, y);
  ++checked;
  if (u_of(ref) == u_of(got)) return;
  if (std::fabs(ref) < 0x1p-11f && std::fabs(got) < 0x1p-10f && std::signbit(ref) == std::signbit(got))
    return;
  if (failed++ < 5) std::printf("FAIL x=%a s=%a ref=%a got=%a\n", x, s, ref, got);
}
int main() {
  uint32_t amaxes[160];
  int n = 0;
  // powers of two, all-ones significands and random, with scale in [2^-53, 2^119]
  for (int e = -44; e <= 127; e += 19) {
    amaxes[n++] = (uint32_t)(e + 127) << 23;
    amaxes[n++] = ((uint32_t)(e + 127) << 23) | 0x7fffffu;
  }
  amaxes[n++] = 0x43e00000u;  // 448: scale 1
  amaxes[n++] = 0x43dfffffu;  // scale 0x1.fffffep-1
  amaxes[n++] = 0x43e00001u;
  while (n < 160) amaxes[n++] = (uint32_t)((next() % (127 + 44)) + 127 - 44) << 23 | (uint32_t)(next() & 0x7fffff);
  for (int k = 0; k < n; ++k) {
    const float amax = f_of(amaxes[k]);
    const float s = amax / 448.0f;
    if (!(s >= 0x1p-53f && s <= 0x1.fffffep127f)) continue;
    const float y = 1.0f / s;
    for (int j = 0; j < 200000; ++j) {  // random x in [-amax, amax]
      const double r = (double)(next() >> 11) / 9007199254740992.0 * 2.0 - 1.0;
      check((float)(r * amax), s, y);
    }
    for (int e = -12; e <= 8; ++e)      // quotients near e4m3 midpoints and 448
      for (int m = 0; m < 16; ++m) {
        const double qm = (e >= -6 ? (8 + m + 0.5) / 8.0 * std::ldexp(1.0, e)
                                   : (m + 0.5) * std::ldexp(1.0, -9));
        const float x0 = (float)(qm * s);
        for (int d = -4; d <= 4; ++d) {
          const float x = f_of(u_of(x0) + d);
          if (std::fabs(x) <= amax) { check(x, s, y); check(-x, s, y); }
        }
      }
    for (int d = -64; d <= 64; ++d) { const float x = f_of(u_of(amax) + d); if (std::fabs(x) <= amax) check(x, s, y); }
    if (k % 16 == 0) {                  // every x in two windows of quotients
      for (float lo : {1.0f, 0x1p-11f}) {
        const uint32_t a = u_of(lo * s), b = u_of(lo * s * 1.25f);
        for (uint32_t u = a; u <= b && u - a < (1u << 21); ++u) { check(f_of(u), s, y); check(-f_of(u), s, y); }
      }
    }
  }
  // storage_scale: RN(amax / 448) bit for bit, for every 13th fp32 amax from
  // 2^-100 to FLT_MAX and every fp32 of two whole binades
  long s_checked = 0, s_failed = 0;
  auto check_scale = [&](float amax) {
    ++s_checked;
    if (u_of(fp8kv::storage_scale(amax)) != u_of(amax / 448.0f) && s_failed++ < 5)
      std::printf("FAIL amax=%a\n", amax);
  };
  for (uint32_t u = u_of(0x1p-100f); u < 0x7f800000u; u += 13) check_scale(f_of(u));
  for (uint32_t u = u_of(1.0f); u < u_of(4.0f); ++u) check_scale(f_of(u));
  check_scale(0.0f);
  check_scale(0x1p-149f);
  check_scale(0x1.fffffep127f);
  checked += s_checked;
  failed += s_failed;
  std::printf("%ld %ld\n", checked, failed);
  return 0;
}
"""


def test_quotient_rn_matches_division_where_codes_depend_on_it(tmp_path):
    src = tmp_path / "quot.cpp"
    src.write_text(SRC)
    exe = tmp_path / "quot"
    subprocess.run([build.HIPCC, "-x", "hip", "--offload-arch=gfx950", "-O2", "-std=c++17",
                    "-ffp-contract=off", "-I", build.CSRC, str(src), "-o", str(exe)],
                   check=True, capture_output=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout
    checked, failed = map(int, out.split()[-2:])
    assert checked > 10_000_000
    assert failed == 0, out
