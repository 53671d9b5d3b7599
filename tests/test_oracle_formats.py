"""Pins of the oracle's number formats (CPU only).

The e4m3 table and encoder are pinned to the OCP e4m3fn definition (closed
form, hand-derived fixture, brute-force nearest search with exact rational
comparisons) and to torch's CPU float8_e4m3fn conversion, a library routine.
The bf16 rounding is pinned to torch's CPU bfloat16 conversion and to a
brute-force nearest search.
"""
from concurrent.futures import ThreadPoolExecutor
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from golden_io import e4m3_encode_cases

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def test_e4m3_table_closed_form():
    vals = oracle.e4m3_value(np.arange(256))
    nan = np.isnan(vals)
    assert nan.sum() == 2 and nan[0x7F] and nan[0xFF]
    assert vals[0x7E] == 448.0 and vals[0xFE] == -448.0
    assert vals[0x01] == 2.0 ** -9 and vals[0x08] == 2.0 ** -6
    assert vals[0x38] == 1.0
    pos = vals[:0x7F]
    assert np.all(np.diff(pos) > 0), "non-negative codes must increase"
    # sign symmetry: code | 0x80 negates (0x80 is -0)
    assert np.array_equal(vals[0x80:0xFF], -pos)
    assert np.signbit(vals[0x80])
    # 254 finite values, none larger than 448
    assert np.nanmax(np.abs(vals)) == 448.0


def test_e4m3_table_matches_torch():
    t = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn)
    ref = t.to(torch.float64).numpy()
    vals = oracle.e4m3_value(np.arange(256))
    assert np.array_equal(np.isnan(ref), np.isnan(vals))
    ok = ~np.isnan(ref)
    assert np.array_equal(ref[ok], vals[ok])
    assert np.array_equal(np.signbit(ref[ok]), np.signbit(vals[ok]))


def test_e4m3_encode_golden():
    for x, code, why in e4m3_encode_cases():
        got = int(oracle.e4m3_encode(np.array([x], np.float32))[0])
        assert got == code, f"{x}: got {got:#04x}, want {code:#04x} ({why})"


def _nearest_e4m3(x: float) -> int:
    """Brute force: the finite e4m3 code nearest to x, ties to the even code,
    magnitudes above 448 saturated.  Exact rational comparisons."""
    mags = [Fraction(float(v)) for v in oracle.e4m3_value(np.arange(0x7F))]
    a = min(abs(Fraction(x)), Fraction(448))
    best, best_d = None, None
    for code, m in enumerate(mags):
        d = abs(m - a)
        if best is None or d < best_d or (d == best_d and code % 2 == 0 and best % 2 == 1):
            best, best_d = code, d
    neg = np.signbit(np.float32(x))
    return best | (0x80 if neg else 0)


def test_e4m3_encode_bruteforce():
    rng = np.random.default_rng(11)
    mags = oracle.e4m3_value(np.arange(0x7F))
    mids = (mags[:-1] + mags[1:]) / 2
    xs = [0.0, -0.0, 448.0, 470.0, 1e9, -1e9]
    for m in mids:  # every midpoint and its fp32 neighbours
        f = np.float32(m)
        xs += [float(f), float(np.nextafter(f, np.float32(0))),
               float(np.nextafter(f, np.float32(np.inf)))]
    xs += list(rng.standard_normal(300) * 50)
    xs += list(np.exp(rng.uniform(np.log(1e-6), np.log(440), 300)))
    xs = np.array(xs, np.float32)
    xs = np.concatenate([xs, -xs])
    got = oracle.e4m3_encode(xs)
    for x, g in zip(xs, got):
        assert int(g) == _nearest_e4m3(float(x)), f"x={float(x)!r}"


def _chunk_check(lo: int, hi: int, negate: bool) -> int:
    bits = np.arange(lo, hi, dtype=np.uint32)
    if negate:
        bits |= np.uint32(0x80000000)
    x = bits.view(np.float32)
    got = oracle.e4m3_encode(x)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return int(np.count_nonzero(got != ref))


def test_e4m3_encode_exhaustive_vs_torch():
    """Every fp32 with |y| <= 448 (both signs): oracle == torch CPU RNE."""
    top = int(np.array([448.0], np.float32).view(np.uint32)[0]) + 1
    step = 1 << 23
    jobs = [(lo, min(lo + step, top), neg) for lo in range(0, top, step)
            for neg in (False, True)]
    with ThreadPoolExecutor(max_workers=8) as ex:
        bad = sum(ex.map(lambda j: _chunk_check(*j), jobs))
    assert bad == 0


def test_e4m3_encode_saturates():
    x = np.array([448.0, 448.5, 463.9, 464.0, 500.0, 1e10, 3.4e38], np.float32)
    assert np.all(oracle.e4m3_encode(x) == 0x7E)
    assert np.all(oracle.e4m3_encode(-x) == 0xFE)


def _nearest_bf16(x: float) -> int:
    """Brute force over the two bf16 neighbours by exact rational distance."""
    a = abs(Fraction(x))
    f32 = np.array([abs(x)], np.float64).astype(np.float32)
    u = int(f32.view(np.uint32)[0]) & 0xFFFF0000
    cands = []
    for base in (u - 0x10000, u, u + 0x10000, u + 0x20000):
        if 0 <= base <= 0x7F7F0000:
            v = np.array([base], np.uint32).view(np.float32)[0]
            cands.append((abs(Fraction(float(v)) - a), (base >> 16) & 1, base >> 16))
    cands.sort()
    d0 = cands[0][0]
    ties = [c for c in cands if c[0] == d0]
    pick = min(ties, key=lambda c: c[1])[2]
    return pick | (0x8000 if np.signbit(x) else 0)


def test_bf16_round_f32_vs_torch():
    rng = np.random.default_rng(3)
    bits = rng.integers(0, 2 ** 32, size=1 << 22, dtype=np.uint64).astype(np.uint32)
    # ties and near-ties: low halves 0x8000 and its neighbours
    ties = (rng.integers(0, 2 ** 16, size=1 << 16, dtype=np.uint64).astype(np.uint32) << 16)
    bits = np.concatenate([bits, ties | 0x8000, ties | 0x7FFF, ties | 0x8001,
                           np.arange(0, 1 << 20, dtype=np.uint32)])
    x = bits.view(np.float32)
    x = x[np.isfinite(x) & (np.abs(x) < np.float32(3.3e38))]
    got = oracle.bf16_round_f32(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, ref)


def test_bf16_round_f64_bruteforce():
    rng = np.random.default_rng(5)
    xs = list(rng.standard_normal(400) * np.exp(rng.uniform(-80, 80, 400)))
    # exact bf16 midpoints in fp64 and their fp64 neighbours
    for _ in range(200):
        b = int(rng.integers(0x0080, 0x7F00))
        lo = float(np.array([b << 16], np.uint32).view(np.float32)[0])
        hi = float(np.array([(b + 1) << 16], np.uint32).view(np.float32)[0])
        mid = (lo + hi) / 2
        xs += [mid, np.nextafter(mid, 0.0), np.nextafter(mid, np.inf)]
    xs += [2.0 ** -130, 3 * 2.0 ** -134, 2.0 ** -133 * 1.5]  # bf16 subnormals
    for x in xs:
        for s in (x, -x):
            assert oracle.bf16_round(s) == _nearest_bf16(s), repr(s)
