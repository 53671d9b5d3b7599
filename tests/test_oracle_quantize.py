"""Pins of the oracle's append quantisation (CPU only).

Rule (storage section of the page "kadirnar/kernel-agent/fp8-kv-cache"): one
fp32 scale per (token, KV head) row, scale = amax(|row|) / 448, e4m3 codes.
Pinned by the hand-derived fixture, by exact-rational checks that the scale is
the correctly rounded quotient and each code the nearest e4m3 value, by the
invariant that a row's amax maps to code 448, and by torch's CPU float8
conversion applied to the same fp32 quotient.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from golden_io import quantize_cases


def test_quantize_golden():
    for case in quantize_cases():
        x = np.array([case["x"]], np.float32)
        codes, scales = oracle.quantize_rows(x)
        assert float(scales[0]) == case["scale"], case
        assert list(codes[0]) == case["codes"], case


def _rows(seed, n=256, d=128):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((n, d)).astype(np.float32)
    mag = np.exp(rng.uniform(np.log(1e-38), np.log(1e30), size=(n, 1)))
    x = (x * mag).astype(np.float32)
    x[0] = 0.0
    x[1, ::3] = -0.0
    x[2] *= np.float32(1e-40)   # subnormal amax: scale is a subnormal fp32
    x[3] = np.float32(2.0 ** -149) * np.arange(d, dtype=np.float32)
    return x


def _nearest_fp32_ok(value: np.float32, exact: Fraction) -> bool:
    v = Fraction(float(value))
    lo = Fraction(float(np.nextafter(value, np.float32(-np.inf))))
    hi = Fraction(float(np.nextafter(value, np.float32(np.inf))))
    return abs(v - exact) <= abs(lo - exact) and abs(v - exact) <= abs(hi - exact)


@pytest.mark.parametrize("seed", [0, 1])
def test_scale_is_correctly_rounded_quotient(seed):
    x = _rows(seed)
    _, scales = oracle.quantize_rows(x)
    for r in range(x.shape[0]):
        amax = max(abs(Fraction(float(v))) for v in x[r])
        assert _nearest_fp32_ok(scales[r], amax / 448), r


@pytest.mark.parametrize("seed", [0, 1])
def test_codes_are_nearest_e4m3_of_quotient(seed):
    x = _rows(seed, n=64)
    codes, scales = oracle.quantize_rows(x)
    vals = oracle.e4m3_value(np.arange(0x7F))
    grid = [Fraction(float(v)) for v in vals]
    for r in range(x.shape[0]):
        s = scales[r]
        if s == 0:
            assert np.all(codes[r] == 0)
            continue
        q = (x[r] / s).astype(np.float32)      # the fp32 quotient
        for j in range(x.shape[1]):
            a = min(abs(Fraction(float(q[j]))), Fraction(448))
            c = int(codes[r, j]) & 0x7F
            d = abs(grid[c] - a)
            assert all(d <= abs(g - a) for g in grid), (r, j)
            assert (codes[r, j] >> 7) == int(np.signbit(x[r, j])), (r, j)


def test_amax_maps_to_448():
    x = _rows(2)
    codes, scales = oracle.quantize_rows(x)
    normal = scales >= np.float32(2.0 ** -126)
    vals = np.abs(oracle.e4m3_value(codes))
    assert normal.sum() > 200
    assert np.all(vals[normal].max(axis=1) == 448.0)
    assert np.all(vals <= 448.0)


def test_matches_torch_on_same_quotient():
    x = _rows(3)
    codes, scales = oracle.quantize_rows(x)
    ok = scales >= np.float32(2.0 ** -126)    # |x / scale| <= 464 here
    xt = torch.from_numpy(x[ok])
    st = torch.from_numpy(scales[ok])[:, None]
    ref = (xt / st).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(codes[ok], ref)


def test_round_trip_error_bound():
    """|dec(code) * scale - x| is at most half an e4m3 spacing (times scale)
    plus the fp32 rounding of the quotient, for normal-scale rows."""
    x = _rows(4)
    codes, scales = oracle.quantize_rows(x)
    ok = scales >= np.float32(2.0 ** -126)
    deq = oracle.e4m3_value(codes[ok]) * scales[ok, None].astype(np.float64)
    q = np.abs(x[ok].astype(np.float64) / scales[ok, None])
    e = np.maximum(np.floor(np.log2(np.maximum(q, 2.0 ** -6))), -6)
    half = 2.0 ** (e - 4) * scales[ok, None]
    err = np.abs(deq - x[ok].astype(np.float64))
    assert np.all(err <= half * (1 + 2 ** -20) + np.abs(x[ok]) * 2 ** -23)


def test_bf16_store_rows():
    rng = np.random.default_rng(9)
    k = rng.standard_normal((5, 2, 8)).astype(np.float32)
    v = rng.standard_normal((5, 2, 8)).astype(np.float32)
    s = oracle.store_rows("K16V8", k, v)
    ref = torch.from_numpy(k).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(s["k16"], ref)
    c, sc = oracle.quantize_rows(v)
    assert np.array_equal(s["v8"], c) and np.array_equal(s["vs"], sc)
    b = oracle.store_rows("BF16", k, v)
    assert set(b) == {"k16", "v16"}


# ------------------------------------------------------------ dequantisation

def _dequant_reference(codes, scales):
    """Independent: the e4m3 value table times the scale as an IEEE fp32
    product (numpy, round to nearest), then torch's RNE cast to bfloat16."""
    import torch
    vals = oracle.e4m3_value(codes).astype(np.float32)
    prod = (vals * scales[..., None].astype(np.float32)).astype(np.float32)
    return torch.from_numpy(prod).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_dequantize_matches_fp32_product_then_bf16():
    rng = np.random.default_rng(71)
    scales = np.concatenate([
        np.float32(2.0) ** rng.integers(-149, 0, 16).astype(np.float32),   # powers of two
        rng.random(24, dtype=np.float32) * np.float32(4.0),
        (rng.random(12, dtype=np.float32) * np.float32(1e-38)),            # subnormal scales
        np.float32([0.0, 1.0, 1.0 / 448.0, 3.4e38 / 448.0]),
    ]).astype(np.float32)
    codes = np.tile(np.arange(256, dtype=np.uint8), (scales.size, 1))
    codes[:, [0x7F, 0xFF]] = 0                      # no NaN codes in a stored row
    got = oracle.dequantize_rows(codes, scales)
    assert np.array_equal(got, _dequant_reference(codes, scales))


def test_dequantize_power_of_two_scale_is_exact():
    """e4m3 values have 4 significant bits (bf16: 8), so with a power-of-two
    scale inside the normal range the result is the exact product."""
    codes = np.arange(256, dtype=np.uint8).reshape(1, 256).copy()
    codes[0, [0x7F, 0xFF]] = 0
    for e in (-20, -6, 0, 5):
        s = np.array([2.0 ** e], np.float32)
        got = oracle.bf16_value(oracle.dequantize_rows(codes, s))
        want = oracle.e4m3_value(codes).astype(np.float64) * 2.0 ** e
        assert np.array_equal(got, want), e


def test_dequantize_round_trip_error():
    """dequant(quant(x)) is within half an e4m3 step (times the scale) of x,
    plus the bf16 rounding of the result."""
    rng = np.random.default_rng(72)
    x = (rng.standard_normal((200, 64)) * 3).astype(np.float32)
    codes, scales = oracle.quantize_rows(x)
    y = oracle.bf16_value(oracle.dequantize_rows(codes, scales))
    err = np.abs(y - x.astype(np.float64))
    bound = (np.abs(x) * 2.0 ** -4 + scales[:, None] * 2.0 ** -10) + np.abs(y) * 2.0 ** -8
    assert np.all(err <= bound)
