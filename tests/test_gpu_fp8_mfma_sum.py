"""The fp8 matrix instruction's own sum, measured on the device: the bound the
oracle's narrow-QK rounding interval allows it (ORC_NARROW_SUM_ERR in
oracle/oracle.c, 2^-10 of the absolute sum of the products).

Narrow QK ("FP8 KV attention: hardware paths and tile preparation", "AMD
CDNA 3") feeds e4m3 query and key codes to v_mfma_scale_f32_16x16x128_f8f6f4
with unit block scales, one instruction per 16 keys at head_dim 128.  The
instruction's fp32 result is not the correctly rounded sum of its 128 exact
code products.  This test drives the same instruction through a fixture
(tests/hw/fp8_mfma_probe.hip, built by __graft_entry__.build()) on seeded code
vectors and compares every result with the exact sum: every product of two
e4m3 values is an integer multiple of 2^-18 below 2^18, so 128 of them sum
exactly in fp64.  Code sets: every finite code, normal codes only, half
subnormal codes, and rows quantised from N(0,1) and from biased-key data by
the cache-row rule (what the kernel meets).  The worst error seen, as a power
of two of the absolute product sum, is printed.
"""
import ctypes
import os

import numpy as np
import pytest
import torch

import oracle

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "hw", "libfp8mfma_probe.so")
BOUND_LOG2 = -10.0     # ORC_NARROW_SUM_ERR
N_TILES = 512          # 512 x 256 = 131,072 dot products per code set

FINITE = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
NORMAL = np.array([c for c in FINITE if (c & 0x78) != 0], np.uint8)
SUBNORMAL = np.array([c for c in FINITE if (c & 0x78) == 0], np.uint8)


def _probe(a, b):
    assert a.shape == b.shape == (N_TILES, 16, 128) and a.dtype == b.dtype == np.uint8
    lib = ctypes.CDLL(LIB)
    lib.fp8_mfma_probe.restype = ctypes.c_int
    lib.fp8_mfma_probe.argtypes = [ctypes.c_void_p] * 3 + [ctypes.c_int, ctypes.c_void_p]
    da = torch.from_numpy(np.ascontiguousarray(a)).cuda()
    db = torch.from_numpy(np.ascontiguousarray(b)).cuda()
    out = torch.full((N_TILES, 16, 16), float("nan"), device="cuda")
    st = lib.fp8_mfma_probe(da.data_ptr(), db.data_ptr(), out.data_ptr(), N_TILES,
                            torch.cuda.current_stream().cuda_stream)
    assert st == 0, st
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64)


def _codes_from(rng, pool, shape):
    return pool[rng.integers(0, pool.size, size=shape)]


def _quantised(rng, shape, bias):
    x = rng.standard_normal(size=shape).astype(np.float32)
    if bias:
        x[..., rng.choice(128, size=8, replace=False)] += np.float32(20.0)
    return oracle.quantize_rows(x)[0]


def _case(name, rng):
    shape = (N_TILES, 16, 128)
    if name == "finite":
        return _codes_from(rng, FINITE, shape), _codes_from(rng, FINITE, shape)
    if name == "normal":
        return _codes_from(rng, NORMAL, shape), _codes_from(rng, NORMAL, shape)
    if name == "half_subnormal":
        def mixed():
            x = _codes_from(rng, FINITE, shape)
            sub = rng.random(shape) < 0.5
            x[sub] = _codes_from(rng, SUBNORMAL, int(sub.sum()))
            return x
        return mixed(), mixed()
    if name == "quantised_rows":
        return _quantised(rng, shape, False), _quantised(rng, shape, True)
    raise ValueError(name)


@pytest.mark.skipif(not os.path.exists(LIB), reason="probe fixture not built")
@pytest.mark.parametrize("name", ["finite", "normal", "half_subnormal", "quantised_rows"])
def test_fp8_instruction_sum_within_oracle_bound(name):
    rng = np.random.default_rng(["finite", "normal", "half_subnormal",
                                 "quantised_rows"].index(name) + 19)
    a, b = _case(name, rng)
    got = _probe(a, b)
    va = oracle.e4m3_value(a)                           # exact fp64 values
    vb = oracle.e4m3_value(b)
    exact = np.einsum("tik,tjk->tij", va, vb)           # exact: see the docstring
    abs_sum = np.einsum("tik,tjk->tij", np.abs(va), np.abs(vb))
    err = np.abs(got - exact)
    zero = abs_sum == 0
    assert np.all(err[zero] == 0)
    ratio = err[~zero] / abs_sum[~zero]
    worst = float(ratio.max())
    frac_exact = float(np.mean(err == 0))
    print(f"{name}: worst |fp8 instruction - exact| = 2^{np.log2(max(worst, 2.0 ** -60)):.2f}"
          f" of sum|products| (bound 2^{BOUND_LOG2:.0f}); exact in {100 * frac_exact:.1f}%"
          f" of {err.size} dot products", flush=True)
    assert worst <= 2.0 ** BOUND_LOG2, (name, worst)
