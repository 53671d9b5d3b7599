"""reciprocal_rn (device.h): the hardware reciprocal and one Newton step.
The append's codes rely on it returning the correctly rounded reciprocal
RN(1 / s) of every scale it is used for, [2^-53, 2^125] (quotient_rn's
correction step needs RN(1 / s)).  This test runs the library's function on
the device (fixture tests/hw/reciprocal_probe.hip, built by
__graft_entry__.build()) for every fp32 s in that range, 1.5 G values, and
compares each with the correctly rounded division 1.0f / s; it also shows
that the range ends where it must: from 2^126 on (1 / s subnormal) the two
differ."""
import ctypes
import os

import pytest
import torch

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "hw", "libreciprocal_probe.so")


def _count(lo: int, hi: int):
    lib = ctypes.CDLL(LIB)
    lib.reciprocal_probe_launch.restype = ctypes.c_int
    lib.reciprocal_probe_launch.argtypes = [ctypes.c_uint32, ctypes.c_uint32, ctypes.c_void_p,
                                            ctypes.c_void_p, ctypes.c_void_p]
    bad = torch.zeros(1, dtype=torch.int64, device="cuda")
    kept = torch.zeros(17, dtype=torch.int32, device="cuda")
    st = lib.reciprocal_probe_launch(lo, hi, bad.data_ptr(), kept.data_ptr(),
                                     torch.cuda.current_stream().cuda_stream)
    assert st == 0, st
    torch.cuda.synchronize()
    k = kept.cpu().numpy().view("uint32")
    return int(bad.item()), [hex(int(x)) for x in k[1:1 + min(int(k[0]), 16)]]


def test_reciprocal_rn_is_correctly_rounded_on_its_range():
    lo, hi = 0x25000000, 0x7C7FFFFF  # 2^-53 .. the largest fp32 below 2^126 (2^125 included)
    n_bad, kept = _count(lo, hi)
    print(f"reciprocal_rn: {hi - lo + 1} scales, {n_bad} differ from 1/s")
    assert n_bad == 0, kept


def test_reciprocal_rn_range_ends_where_one_over_s_is_subnormal():
    n_bad, _ = _count(0x7E800000, 0x7E80FFFF)  # s in [2^126, 2^126 + 65535 ulp]
    assert n_bad > 0
