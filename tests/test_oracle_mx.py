"""Pins of the oracle's block-scaled (MX) K path (CPU only).

MXFP8 for block-scaled QK (hardware notes, "Measure block-scaled QK"): e4m3
elements with one power-of-two scale 2^E per block of 32 consecutive values.
Scale policy (a reading; the pages leave it to be validated): E =
ceil(log2(fp32(amax / 448))), clamped to [-126, 127], so that nothing clamps.

* E against its definition, computed exactly (fractions) over wide random and
  edge amax values.
* Codes against a brute-force nearest-e4m3 search of the exact quotient.
* Invariants: no quotient beyond 448 (up to the fp32 rounding of amax/448),
  every nonzero block's largest code value above 224, hand-derived values.
* Attention: textbook fp64 softmax on the dequantised keys (code * 2^E) with
  unrounded P; block-scaled query rows alike; online equals two-pass.
* The format's error against the BF16 cache, reported next to per-row K8V8.
"""
import math
from fractions import Fraction

import numpy as np
import pytest
import scipy.special

import oracle
from fp8_kv_cache_append_amd import synth

FINITE = np.array([c for c in range(256) if c & 0x7F != 0x7F], np.uint8)
FINITE_VALUES = [Fraction(float(v)) for v in oracle.e4m3_value(FINITE)]


def _exact_exponent(amax: float) -> int:
    s = float(np.float32(amax) / np.float32(448.0))      # correctly rounded fp32
    if not s >= 2.0 ** -126:
        return -126
    e = math.ceil(math.log2(s))
    while 2.0 ** e < s:          # guard log2 rounding: smallest e with 2^e >= s
        e += 1
    while 2.0 ** (e - 1) >= s:
        e -= 1
    return min(e, 127)


def test_exponent_matches_definition():
    rng = np.random.default_rng(1)
    vals = list(np.float32(np.exp2(rng.uniform(-140, 127.9, size=4000))))
    vals += [0.0, 448.0, 449.0, 896.0, 1.0, 1e-40, 3e38, 448.0 * 2.0 ** -126,
             np.nextafter(np.float32(448.0), np.float32(1000.0))]
    for a in vals:
        assert oracle.mx_exponent(float(a)) == _exact_exponent(float(a)), a


def _nearest_code(y: Fraction) -> int:
    y = max(min(y, Fraction(448)), Fraction(-448))
    best, bd = None, None
    for c, v in zip(FINITE, FINITE_VALUES):
        dd = abs(v - y)
        if bd is None or dd < bd or (dd == bd and int(c) % 2 == 0 and int(best) % 2 == 1):
            best, bd = c, dd
    # the sign of zero follows the input
    if FINITE_VALUES[list(FINITE).index(best)] == 0:
        return 0x80 if y < 0 else 0x00
    return int(best)


def test_codes_match_brute_force():
    rng = np.random.default_rng(2)
    x = (rng.standard_normal((6, 128)) * np.exp2(rng.integers(-20, 20, size=(6, 1)))).astype(
        np.float32)
    x[0, :32] = 0.0                     # a zero block
    x[1, 5] *= 300                      # an outlier in a block
    codes, exps = oracle.quantize_rows_mx(x)
    for r in range(x.shape[0]):
        for b in range(4):
            blk = x[r, 32 * b:32 * b + 32]
            e = _exact_exponent(float(np.abs(blk).max()))
            assert int(exps[r, b]) == e + 127
            for j in range(32):
                want = _nearest_code(Fraction(float(blk[j])) / Fraction(2) ** e)
                assert int(codes[r, 32 * b + j]) == want, (r, b, j)


def test_invariants_and_hand_values():
    rng = np.random.default_rng(3)
    x = (rng.standard_normal((64, 128)) * 3).astype(np.float32)
    codes, exps = oracle.quantize_rows_mx(x)
    e = exps.astype(np.int64) - 127
    q = x.reshape(64, 4, 32) / np.exp2(e)[..., None]
    assert np.abs(q).max() <= 448.0 * (1 + 2.0 ** -22)
    top = np.abs(oracle.e4m3_value(codes).reshape(64, 4, 32)).max(-1)
    assert top.min() >= 224.0
    # hand-derived: amax 448 -> E = 0, code of 448 is 0x7E; amax 1 -> E = -8,
    # 1.0 * 2^8 = 256 = 0x78; amax 449 -> E = 1, 449 / 2 = 224.5 -> 224 = 0x76
    for amax, e_want, code_want in ((448.0, 0, 0x7E), (1.0, -8, 0x78), (449.0, 1, 0x76)):
        blk = np.zeros((1, 32), np.float32)
        blk[0, 7] = amax
        c, ex = oracle.quantize_rows_mx(blk)
        assert int(ex[0, 0]) - 127 == e_want and int(c[0, 7]) == code_want


def _mx_inputs(seed, dist="outliers"):
    w = synth.Workload("t", 2, 16, 2, 128, np.array([90, 70], np.int32), dist, seed=seed)
    seqs = [synth.kv_sequence(w, b) for b in range(w.batch)]
    q_bits = synth.q_bf16_bits(seed, (w.batch, w.q_heads, 128))
    return w, q_bits, [s[0] for s in seqs], [s[1] for s in seqs]


def _deq_mx(store):
    k = oracle.e4m3_value(store["k8"]) * np.exp2(
        store["kx"].astype(np.int64) - 127).repeat(32, axis=-1)
    v = oracle.e4m3_value(store["v8"]) * store["vs"][..., None].astype(np.float64)
    return k, v


@pytest.mark.parametrize("narrow", [False, True])
def test_unrounded_equals_textbook(narrow):
    w, q_bits, ks, vs = _mx_inputs(4)
    g = w.group
    if narrow:
        qc, qx = oracle.quantize_q_mx(q_bits)
        q = oracle.e4m3_value(qc) * np.exp2(qx.astype(np.int64) - 127).repeat(32, axis=-1)
    else:
        q = oracle.bf16_value(q_bits)
    want = np.zeros(q_bits.shape)
    for b in range(w.batch):
        k, v = _deq_mx(oracle.store_rows("MXK8V8", ks[b], vs[b]))
        for h in range(w.q_heads):
            s = k[:, h // g] @ q[b, h] * float(np.float32(w.sm_scale))
            want[b, h] = scipy.special.softmax(s) @ v[:, h // g]
    got = oracle.decode("MXK8V8", q_bits, ks, vs, w.sm_scale, round_p=False, q8=narrow)
    assert oracle.rel_l2(got, want) < 1e-12


def test_v_side_is_the_k8v8_one():
    w, q_bits, ks, vs = _mx_inputs(5)
    a = oracle.store_rows("MXK8V8", ks[0], vs[0])
    b = oracle.store_rows("K8V8", ks[0], vs[0])
    assert np.array_equal(a["v8"], b["v8"]) and np.array_equal(a["vs"], b["vs"])


@pytest.mark.parametrize("narrow", [False, True])
def test_online_equals_two_pass(narrow):
    w, q_bits, ks, vs = _mx_inputs(6)
    store = oracle.store_rows("MXK8V8", ks[0], vs[0])
    view = {k: np.ascontiguousarray(a[:, 0]) for k, a in store.items()}
    rows = q_bits[0, :8]
    q8 = None
    if narrow:
        qc, qx = oracle.quantize_q_mx(rows)
        q8 = (qc, None, qx)
    n_valid = np.array([90, 89, 1, 0, 64, 65, 33, 17], np.int32)
    two = oracle.attend_rows("MXK8V8", rows, view, n_valid, w.sm_scale, q8=q8)
    on, _, _, _ = oracle.attend_rows_online("MXK8V8", rows, view, n_valid, w.sm_scale, 16, 48,
                                            q8=q8)
    assert oracle.rel_l2(on, two) < 1e-12


def test_error_against_bf16_reported():
    """Block scales are powers of two, so unlike the per-row scale they
    cannot map a row's largest element exactly onto 448: on Gaussian data MX
    matches per-row K8V8, on rows dominated by outliers or biased channels it
    is worse."""
    for dist in ("normal", "outliers", "bias"):
        w, q_bits, ks, vs = _mx_inputs(7, dist)
        ref = oracle.decode("BF16", q_bits, ks, vs, w.sm_scale)
        e = {m: oracle.rel_l2(oracle.decode(m, q_bits, ks, vs, w.sm_scale), ref)
             for m in ("K8V8", "MXK8V8")}
        print(f"{dist}: K8V8 {e['K8V8']:.4f}  MXK8V8 {e['MXK8V8']:.4f}")
        assert e["MXK8V8"] < 3 * e["K8V8"]
