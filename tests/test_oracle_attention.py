"""Pins of the oracle's attention (CPU only).

* The hand-derived fixture (golden/attention_tiny.txt).
* Textbook fp64 attention on dequantised K/V (numpy + scipy softmax) equals
  the oracle with unrounded P: this fixes the score (K scale outside the dot
  product, sm_scale, GQA head mapping h -> h // G), the V scale fold, the
  masking and the normaliser.
* Closed forms with bf16 rounding of P: one key; inputs whose P values are
  exact in bf16.
* The online form (tiles, splits, power-of-two merge) equals the two-pass
  form (FA page, section 2.1: an identity transformation).
* Negative controls from the fp8-kv-cache page's accuracy section (V scale
  times 1.05, one token's scale for every token) and an off-by-one block
  must move the output past the 1e-3 gate.
"""
import math
from fractions import Fraction

import numpy as np
import pytest
import scipy.special

import oracle
from golden_io import attention_case

GATE_REL = 1e-3


# Which side each mode stores as e4m3 codes + fp32 scale (the rest is bf16),
# written out here independently of the oracle's own tables.
_K8 = {"K8V8": True, "K16V8": False, "BF16": False, "K8V16": True}
_V8 = {"K8V8": True, "K16V8": True, "BF16": False, "K8V16": False}


def _deq(mode, store):
    assert set(store) == ({"k8", "ks"} if _K8[mode] else {"k16"}) | (
        {"v8", "vs"} if _V8[mode] else {"v16"}), (mode, sorted(store))
    if _K8[mode]:
        k = oracle.e4m3_value(store["k8"]) * store["ks"][..., None].astype(np.float64)
    else:
        k = oracle.bf16_value(store["k16"])
    if _V8[mode]:
        v = oracle.e4m3_value(store["v8"]) * store["vs"][..., None].astype(np.float64)
    else:
        v = oracle.bf16_value(store["v16"])
    return k, v


def brute_decode(mode, q_bits, k_seqs, v_seqs, sm_scale, lens=None):
    """Textbook softmax(q K^T * sm_scale) V in fp64 on dequantised K/V."""
    b_n, hq, d = q_bits.shape
    hkv = k_seqs[0].shape[1]
    g = hq // hkv
    q = oracle.bf16_value(q_bits)
    out = np.zeros((b_n, hq, d))
    for b in range(b_n):
        k, v = _deq(mode, oracle.store_rows(mode, k_seqs[b], v_seqs[b]))
        n = k.shape[0] if lens is None else lens[b]
        if n == 0:
            continue
        for h in range(hq):
            s = k[:n, h // g] @ q[b, h] * float(np.float32(sm_scale))
            out[b, h] = scipy.special.softmax(s) @ v[:n, h // g]
    return out


def _inputs(seed, b=2, hq=8, hkv=2, d=32, t=50, outliers=True):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((b, hq, d)).astype(np.float32)
    q_bits = oracle.bf16_round_f32(q)
    ks, vs = [], []
    for _ in range(b):
        k = rng.standard_normal((t, hkv, d)).astype(np.float32)
        v = rng.standard_normal((t, hkv, d)).astype(np.float32)
        if outliers:
            k[rng.random(k.shape) < 0.02] *= 10
            v[rng.random(v.shape) < 0.02] *= 10
        ks.append(k)
        vs.append(v)
    return q_bits, ks, vs


# ------------------------------------------------------------ golden

def test_attention_golden():
    c = attention_case()
    k = np.array(c["k"], np.float32)[:, None, :]
    v = np.array(c["v"], np.float32)[:, None, :]
    q_bits = oracle.bf16_round_f32(np.array(c["q"], np.float32))[None, None, :]
    sm = float(np.float32(c["sm_scale"]))
    for key, want in c["out"].items():
        parts = key.split()
        if parts[0] == "unrounded":
            got = oracle.decode("K8V8", q_bits, [k], [v], sm, round_p=False)
        else:
            mode, n = parts[1], int(parts[2])
            got = oracle.decode(mode, q_bits, [k[:n]], [v[:n]], sm)
        np.testing.assert_allclose(got[0, 0], want, rtol=1e-6, atol=1e-9, err_msg=key)


# ------------------------------------------------------------ brute force

@pytest.mark.parametrize("mode", ["K8V8", "K16V8", "BF16", "K8V16"])
@pytest.mark.parametrize("g", [1, 2, 4, 7])
def test_unrounded_equals_textbook_softmax(mode, g):
    hkv = 2
    q_bits, ks, vs = _inputs(7 + g, b=2, hq=g * hkv, hkv=hkv, d=16, t=13)
    sm = 1.0 / math.sqrt(16)
    got = oracle.decode(mode, q_bits, ks, vs, sm, round_p=False)
    ref = brute_decode(mode, q_bits, ks, vs, sm)
    np.testing.assert_allclose(got, ref, rtol=1e-11, atol=1e-12)


def test_masked_prefix_equals_truncated_sequence():
    q_bits, ks, vs = _inputs(21, b=1, hq=4, hkv=1, d=8, t=16)
    sm = 0.3
    store = oracle.store_rows("K8V8", ks[0], vs[0])
    view = {k: a[:, 0] for k, a in store.items()}
    for n in range(0, 17):
        got = oracle.attend_rows("K8V8", q_bits[0], view, n, sm, round_p=False)
        ref = brute_decode("K8V8", q_bits, ks, vs, sm, lens=[n])[0]
        np.testing.assert_allclose(got, ref, rtol=1e-11, atol=1e-12)


def test_empty_sequence_outputs_zero():
    q_bits, ks, vs = _inputs(3, b=1, hq=2, hkv=1, d=8, t=4)
    got = oracle.decode("K8V8", q_bits, [ks[0][:0]], [vs[0][:0]], 0.5)
    assert np.all(got == 0.0)


# ------------------------------------------------------------ bf16 rounding of P

def _nearest_bf16(x: float) -> float:
    """Brute-force nearest bf16 (ties to even) by exact rational distance."""
    if x == 0:
        return 0.0
    f = np.array([abs(x)], np.float64).astype(np.float32).view(np.uint32)[0] & 0xFFFF0000
    best = None
    for base in (int(f) - 0x10000, int(f), int(f) + 0x10000):
        if base < 0:
            continue
        v = float(np.array([base], np.uint32).view(np.float32)[0])
        key = (abs(Fraction(v) - Fraction(abs(x))), (base >> 16) & 1)
        if best is None or key < best[0]:
            best = (key, v)
    return math.copysign(best[1], x)


@pytest.mark.parametrize("mode", ["K8V8", "K16V8", "BF16", "K8V16"])
def test_single_key_closed_form(mode):
    """One key: M = ceil(s), p = 2^(s - M), o = bf16(p * vs) * V / p."""
    rng = np.random.default_rng(41)
    for trial in range(20):
        k = (rng.standard_normal((1, 1, 16)) * 3).astype(np.float32)
        v = (rng.standard_normal((1, 1, 16)) * 3).astype(np.float32)
        q_bits = oracle.bf16_round_f32(rng.standard_normal((1, 1, 16)).astype(np.float32))
        sm = 0.25
        store = oracle.store_rows(mode, k, v)
        kd, _ = _deq(mode, store)
        s = float(kd[0, 0] @ oracle.bf16_value(q_bits[0, 0])) * sm * math.log2(math.e)
        p = 2.0 ** (s - math.ceil(s))
        if not _V8[mode]:
            vs, vhat = 1.0, oracle.bf16_value(store["v16"][0, 0])
        else:
            vs, vhat = float(store["vs"][0, 0]), oracle.e4m3_value(store["v8"][0, 0])
        want = _nearest_bf16(p * vs) * vhat / p
        got = oracle.decode(mode, q_bits, [k], [v], sm)[0, 0]
        np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-300)


def test_bf16_exact_inputs_match_textbook():
    """Integer log2 scores and power-of-two V scales make every P exact in
    bf16, so rounding must leave the textbook result unchanged."""
    d = 4
    # keys give q.K = 0, -1, -2, -3 in log2 units with q = e_0, sm_scale = ln 2
    k = np.zeros((4, 1, d), np.float32)
    k[:, 0, 0] = [0.0, -1.0, -2.0, -3.0]
    k[:, 0, 1] = 448.0 / 64        # amax 7 -> k_scale 2^-6 exactly
    v = np.zeros((4, 1, d), np.float32)
    v[:, 0, 2] = [7.0, 3.5, -7.0, 1.75]  # v_scale 2^-6, 2^-7, 2^-6, 2^-8
    q_bits = oracle.bf16_round_f32(np.array([[[1.0, 0.0, 0.0, 0.0]]], np.float32))
    sm = float(np.float32(math.log(2)))
    got = oracle.decode("K8V8", q_bits, [k], [v], sm)
    ref = oracle.decode("K8V8", q_bits, [k], [v], sm, round_p=False)
    np.testing.assert_allclose(got, ref, rtol=1e-7)
    tb = brute_decode("K8V8", q_bits, [k], [v], sm)
    np.testing.assert_allclose(got, tb, rtol=1e-7)


def test_rounding_is_after_the_v_scale_fold():
    """Rounding p before the V-scale fold would change the golden result."""
    c = attention_case()
    k = np.array(c["k"], np.float32)[:, None, :]
    v = np.array(c["v"], np.float32)[:, None, :]
    q_bits = oracle.bf16_round_f32(np.array(c["q"], np.float32))[None, None, :]
    sm = float(np.float32(c["sm_scale"]))
    got = oracle.decode("K8V8", q_bits, [k], [v], sm)[0, 0]
    unr = oracle.decode("K8V8", q_bits, [k], [v], sm, round_p=False)[0, 0]
    assert abs(got[1] - 0.199609375) < 1e-7 and abs(unr[1] - 0.2) < 1e-7


# ------------------------------------------------------------ online == two-pass

@pytest.mark.parametrize("mode", ["K8V8", "K16V8", "BF16", "K8V16"])
@pytest.mark.parametrize("tile,split", [(16, 64), (64, 64), (64, 256), (7, 30), (64, 10000)])
def test_online_split_equals_two_pass(mode, tile, split):
    q_bits, ks, vs = _inputs(5, b=1, hq=8, hkv=1, d=32, t=300)
    store = oracle.store_rows(mode, ks[0], vs[0])
    view = {k: a[:, 0] for k, a in store.items()}
    rows = q_bits[0]
    for n_valid in ([300] * 8, [0, 1, 2, 63, 64, 65, 299, 300]):
        two = oracle.attend_rows(mode, rows, view, n_valid, 0.17)
        on, pacc, pl, pm = oracle.attend_rows_online(mode, rows, view, n_valid, 0.17,
                                                     tile, split)
        np.testing.assert_allclose(on, two, rtol=1e-12, atol=1e-13)
        # merging the partials by hand reproduces the output
        with np.errstate(invalid="ignore"):
            mstar = np.max(np.where(np.isfinite(pm), pm, -np.inf), axis=0)
            w = np.where(np.isfinite(pm), np.exp2(pm - mstar), 0.0)
        lsum = (w * pl).sum(axis=0)
        acc = (w[..., None] * pacc).sum(axis=0)
        merged = np.where(lsum[:, None] > 0, acc / np.where(lsum > 0, lsum, 1)[:, None], 0)
        np.testing.assert_allclose(merged, two, rtol=1e-12, atol=1e-13)
        # references are integers; empty splits carry M = -inf and l = 0
        fin = np.isfinite(pm)
        assert np.all(pm[fin] == np.round(pm[fin]))
        assert np.all(pl[~fin] == 0)


# ------------------------------------------------------------ prefill

def brute_prefill(mode, q_bits, k, v, q_pos0, sm):
    lq, hq, d = q_bits.shape
    hkv = k.shape[1]
    g = hq // hkv
    kd, vd = _deq(mode, oracle.store_rows(mode, k, v))
    q = oracle.bf16_value(q_bits)
    out = np.zeros((lq, hq, d))
    for i in range(lq):
        n = min(q_pos0 + i + 1, k.shape[0])
        for h in range(hq):
            s = kd[:n, h // g] @ q[i, h] * float(np.float32(sm))
            out[i, h] = scipy.special.softmax(s) @ vd[:n, h // g]
    return out


@pytest.mark.parametrize("q_pos0", [0, 7])
@pytest.mark.parametrize("mode", ["K8V8", "BF16"])
def test_prefill_causal_equals_textbook(q_pos0, mode):
    rng = np.random.default_rng(13 + q_pos0)
    lkv, hq, hkv, d = 40, 4, 2, 16
    lq = lkv - q_pos0
    k = rng.standard_normal((lkv, hkv, d)).astype(np.float32)
    v = rng.standard_normal((lkv, hkv, d)).astype(np.float32)
    q_bits = oracle.bf16_round_f32(rng.standard_normal((lq, hq, d)).astype(np.float32))
    got = oracle.prefill(mode, q_bits, k, v, q_pos0, 0.25, round_p=False)
    ref = brute_prefill(mode, q_bits, k, v, q_pos0, 0.25)
    np.testing.assert_allclose(got, ref, rtol=1e-11, atol=1e-12)
    # with bf16 P the causal rows equal decode rows of the truncated sequence
    got_r = oracle.prefill(mode, q_bits, k, v, q_pos0, 0.25, rows=[0, lq - 1])
    for i in (0, lq - 1):
        n = q_pos0 + i + 1
        dec = oracle.decode(mode, q_bits[i][None], [k[:n]], [v[:n]], 0.25)[0]
        np.testing.assert_array_equal(got_r[i], dec)


# ------------------------------------------------------------ exactness facts

def test_bf16_times_e4m3_products_exact_in_fp32():
    """The fp8-kv-cache page's math section: bf16 x e4m3 products are exact
    in fp32 (8 + 4 significant bits), for products in the normal range."""
    bits = np.arange(1 << 16, dtype=np.uint32) << 16
    qv = bits.view(np.float32)
    qv = qv[np.isfinite(qv) & (np.abs(qv) < 2.0 ** 100) & (np.abs(qv) > 2.0 ** -100)]
    ev = oracle.e4m3_value(np.arange(256))
    ev = ev[np.isfinite(ev) & (ev != 0)].astype(np.float32)
    p32 = (qv[:, None] * ev[None, :]).astype(np.float64)
    p64 = qv.astype(np.float64)[:, None] * ev.astype(np.float64)[None, :]
    assert np.array_equal(p32, p64)


def test_scale_factorisation():
    """Q . (s K)^T = s (Q . K^T) for a per-row scale (hardware notes, CDNA 3)."""
    rng = np.random.default_rng(2)
    q = rng.standard_normal(128)
    kq = oracle.e4m3_value(rng.integers(0, 0x7E, size=(64, 128)))
    s = np.exp(rng.uniform(-20, 5, 64))
    a = (s[:, None] * kq) @ q
    b = s * (kq @ q)
    np.testing.assert_allclose(a, b, rtol=1e-13)


# ------------------------------------------------------------ negative controls

def _cfg2_like(seed=17, t=256):
    return _inputs(seed, b=2, hq=16, hkv=2, d=128, t=t)


def _decode_with(mode, q_bits, stores, sm):
    b_n, hq, d = q_bits.shape
    hkv = stores[0]["vs" if mode != "BF16" else "v16"].shape[1]
    g = hq // hkv
    out = np.zeros((b_n, hq, d))
    for b in range(b_n):
        for h in range(hkv):
            view = {k: np.ascontiguousarray(a[:, h]) for k, a in stores[b].items()}
            n = view["v8"].shape[0]
            out[b, h * g:(h + 1) * g] = oracle.attend_rows(
                mode, q_bits[b, h * g:(h + 1) * g], view, n, sm)
    return out


def test_negative_controls_fail_gate():
    q_bits, ks, vs = _cfg2_like()
    sm = 1 / math.sqrt(128)
    stores = [oracle.store_rows("K8V8", k, v) for k, v in zip(ks, vs)]
    good = _decode_with("K8V8", q_bits, stores, sm)
    np.testing.assert_allclose(good, oracle.decode("K8V8", q_bits, ks, vs, sm), rtol=0, atol=0)

    bad = [dict(s, vs=(s["vs"] * np.float32(1.05)).astype(np.float32)) for s in stores]
    assert oracle.rel_l2(_decode_with("K8V8", q_bits, bad, sm), good) > GATE_REL

    one = [dict(s, ks=np.broadcast_to(s["ks"][:1], s["ks"].shape).copy(),
                vs=np.broadcast_to(s["vs"][:1], s["vs"].shape).copy()) for s in stores]
    assert oracle.rel_l2(_decode_with("K8V8", q_bits, one, sm), good) > GATE_REL

    # block table off by one: the second 16-token block reads the third
    def shift(a):
        a = a.copy()
        a[16:32] = a[32:48]
        return a
    off = [{k: shift(a) for k, a in s.items()} for s in stores]
    assert oracle.rel_l2(_decode_with("K8V8", q_bits, off, sm), good) > GATE_REL


def test_fp8_error_is_reported_in_expected_range():
    q_bits, ks, vs = _cfg2_like(t=128)
    sm = 1 / math.sqrt(128)
    e8 = oracle.fp8_kv_error(q_bits, ks, vs, sm, "K8V8")
    e16 = oracle.fp8_kv_error(q_bits, ks, vs, sm, "K16V8")
    assert 0.005 < e8 < 0.2 and 0.001 < e16 < e8
    assert oracle.fp8_kv_error(q_bits, ks, vs, sm, "BF16") == 0.0


# ------------------------------------------------------------ rounding bounds

def _fp32_attention(mode, q_bits, k, v, sm):
    """An independent fp32 computation of the method (numpy fp32 BLAS dot
    products, fp32 scale products and exp2, torch bf16 rounding of P): the
    kind of result a GPU produces."""
    import torch
    store = oracle.store_rows(mode, k, v)
    b_k = (oracle.e4m3_value(store["k8"]) if _K8[mode]
           else oracle.bf16_value(store["k16"])).astype(np.float32)
    b_v = (oracle.e4m3_value(store["v8"]) if _V8[mode]
           else oracle.bf16_value(store["v16"])).astype(np.float64)
    ks = store["ks"] if _K8[mode] else np.ones(k.shape[:2], np.float32)
    vs = store["vs"] if _V8[mode] else np.ones(k.shape[:2], np.float32)
    q = oracle.bf16_value(q_bits).astype(np.float32)
    hq, hkv = q.shape[0], k.shape[1]
    g = hq // hkv
    c = np.float32(np.float32(sm) * np.float32(1.4426950408889634))
    out = np.zeros(q.shape)
    for h in range(hq):
        kh = h // g
        s = (b_k[:, kh] @ q[h]).astype(np.float32)             # fp32 BLAS dot
        s = (s * ks[:, kh]).astype(np.float32) * c
        m = np.float32(np.ceil(s.max()))
        p = np.exp2((s - m).astype(np.float32)).astype(np.float32)
        w = (p * vs[:, kh]).astype(np.float32)
        pt = torch.from_numpy(w).to(torch.bfloat16).to(torch.float64).numpy()
        out[h] = (pt[:, None] * b_v[:, kh]).sum(0) / p.astype(np.float64).sum()
    return out


@pytest.mark.parametrize("mode", ["K8V8", "K16V8", "BF16", "K8V16"])
def test_rounding_bounds_contain_an_fp32_computation(mode):
    """[lo, hi] holds every output reachable by rounding an ambiguous P either
    way, so an independent fp32 computation must land inside it (up to the
    smooth fp32 change of p, ~1e-6).  The explicit tie case is
    test_rounding_bounds_at_a_bf16_midpoint."""
    q_bits, ks, vs = _inputs(31, b=6, hq=16, hkv=2, d=128, t=40)
    sm = float(np.float32(1 / math.sqrt(128)))
    out, lo, hi = oracle.decode(mode, q_bits, ks, vs, sm, bounds=True)
    assert np.all(lo <= out) and np.all(out <= hi)
    # the window is the worst-case fp32 summation bound: a few 1e-3 at most
    assert oracle.rel_l2(hi, lo) < 5e-3
    assert np.count_nonzero(hi > lo) > 0.1 * hi.size   # ambiguous P do occur
    for b in range(q_bits.shape[0]):
        o32 = _fp32_attention(mode, q_bits[b], ks[b], vs[b], sm)
        slack = 2e-6 * (np.abs(out[b]) + 0.1)
        assert np.all(o32 >= lo[b] - slack) and np.all(o32 <= hi[b] + slack)


def test_rounding_bounds_collapse_without_rounding():
    q_bits, ks, vs = _inputs(32, b=1, hq=4, hkv=1, d=32, t=20)
    out, lo, hi = oracle.decode("K8V8", q_bits, ks, vs, 0.2, round_p=False, bounds=True)
    assert np.array_equal(lo, out) and np.array_equal(hi, out)


def test_rounding_bounds_at_a_bf16_midpoint():
    """v_scale = 1 + 2^-8 is the midpoint between bf16 1 and 1 + 2^-7; with
    p = 1 both roundings are valid, so the bounds span V and V (1 + 2^-7)."""
    k = np.zeros((1, 1, 64), np.float32)
    v = np.zeros((1, 1, 64), np.float32)
    v[0, 0, 0] = 449.75                      # amax / 448 = 1 + 2^-8 exactly
    q_bits = oracle.bf16_round_f32(np.zeros((1, 1, 64), np.float32))  # s = 0, p = 1
    out, lo, hi = oracle.decode("K16V8", q_bits, [k], [v], 0.1, bounds=True)
    assert out[0, 0, 0] == 448.0             # ties to even: P = 1
    assert lo[0, 0, 0] == 448.0 and hi[0, 0, 0] == 448.0 * (1 + 2 ** -7)
