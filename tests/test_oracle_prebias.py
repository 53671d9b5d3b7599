"""Pins of the oracle's pre-bias residual K path (CPU only).

Hardware notes, "Treat numerical safety and kernel speed as separate gates",
and the fused-quantisation README, "Bias-aware symmetric FP8": quantise the
pre-bias K residual, keep the fixed K bias exact, apply the equivalent
score-space correction.  The stored rows are the residual r_t; the key is
r_t + b; the score is ((q . r_t) k_scale_t + q . b) sm_scale log2(e).

* A zero bias gives the bias-free result bit for bit.
* Textbook fp64 softmax on the reconstructed keys (dequantised residual +
  bias) equals the oracle with unrounded P.
* q . b is one constant per query row: with unrounded P the output equals
  the bias-free output on the same residual rows (softmax ignores a row
  constant), while the bf16 rounding of P does see it.  A bias applied per
  token (scaled by k_scale, say) fails the first check.
* Online (tiles, splits, merge) equals two-pass with the bias.
* On the biased-key workload the pre-bias K8V8 error against the BF16 cache
  of the full keys is far below the post-bias K8V8 error.
"""
import numpy as np
import pytest
import scipy.special

import oracle
from fp8_kv_cache_append_amd import synth
from test_oracle_attention import _deq

MODES = ["K8V8", "K16V8", "BF16", "K8V16"]


def _biased(seed, b=2, hq=8, hkv=2, t=80):
    lens = np.full(b, t, np.int32)
    w = synth.Workload("t", b, hq, hkv, 128, lens, "bias", seed=seed)
    parts = [synth.kv_sequence_prebias(w, i) for i in range(b)]
    q_bits = synth.q_bf16_bits(seed, (b, hq, 128))
    return w, q_bits, [p[0] for p in parts], [p[1] for p in parts], parts[0][2]


@pytest.mark.parametrize("mode", MODES)
def test_zero_bias_is_the_bias_free_path(mode):
    w, q_bits, ks, vs, bias = _biased(1)
    plain = oracle.decode(mode, q_bits, ks, vs, w.sm_scale)
    zero = oracle.decode(mode, q_bits, ks, vs, w.sm_scale, k_bias=np.zeros_like(bias))
    assert np.array_equal(plain, zero)


@pytest.mark.parametrize("mode", MODES)
def test_unrounded_equals_textbook_on_reconstructed_keys(mode):
    w, q_bits, ks, vs, bias = _biased(2)
    g = w.group
    q = oracle.bf16_value(q_bits)
    want = np.zeros(q_bits.shape)
    for b in range(w.batch):
        kr, v = _deq(mode, oracle.store_rows(mode, ks[b], vs[b]))
        for h in range(w.q_heads):
            key = kr[:, h // g] + bias[h // g].astype(np.float64)
            s = key @ q[b, h] * float(np.float32(w.sm_scale))
            want[b, h] = scipy.special.softmax(s) @ v[:, h // g]
    got = oracle.decode(mode, q_bits, ks, vs, w.sm_scale, round_p=False, k_bias=bias)
    assert oracle.rel_l2(got, want) < 1e-12


@pytest.mark.parametrize("mode", ["K8V8", "K16V8"])
def test_bias_is_a_row_constant_of_the_score(mode):
    w, q_bits, ks, vs, bias = _biased(3)
    free_u = oracle.decode(mode, q_bits, ks, vs, w.sm_scale, round_p=False)
    bias_u = oracle.decode(mode, q_bits, ks, vs, w.sm_scale, round_p=False, k_bias=bias)
    assert oracle.rel_l2(bias_u, free_u) < 1e-12
    free_r = oracle.decode(mode, q_bits, ks, vs, w.sm_scale)
    bias_r = oracle.decode(mode, q_bits, ks, vs, w.sm_scale, k_bias=bias)
    assert 0 < oracle.rel_l2(bias_r, free_r) < 1e-2   # only through the rounding of P


@pytest.mark.parametrize("tile,split", [(64, 256), (16, 48)])
def test_online_equals_two_pass_with_bias(tile, split):
    w, q_bits, ks, vs, bias = _biased(4, b=1, hq=8, hkv=1, t=300)
    store = oracle.store_rows("K8V8", ks[0], vs[0])
    view = {k: np.ascontiguousarray(a[:, 0]) for k, a in store.items()}
    n_valid = np.array([300, 299, 1, 0, 64, 65, 200, 17], np.int32)
    two = oracle.attend_rows("K8V8", q_bits[0], view, n_valid, w.sm_scale, k_bias=bias[0])
    on, _, _, _ = oracle.attend_rows_online("K8V8", q_bits[0], view, n_valid, w.sm_scale,
                                            tile, split, k_bias=bias[0])
    assert oracle.rel_l2(on, two) < 1e-12


def test_pre_bias_repairs_the_biased_key_error():
    """The biased-key workload: K = N(0,1) + 20 on 8 channels.  Post-bias
    K8V8 error against the BF16 cache of the full keys is ~0.1 (the bias
    sets the scale and crushes the residual); pre-bias K8V8 is at the
    format's usual level."""
    w, q_bits, ks, vs, bias = _biased(5, b=2, hq=32, hkv=8, t=512)
    full = [k + bias[None] for k in ks]
    ref = oracle.decode("BF16", q_bits, full, vs, w.sm_scale)
    post = oracle.rel_l2(oracle.decode("K8V8", q_bits, full, vs, w.sm_scale), ref)
    pre = oracle.rel_l2(oracle.decode("K8V8", q_bits, ks, vs, w.sm_scale, k_bias=bias), ref)
    print(f"biased keys vs BF16: post-bias K8V8 {post:.4f}, pre-bias K8V8 {pre:.4f}")
    assert post > 0.05
    assert pre < post / 2
