"""GPU parity of the block-scaled K cache (FP8KV_MXK8V8) against the oracle.

* fp8kv_append writes the oracle's bytes: e4m3 codes and one E8M0 byte per
  32-value K block (the MXK8V8 rule), V as in K8V8; bit-exact.
* fp8kv_decode (bf16 Q; K codes converted by their block's power-of-two
  scale, exactly) meets the main gate (test_gpu_decode._gate).
* fp8kv_decode_q8 (block-scaled QK: Q quantised per 32-value block, the
  matrix instruction applies both operands' block scales) meets the narrow
  gates of test_gpu_decode_q8: exact on one-hot keys, the derived bar on
  general inputs.
* The entry points that do not take such a cache reject it.
"""
import numpy as np
import pytest
import torch

import oracle
from fp8_kv_cache_append_amd import binding, synth
from gpu_util import DEV, append_seq, decode, make_cache, q_tensor, read_rows
from test_gpu_decode import _gate
from test_gpu_decode_q8 import _narrow_gate, decode_q8

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("layout", ["token", "head"])
@pytest.mark.parametrize("d", [64, 128])
def test_mx_append_bytes_match_oracle(d, layout):
    rng = np.random.default_rng(d)
    n, hkv = 300, 2
    k = (rng.standard_normal((n, hkv, d)) * np.exp2(rng.integers(-30, 30, size=(n, hkv, 1)))
         ).astype(np.float32)
    k[3, 0, :32] = 0.0                        # a zero block
    k[4, 1, 5] *= 1000.0                      # an outlier
    k[5, 0, :] = np.float32(1e-39)            # subnormal values
    k[6, 1, 32:64] = np.float32(448.0)        # a block at exactly 448
    v = rng.standard_normal((n, hkv, d)).astype(np.float32)
    w = synth.Workload("t", 1, 2 * hkv, hkv, d, np.array([n], np.int32), "normal",
                       block_size=16, shuffle_blocks=True, seed=5)
    cache = make_cache("MXK8V8", w, layout=layout)
    append_seq(cache, 0, k, v)
    got = read_rows(cache, 0, n)
    want = oracle.store_rows("MXK8V8", k, v)
    for key in ("k8", "kx", "v8", "vs"):
        assert np.array_equal(got[key], want[key]), key


SHAPES = [
    # (q_heads, kv_heads, head_dim, lens, block_size)
    (16, 2, 128, [300, 0, 1, 64, 65, 257, 512, 1000], 0),
    (32, 8, 128, [700, 16, 1, 1024, 33], 16),
    (4, 1, 64, [128, 63], 16),
    (16, 1, 64, [129, 1500], 64),
]


def _filled(w, layout="token"):
    seqs = [synth.kv_sequence(w, b) for b in range(w.batch)]
    cache = make_cache("MXK8V8", w, layout=layout)
    for b, (k, v) in enumerate(seqs):
        append_seq(cache, b, k, v)
    q_bits = synth.q_bf16_bits(w.seed, (w.batch, w.q_heads, w.head_dim))
    return cache, seqs, q_bits


@pytest.mark.parametrize("layout", ["token", "head"])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: f"hq{s[0]}_hkv{s[1]}_d{s[2]}_bs{s[4]}")
def test_mx_decode_bf16_q(shape, layout):
    hq, hkv, d, lens, bs = shape
    lens = np.array(lens, np.int32)
    w = synth.Workload("t", len(lens), hq, hkv, d, lens, "outliers", block_size=bs,
                       shuffle_blocks=bs > 0, seed=hq + d + bs + 9)
    cache, seqs, q_bits = _filled(w, layout)
    got = decode(cache, q_bits, lens, w.group, w.sm_scale)
    ref, lo, hi = oracle.decode("MXK8V8", q_bits, [s[0] for s in seqs], [s[1] for s in seqs],
                                w.sm_scale, bounds=True)
    _gate(got, ref, lo, hi, ("MXK8V8", "bf16 Q", shape))


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: f"hq{s[0]}_hkv{s[1]}_d{s[2]}_bs{s[4]}")
def test_mx_decode_block_scaled_qk(shape):
    hq, hkv, d, lens, bs = shape
    lens = np.array(lens, np.int32)
    w = synth.Workload("t", len(lens), hq, hkv, d, lens, "outliers", block_size=bs,
                       shuffle_blocks=bs > 0, seed=hq + d + bs + 10)
    cache, seqs, q_bits = _filled(w)
    got = decode_q8(cache, q_bits, lens, w.group, w.sm_scale)
    _narrow_gate(got, "MXK8V8", q_bits, [s[0] for s in seqs], [s[1] for s in seqs], w.sm_scale,
                 ("MXK8V8", "block-scaled QK", shape))


@pytest.mark.parametrize("d", [64, 128])
def test_mx_block_scaled_qk_one_hot_keys_are_exact(d):
    """One nonzero K value per row, at d = (t + 5h) % D, spread over every
    block: each score is one exact product times two block scales, so the
    block-scaled instruction must match the oracle to fp32 precision."""
    hq, hkv, n = 16, 2, 300
    lens = np.array([n, 257, 64, 1], np.int32)
    w = synth.Workload("t", len(lens), hq, hkv, d, lens, "normal", block_size=16,
                       shuffle_blocks=True, seed=29 + d)
    rng = np.random.default_rng(d + 1)
    seqs = []
    for b in range(w.batch):
        k = np.zeros((int(lens[b]), hkv, d), np.float32)
        t = np.arange(int(lens[b]))
        for h in range(hkv):
            k[t, h, (t + 5 * h) % d] = (rng.standard_normal(t.size) * 3).astype(np.float32)
        v = rng.standard_normal((int(lens[b]), hkv, d)).astype(np.float32)
        seqs.append((k, v))
    q_bits = synth.q_bf16_bits(w.seed, (w.batch, w.q_heads, w.head_dim))
    cache = make_cache("MXK8V8", w)
    for b, (k, v) in enumerate(seqs):
        append_seq(cache, b, k, v)
    got = decode_q8(cache, q_bits, w.lens, w.group, w.sm_scale)
    ref, lo, hi = oracle.decode("MXK8V8", q_bits, [s[0] for s in seqs], [s[1] for s in seqs],
                                w.sm_scale, bounds=True, q8=True)
    _gate(got, ref, lo, hi, ("MXK8V8", "block-scaled QK, one-hot keys", d))


def test_mx_b16_t2048_errors_reported():
    """The benchmark shape: parity of both paths on sampled pairs, and each
    format's error against the BF16 cache (GPU against GPU)."""
    w = synth.decode_b16_gqa8_d128(2048)
    cache, seqs, q_bits = _filled(w)
    pairs = [(b, h) for b in (0, 9) for h in (0, 1)]
    got = decode(cache, q_bits, w.lens, w.group, w.sm_scale)
    ref, lo, hi = oracle.decode("MXK8V8", q_bits, [s[0] for s in seqs], [s[1] for s in seqs],
                                w.sm_scale, pairs=pairs, bounds=True)
    _gate(got, ref, lo, hi, ("MXK8V8", "b16 t2048"))
    full = make_cache("BF16", w)
    per_row = make_cache("K8V8", w)
    for b, (k, v) in enumerate(seqs):
        append_seq(full, b, k, v)
        append_seq(per_row, b, k, v)
    r = decode(full, q_bits, w.lens, w.group, w.sm_scale)
    e_row = oracle.rel_l2(decode(per_row, q_bits, w.lens, w.group, w.sm_scale), r)
    e_mx = oracle.rel_l2(got, r)
    e_mxq = oracle.rel_l2(decode_q8(cache, q_bits, w.lens, w.group, w.sm_scale), r)
    print(f"vs BF16 (GPU): K8V8 {e_row:.4f}  MXK8V8 bf16 Q {e_mx:.4f}  "
          f"MXK8V8 block-scaled QK {e_mxq:.4f}")
    assert e_mx < 3 * e_row


def test_mx_cache_rejected_where_unsupported():
    w = synth.Workload("t", 2, 8, 2, 128, np.array([10, 20], np.int32), "normal", seed=3)
    cache = make_cache("MXK8V8", w)
    q = q_tensor(synth.q_bf16_bits(1, (2, 8, 128)))
    lens = torch.tensor([10, 20], dtype=torch.int32, device=DEV)
    out = torch.empty((2, 8, 128), device=DEV)
    ws = torch.empty(binding.fp8kv_decode_workspace_bytes(cache, 2, 4, 20) // 4 + 4, device=DEV)
    kn = torch.zeros((2, 2, 128), device=DEV)
    with pytest.raises(binding.Fp8kvError) as e:
        binding.fp8kv_decode_append(cache, kn, kn, q, 4, lens, 20, w.sm_scale, out, ws)
    assert e.value.status == -4
    qp = q_tensor(synth.q_bf16_bits(1, (20, 8, 128)))
    with pytest.raises(binding.Fp8kvError) as e:
        binding.fp8kv_prefill(cache, qp, 4, torch.tensor([0, 20], dtype=torch.int32, device=DEV),
                              torch.zeros(1, dtype=torch.int32, device=DEV), lens[1:], 20,
                              w.sm_scale, torch.empty((20, 8, 128), device=DEV))
    assert e.value.status == -4
    dst = make_cache("BF16", w)
    with pytest.raises(binding.Fp8kvError) as e:
        binding.fp8kv_dequantize(cache, dst)
    assert e.value.status == -4
