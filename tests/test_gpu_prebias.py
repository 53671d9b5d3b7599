"""GPU parity of pre-bias residual caches (fp8kv_cache.k_bias) against the
oracle's bias path (oracle.decode(..., k_bias=...)).

The cache stores the residual rows r (appended by the ordinary fp8kv_append)
and the exact bias b; decode adds (q . b) * sm_scale * log2(e) to every
score of query row q.  Gate: the bf16 path's (test_gpu_decode._gate).  Also
the measured repair of the biased-key workload's error, the fused append on
such a cache, and the entry points that reject it.
"""
import numpy as np
import pytest
import torch

import oracle
from fp8_kv_cache_append_amd import binding, synth
from gpu_util import DEV, append_seq, decode, make_cache, q_tensor
from test_gpu_decode import _gate

pytestmark = pytest.mark.gpu


def _biased_cache(mode, w):
    parts = [synth.kv_sequence_prebias(w, b) for b in range(w.batch)]
    cache = make_cache(mode, w)
    for b, (r, v, _) in enumerate(parts):
        append_seq(cache, b, r, v)
    bias = parts[0][2]
    cache.k_bias = torch.from_numpy(bias).to(DEV)
    return cache, [p[0] for p in parts], [p[1] for p in parts], bias


SHAPES = [
    # (q_heads, kv_heads, head_dim, lens, block_size)
    (32, 8, 128, [700, 16, 1, 1024, 33], 16),
    (16, 2, 128, [300, 0, 1, 64, 65, 257, 512, 1000], 0),
    (4, 1, 64, [128, 63], 16),
]


@pytest.mark.parametrize("mode", ["K8V8", "K16V8", "BF16", "K8V16"])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: f"hq{s[0]}_hkv{s[1]}_d{s[2]}_bs{s[4]}")
def test_pre_bias_decode_matches_oracle(mode, shape):
    hq, hkv, d, lens, bs = shape
    lens = np.array(lens, np.int32)
    w = synth.Workload("t", len(lens), hq, hkv, d, lens, "bias", block_size=bs,
                       shuffle_blocks=bs > 0, seed=hq + d + bs + 2)
    cache, rs, vs, bias = _biased_cache(mode, w)
    q_bits = synth.q_bf16_bits(w.seed, (w.batch, w.q_heads, w.head_dim))
    got = decode(cache, q_bits, lens, w.group, w.sm_scale)
    ref, lo, hi = oracle.decode(mode, q_bits, rs, vs, w.sm_scale, bounds=True, k_bias=bias)
    _gate(got, ref, lo, hi, (mode, "pre-bias", shape))
    for b, n in enumerate(lens):
        if n == 0:
            assert np.all(got[b] == 0)


def test_pre_bias_repairs_biased_keys_on_gpu():
    """The biased-key workload (config 4's distribution), 8 sequences of 2048:
    against the BF16 cache of the full keys, post-bias K8V8 (the bias inside
    the quantised rows) and pre-bias K8V8 (residual rows + exact bias), all
    three on the GPU."""
    w = synth.Workload("t", 8, 32, 8, 128, np.full(8, 2048, np.int32), "bias", seed=4)
    q_bits = synth.q_bf16_bits(w.seed, (w.batch, w.q_heads, w.head_dim))
    full = make_cache("BF16", w)
    post = make_cache("K8V8", w)
    for b in range(w.batch):
        k, v = synth.kv_sequence(w, b)
        append_seq(full, b, k, v)
        append_seq(post, b, k, v)
    pre, _, _, _ = _biased_cache("K8V8", w)
    ref = decode(full, q_bits, w.lens, w.group, w.sm_scale)
    e_post = oracle.rel_l2(decode(post, q_bits, w.lens, w.group, w.sm_scale), ref)
    e_pre = oracle.rel_l2(decode(pre, q_bits, w.lens, w.group, w.sm_scale), ref)
    print(f"biased keys vs BF16 (GPU): post-bias K8V8 {e_post:.4f}, pre-bias K8V8 {e_pre:.4f}")
    assert e_post > 0.05 and e_pre < e_post / 2


@pytest.mark.parametrize("mode", ["K8V8", "K16V8"])
def test_pre_bias_fused_append_step(mode):
    """fp8kv_decode_append on a pre-bias cache: k_new is the new token's
    residual; same cache bytes as fp8kv_append, bit-identical output to
    fp8kv_decode, and the oracle gate."""
    lens = np.array([1, 64, 65, 700], np.int32)
    w = synth.Workload("t", len(lens), 32, 8, 128, lens, "bias", block_size=16,
                       shuffle_blocks=True, seed=31)
    parts = [synth.kv_sequence_prebias(w, b) for b in range(w.batch)]
    bias = torch.from_numpy(parts[0][2]).to(DEV)
    fused, plain = make_cache(mode, w), make_cache(mode, w)
    fused.k_bias = plain.k_bias = bias
    k_new = np.zeros((w.batch, w.kv_heads, w.head_dim), np.float32)
    v_new = np.zeros_like(k_new)
    for b, (r, v, _) in enumerate(parts):
        n = int(lens[b])
        append_seq(fused, b, r[:n - 1], v[:n - 1])
        append_seq(plain, b, r[:n], v[:n])
        k_new[b], v_new[b] = r[n - 1], v[n - 1]
    q_bits = synth.q_bf16_bits(w.seed, (w.batch, w.q_heads, w.head_dim))
    max_len = int(lens.max())
    ws = torch.empty(binding.fp8kv_decode_workspace_bytes(fused, w.batch, w.group, max_len) // 4
                     + 4, device=DEV)
    out = torch.full((w.batch, w.q_heads, w.head_dim), float("nan"), device=DEV)
    binding.fp8kv_decode_append(fused, torch.from_numpy(k_new).to(DEV),
                                torch.from_numpy(v_new).to(DEV), q_tensor(q_bits), w.group,
                                torch.from_numpy(lens).to(DEV), max_len, w.sm_scale, out, ws)
    got = out.cpu().numpy()
    want = decode(plain, q_bits, lens, w.group, w.sm_scale)
    for x, y in ((fused.k, plain.k), (fused.v, plain.v), (fused.k_scale, plain.k_scale),
                 (fused.v_scale, plain.v_scale)):
        assert (x is None and y is None) or torch.equal(x, y)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))
    ref, lo, hi = oracle.decode(mode, q_bits, [p[0] for p in parts], [p[1] for p in parts],
                                w.sm_scale, bounds=True, k_bias=parts[0][2])
    _gate(got, ref, lo, hi, (mode, "pre-bias fused append"))


def test_pre_bias_cache_rejected_by_prefill_and_narrow_qk():
    w = synth.Workload("t", 2, 8, 2, 128, np.array([10, 20], np.int32), "bias", seed=3)
    cache, _, _, _ = _biased_cache("K8V8", w)
    q = q_tensor(synth.q_bf16_bits(1, (2, 8, 128)))
    lens = torch.tensor([10, 20], dtype=torch.int32, device=DEV)
    out = torch.empty((2, 8, 128), device=DEV)
    ws = torch.empty(binding.fp8kv_decode_workspace_bytes(cache, 2, 4, 20) // 4 + 4, device=DEV)
    with pytest.raises(binding.Fp8kvError) as e:
        binding.fp8kv_decode_q8(cache, q, 4, lens, 20, w.sm_scale, out, ws)
    assert e.value.status == -4
    qp = q_tensor(synth.q_bf16_bits(1, (20, 8, 128)))
    with pytest.raises(binding.Fp8kvError) as e:
        binding.fp8kv_prefill(cache, qp, 4, torch.tensor([0, 20], dtype=torch.int32, device=DEV),
                              torch.zeros(1, dtype=torch.int32, device=DEV), lens[1:], 20,
                              w.sm_scale, torch.empty((20, 8, 128), device=DEV))
    assert e.value.status == -4
