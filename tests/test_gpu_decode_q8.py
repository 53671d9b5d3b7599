"""GPU parity of narrow QK (fp8kv_decode_q8, fp8kv_decode_append_q8) against
the oracle's narrow path (oracle.decode(..., q8=True)).

The query rows are quantised inside the split kernel by the cache-row rule
and QK runs on the fp8 matrix instruction; the oracle quantises Q with its
own encoder and computes the scores exactly (fp64).

The instruction does not return the correctly rounded fp32 sum of its 128
code products: its sum is unbiased but only good to about 2^-13 of the
absolute sum of the products (measured on gfx950).  That noise moves scores
by ~1e-3 of their size on rows with outliers or biased channels, and through
the bf16 rounding of P the outputs by up to ~1.5e-3 relative L2 from the
exact narrow result (48-case sweep over the three value distributions).
Two gates follow from that:

* one-hot keys (one nonzero code per K row, at every d in turn): the
  instruction sums a single product, exactly, so the result must match the
  oracle to fp32 precision (the bf16 path's gate, rel <= 1e-4).  This pins
  the in-kernel Q codes of every d, the pairing of Q and K bytes in the
  operands and the scale application;
* general inputs: every element inside the oracle's P-rounding interval,
  which on the narrow path also allows the instruction's sum error (up to
  fp32 slack, and the contract's 5e-3 max-abs outside it), and rel L2
  against the exact narrow result at most 1e-3 plus twice the case's own
  P-rounding effect (the oracle with rounded against unrounded P): a flip
  moves one P by one bf16 step, so all flips together move the output by
  about twice the rounding effect at most, and 1e-3 covers the direct score
  noise.  (Sweep of 48 seeded cases: worst 1.5e-3 against a bar of 4-5e-3.)

The error the Q rounding itself adds against bf16 Q is printed, not gated.
"""
import numpy as np
import pytest
import torch

import oracle
from fp8_kv_cache_append_amd import binding, synth
from gpu_util import DEV, append_seq, check_layout, decode, make_cache, q_tensor
from test_gpu_decode import SHAPES, _gate

pytestmark = pytest.mark.gpu

NARROW_MODES = ["K8V8", "K8V16"]


def _narrow_gate(got, mode, q_bits, k_seqs, v_seqs, sm_scale, ctx, pairs=None):
    """The general-input gate of the module docstring."""
    ref, lo, hi = oracle.decode(mode, q_bits, k_seqs, v_seqs, sm_scale, pairs=pairs,
                                bounds=True, q8=True)
    unr = oracle.decode(mode, q_bits, k_seqs, v_seqs, sm_scale, pairs=pairs, round_p=False,
                        q8=True)
    ok = ~np.isnan(ref)
    bar = 1e-3 + 2.0 * oracle.rel_l2(ref[ok], unr[ok])
    print(f"{ctx}: narrow bar rel_l2 <= {bar:.2e}", flush=True)
    _gate(got, ref, lo, hi, ctx, expect_rel=bar, gate_rel=bar)


def decode_q8(cache, q_bits, lens, group, sm_scale):
    lens = np.asarray(lens, np.int32)
    b, hq, d = q_bits.shape
    check_layout(cache.block_table.cpu().numpy(), cache.block_size, lens)
    max_len = int(lens.max()) if b else 0
    ws = torch.empty(max(binding.fp8kv_decode_workspace_bytes(cache, b, group, max_len) // 4, 4),
                     dtype=torch.float32, device=DEV)
    out = torch.full((b, hq, d), float("nan"), dtype=torch.float32, device=DEV)
    binding.fp8kv_decode_q8(cache, q_tensor(q_bits), group, torch.from_numpy(lens).to(DEV),
                            max_len, sm_scale, out, ws)
    return out.cpu().numpy()


def _case(mode, w, with_cache=False, layout="token"):
    seqs = [synth.kv_sequence(w, b) for b in range(w.batch)]
    q_bits = synth.q_bf16_bits(w.seed, (w.batch, w.q_heads, w.head_dim))
    cache = make_cache(mode, w, layout=layout)
    for b, (k, v) in enumerate(seqs):
        append_seq(cache, b, k, v)
    got = decode_q8(cache, q_bits, w.lens, w.group, w.sm_scale)
    return (got, seqs, q_bits, cache) if with_cache else (got, seqs, q_bits)


@pytest.mark.parametrize("layout", ["token", "head"])
@pytest.mark.parametrize("mode", NARROW_MODES)
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: f"hq{s[0]}_hkv{s[1]}_d{s[2]}_bs{s[4]}")
def test_narrow_decode_small_shapes(mode, shape, layout):
    hq, hkv, d, lens, bs = shape
    lens = np.array(lens, np.int32)
    w = synth.Workload("t", len(lens), hq, hkv, d, lens, "outliers", block_size=bs,
                       shuffle_blocks=bs > 0, seed=hq * 7 + d + bs + 1)
    got, seqs, q_bits = _case(mode, w, layout=layout)
    _narrow_gate(got, mode, q_bits, [s[0] for s in seqs], [s[1] for s in seqs], w.sm_scale,
                 (mode, "narrow", shape))
    for b, n in enumerate(lens):
        if n == 0:
            assert np.all(got[b] == 0)


@pytest.mark.parametrize("mode", NARROW_MODES)
def test_narrow_decode_b16_t2048(mode):
    """The benchmark shape, sampled (sequence, KV head) pairs; also prints
    the error the Q rounding adds against the bf16-Q kernel."""
    w = synth.decode_b16_gqa8_d128(2048)
    pairs = [(b, h) for b in (0, 7, 15) for h in (0, 1)]
    got, seqs, q_bits, cache = _case(mode, w, with_cache=True)
    _narrow_gate(got, mode, q_bits, [s[0] for s in seqs], [s[1] for s in seqs], w.sm_scale,
                 (mode, "narrow b16 t2048"), pairs)
    wide = decode(cache, q_bits, w.lens, w.group, w.sm_scale)
    print(f"{mode}: narrow QK vs bf16-Q kernel rel_l2 = {oracle.rel_l2(got, wide):.4f}")


@pytest.mark.parametrize("mode", NARROW_MODES)
def test_narrow_decode_b64_ragged_sampled(mode):
    """Ragged paged batch of 16 sequences of the config-4 kind (biased keys,
    shuffled 16-token blocks, lengths up to 6000), sampled pairs."""
    rng = np.random.default_rng(9)
    lens = rng.integers(1, 6000, size=16).astype(np.int32)
    w = synth.Workload("t", 16, 32, 8, 128, lens, "bias", block_size=16, shuffle_blocks=True,
                       seed=4)
    pairs = [(0, 0), (3, 5), (9, 7), (15, 2)]
    got, seqs, q_bits = _case(mode, w)
    _narrow_gate(got, mode, q_bits, [s[0] for s in seqs], [s[1] for s in seqs], w.sm_scale,
                 (mode, "narrow ragged"), pairs)


@pytest.mark.parametrize("mode", NARROW_MODES)
def test_narrow_append_step_equals_append_then_decode(mode):
    """fp8kv_decode_append_q8 stores the new token exactly as fp8kv_append
    and its output is bit-identical to fp8kv_decode_q8 over that cache."""
    lens = np.array([1, 64, 65, 300, 1000], np.int32)
    w = synth.Workload("t", len(lens), 16, 2, 128, lens, "outliers", block_size=16,
                       shuffle_blocks=True, seed=17)
    seqs = [synth.kv_sequence(w, b) for b in range(w.batch)]
    q_bits = synth.q_bf16_bits(w.seed, (w.batch, w.q_heads, w.head_dim))
    fused, plain = make_cache(mode, w), make_cache(mode, w)
    k_new = np.zeros((w.batch, w.kv_heads, w.head_dim), np.float32)
    v_new = np.zeros_like(k_new)
    for b, (k, v) in enumerate(seqs):
        n = int(lens[b])
        append_seq(fused, b, k[:n - 1], v[:n - 1])
        append_seq(plain, b, k[:n], v[:n])
        k_new[b], v_new[b] = k[n - 1], v[n - 1]
    max_len = int(lens.max())
    ws = torch.empty(binding.fp8kv_decode_workspace_bytes(fused, w.batch, w.group, max_len) // 4
                     + 4, device=DEV)
    out = torch.full((w.batch, w.q_heads, w.head_dim), float("nan"), device=DEV)
    binding.fp8kv_decode_append_q8(fused, torch.from_numpy(k_new).to(DEV),
                                   torch.from_numpy(v_new).to(DEV), q_tensor(q_bits), w.group,
                                   torch.from_numpy(lens).to(DEV), max_len, w.sm_scale, out, ws)
    got = out.cpu().numpy()
    want = decode_q8(plain, q_bits, lens, w.group, w.sm_scale)
    for x, y in ((fused.k, plain.k), (fused.v, plain.v), (fused.k_scale, plain.k_scale),
                 (fused.v_scale, plain.v_scale)):
        assert (x is None and y is None) or torch.equal(x, y)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))
    _narrow_gate(got, mode, q_bits, [s[0] for s in seqs], [s[1] for s in seqs], w.sm_scale,
                 (mode, "narrow fused append"))


@pytest.mark.parametrize("mode", ["K16V8", "BF16"])
def test_narrow_qk_rejects_bf16_keys(mode):
    w = synth.Workload("t", 2, 8, 2, 128, np.array([10, 20], np.int32), "normal", seed=3)
    cache = make_cache(mode, w)
    q = q_tensor(synth.q_bf16_bits(1, (2, 8, 128)))
    out = torch.empty((2, 8, 128), device=DEV)
    ws = torch.empty(binding.fp8kv_decode_workspace_bytes(cache, 2, 4, 20) // 4 + 4, device=DEV)
    with pytest.raises(binding.Fp8kvError) as e:
        binding.fp8kv_decode_q8(cache, q, 4, torch.tensor([10, 20], dtype=torch.int32,
                                                          device=DEV), 20, w.sm_scale, out, ws)
    assert e.value.status == -4


@pytest.mark.parametrize("mode", NARROW_MODES)
@pytest.mark.parametrize("d", [64, 128])
def test_narrow_one_hot_keys_are_exact(mode, d):
    """K row t of head h holds one nonzero value, at d = (t + 5h) % D, so each
    score is one exact code product times the scales: every query element's
    code meets a key, and a wrong code, a mispaired operand byte or a
    misapplied scale moves the output far past the fp32-level gate."""
    hq, hkv, n = 16, 2, 300
    lens = np.array([n, 257, 64, 1], np.int32)
    w = synth.Workload("t", len(lens), hq, hkv, d, lens, "normal", block_size=16,
                       shuffle_blocks=True, seed=23 + d)
    rng = np.random.default_rng(d)
    seqs = []
    for b in range(w.batch):
        k = np.zeros((int(lens[b]), hkv, d), np.float32)
        t = np.arange(int(lens[b]))
        for h in range(hkv):
            k[t, h, (t + 5 * h) % d] = rng.standard_normal(t.size).astype(np.float32) * 3
        v = rng.standard_normal((int(lens[b]), hkv, d)).astype(np.float32)
        seqs.append((k, v))
    q_bits = synth.q_bf16_bits(w.seed, (w.batch, w.q_heads, w.head_dim))
    cache = make_cache(mode, w)
    for b, (k, v) in enumerate(seqs):
        append_seq(cache, b, k, v)
    got = decode_q8(cache, q_bits, w.lens, w.group, w.sm_scale)
    ref, lo, hi = oracle.decode(mode, q_bits, [s[0] for s in seqs], [s[1] for s in seqs],
                                w.sm_scale, bounds=True, q8=True)
    _gate(got, ref, lo, hi, (mode, "narrow one-hot keys", d))
