"""GPU tests of decode plans with one split per (sequence, KV head).

With one split the merge is a division of the split's accumulator by its row
sum, so fp8kv_decode (and the entry points built on it) lets the split kernel
write the output rows and launches no merge kernel.  The output must equal
the two-kernel form, fp8kv_decode_partial with the same plan followed by
fp8kv_decode_merge, bit for bit: with empty and one-key sequences, and with
a value column that is -0 in every key (whose accumulator is -0, which the
merge turns into +0).
"""
import numpy as np
import pytest
import torch

import oracle
from fp8_kv_cache_append_amd import binding, synth
from gpu_util import DEV, append_seq, decode, make_cache, q_tensor
from test_gpu_decode import _gate

pytestmark = pytest.mark.gpu

CASES = [
    # mode, batch, q heads, KV heads, head_dim, lengths, block size
    ("K8V8", 1, 4, 1, 64, [128], 0),                  # config 1's shape
    ("K8V8", 16, 16, 2, 128, [77] * 16, 0),           # the 77-key context sweep
    ("BF16", 3, 8, 2, 128, [100, 0, 1], 16),          # an empty and a one-key sequence
    ("K16V8", 2, 32, 8, 64, [128, 64], 16),
    ("K8V16", 4, 8, 4, 128, [50, 128, 3, 0], 32),
]


def _two_kernels(cache, q_bits, lens, group, sm_scale, chunk, splits):
    b, hq, d = q_bits.shape
    hkv = cache.num_kv_heads
    pacc = torch.full((b, hkv, splits, group, d), float("nan"), device=DEV)
    pml = torch.full((b, hkv, splits, group, 2), float("nan"), device=DEV)
    out = torch.full((b, hq, d), float("nan"), device=DEV)
    lens_t = torch.from_numpy(np.asarray(lens, np.int32)).to(DEV)
    binding.fp8kv_decode_partial(cache, q_tensor(q_bits), group, lens_t, int(max(lens)),
                                 sm_scale, chunk, splits, pacc, pml)
    binding.fp8kv_decode_merge(b, hkv, group, d, splits, pacc, pml, out)
    return out.cpu().numpy()


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[0]}_b{c[1]}_hq{c[2]}_d{c[4]}")
def test_single_split_matches_merge_kernel(case):
    mode, batch, hq, hkv, d, lens, bs = case
    lens = np.asarray(lens, np.int32)
    w = synth.Workload("one_split", batch, hq, hkv, d, lens, "outliers", block_size=bs,
                       shuffle_blocks=bs > 0, seed=hq + d + batch)
    cache = make_cache(mode, w)
    seqs = []
    for b in range(batch):
        k, v = synth.kv_sequence(w, b)
        if b == 0 and len(k):
            v = v.copy()
            v[:, :, 5] = -0.0    # a value column of -0 in every key
        seqs.append((k, v))
        if lens[b]:
            append_seq(cache, b, k[:lens[b]], v[:lens[b]])
    chunk, splits = binding.fp8kv_decode_plan(cache, batch, w.group, int(lens.max()))
    assert splits == 1, (case, chunk, splits)
    q_bits = synth.q_bf16_bits(w.seed + 3, (batch, hq, d))
    got = decode(cache, q_bits, lens, w.group, w.sm_scale)
    want = _two_kernels(cache, q_bits, lens, w.group, w.sm_scale, chunk, splits)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), case
    if lens[0]:
        assert np.all(got[0, :, 5].view(np.uint32) == 0), "the -0 column must come out as +0"
    ref, lo, hi = oracle.decode(mode, q_bits, [s[0][:n] for s, n in zip(seqs, lens)],
                                [s[1][:n] for s, n in zip(seqs, lens)], w.sm_scale, bounds=True)
    _gate(got, ref, lo, hi, case)


@pytest.mark.parametrize("mode", ["K8V8", "K8V16"])
def test_single_split_narrow_qk(mode):
    """Narrow QK (fp8kv_decode_q8) on plans of one split runs the split kernel
    alone as well: its output meets the narrow-QK gate against the oracle's
    narrow path, and the fused-append form (fp8kv_decode_append_q8) is
    bit-identical to fp8kv_append followed by fp8kv_decode_q8."""
    from test_gpu_decode_q8 import _narrow_gate, decode_q8
    lens = np.array([77, 128, 5, 0], np.int32)
    w = synth.Workload("one_split_q8", 4, 16, 2, 128, lens, "outliers", block_size=16,
                       shuffle_blocks=True, seed=41)
    fused, plain = make_cache(mode, w), make_cache(mode, w)
    seqs = [synth.kv_sequence(w, b) for b in range(w.batch)]
    k_new = np.zeros((w.batch, w.kv_heads, w.head_dim), np.float32)
    v_new = np.zeros_like(k_new)
    for b, (k, v) in enumerate(seqs):
        n = int(lens[b])
        if n:
            append_seq(fused, b, k[:n - 1], v[:n - 1])
            append_seq(plain, b, k[:n], v[:n])
            k_new[b], v_new[b] = k[n - 1], v[n - 1]
    chunk, splits = binding.fp8kv_decode_plan(plain, w.batch, w.group, int(lens.max()))
    assert splits == 1, (chunk, splits)
    q_bits = synth.q_bf16_bits(w.seed + 1, (w.batch, w.q_heads, w.head_dim))
    want = decode_q8(plain, q_bits, lens, w.group, w.sm_scale)
    ws = torch.empty(binding.fp8kv_decode_workspace_bytes(fused, w.batch, w.group,
                                                          int(lens.max())) // 4 + 4, device=DEV)
    got = torch.full((w.batch, w.q_heads, w.head_dim), float("nan"), device=DEV)
    binding.fp8kv_decode_append_q8(fused, torch.from_numpy(k_new).to(DEV),
                                   torch.from_numpy(v_new).to(DEV), q_tensor(q_bits), w.group,
                                   torch.from_numpy(lens).to(DEV), int(lens.max()), w.sm_scale,
                                   got, ws)
    got = got.cpu().numpy()
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), mode
    _narrow_gate(want, mode, q_bits, [s[0][:n] for s, n in zip(seqs, lens)],
                 [s[1][:n] for s, n in zip(seqs, lens)], w.sm_scale, ("one split q8", mode))
