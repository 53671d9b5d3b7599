"""GPU parity of the decode step with the append fused in
(fp8kv_decode_append).

The step stores each sequence's new token at position seq_lens[b] - 1 and
attends it with the rest.  Its contract is "fp8kv_append, then fp8kv_decode"
in fewer kernels, so every case checks three things:
  * the cache afterwards is byte-identical to one filled by fp8kv_append
    alone (codes, scales, bf16 bytes, untouched slots);
  * the output is bit-identical to fp8kv_decode over that cache (the same
    register values reach the same arithmetic);
  * the output meets the oracle gate (test_gpu_decode._gate).
"""
import numpy as np
import pytest
import torch

import oracle
from fp8_kv_cache_append_amd import binding, synth
from gpu_util import DEV, append_seq, check_layout, decode, make_cache, q_tensor
from test_gpu_decode import _gate

pytestmark = pytest.mark.gpu


def _step(cache, k_new, v_new, q_bits, lens, group, sm_scale):
    lens = np.asarray(lens, np.int32)
    b, hq, d = q_bits.shape
    assert k_new.shape == v_new.shape == (b, cache.num_kv_heads, d)
    max_len = int(lens.max()) if b else 0
    ws_bytes = binding.fp8kv_decode_workspace_bytes(cache, b, group, max_len)
    ws = torch.empty(max(ws_bytes // 4, 4), dtype=torch.float32, device=DEV)
    out = torch.full((b, hq, d), float("nan"), dtype=torch.float32, device=DEV)
    binding.fp8kv_decode_append(cache, torch.from_numpy(np.ascontiguousarray(k_new)).to(DEV),
                                torch.from_numpy(np.ascontiguousarray(v_new)).to(DEV),
                                q_tensor(q_bits), group, torch.from_numpy(lens).to(DEV),
                                max_len, sm_scale, out, ws)
    return out.cpu().numpy()


def _cache_bytes(cache):
    parts = [cache.k.view(torch.uint8) if cache.k.dtype != torch.uint8 else cache.k,
             cache.v.view(torch.uint8) if cache.v.dtype != torch.uint8 else cache.v]
    parts += [x.view(torch.uint8) for x in (cache.k_scale, cache.v_scale) if x is not None]
    return [p.cpu().numpy().copy() for p in parts]


def _compare(mode, w, lens_attend, news, layout="token"):
    """news[b]: index of the token the step appends (the sequence's last)."""
    seqs = [synth.kv_sequence(w, b) for b in range(w.batch)]
    q_bits = synth.q_bf16_bits(w.seed + 7, (w.batch, w.q_heads, w.head_dim))
    fused, plain = make_cache(mode, w, layout=layout), make_cache(mode, w, layout=layout)
    k_new = np.zeros((w.batch, w.kv_heads, w.head_dim), np.float32)
    v_new = np.zeros_like(k_new)
    for b, (k, v) in enumerate(seqs):
        n = int(w.lens[b])
        j = news[b]
        assert j == n - 1
        append_seq(fused, b, k[:j], v[:j])
        append_seq(plain, b, k[:j + 1], v[:j + 1])
        k_new[b], v_new[b] = k[j], v[j]
    got = _step(fused, k_new, v_new, q_bits, lens_attend, w.group, w.sm_scale)
    want = decode(plain, q_bits, lens_attend, w.group, w.sm_scale)
    for x, y in zip(_cache_bytes(fused), _cache_bytes(plain)):
        assert np.array_equal(x, y), (mode, "cache bytes differ")
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), (mode, "output differs")
    return seqs, q_bits, got


SHAPES = [
    # (q_heads, kv_heads, head_dim, lens, block_size)
    (16, 2, 128, [1, 64, 65, 200, 256, 257, 1000], 0),
    (32, 8, 128, [700, 16, 1, 1024, 33], 16),
    (4, 1, 64, [128, 63, 2], 16),
    (28, 4, 128, [513, 2000], 32),
]


@pytest.mark.parametrize("layout", ["token", "head"])
@pytest.mark.parametrize("mode", ["K8V8", "K16V8", "BF16", "K8V16"])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: f"hq{s[0]}_hkv{s[1]}_d{s[2]}_bs{s[4]}")
def test_fused_append_matches_append_then_decode(mode, shape, layout):
    hq, hkv, d, lens, bs = shape
    lens = np.array(lens, np.int32)
    w = synth.Workload("t", len(lens), hq, hkv, d, lens, "outliers", block_size=bs,
                       shuffle_blocks=bs > 0, seed=hq * 13 + d + bs)
    seqs, q_bits, got = _compare(mode, w, lens, [int(n) - 1 for n in lens], layout)
    ref, lo, hi = oracle.decode(mode, q_bits, [s[0] for s in seqs], [s[1] for s in seqs],
                                w.sm_scale, bounds=True)
    _gate(got, ref, lo, hi, (mode, "fused append", shape))


@pytest.mark.parametrize("mode", ["K8V8", "K16V8"])
def test_fused_append_b16_t2048(mode):
    """The benchmark step's shape: 16 sequences x 16q/2kv x D128, the 2048th
    key appended by the step."""
    w = synth.decode_b16_gqa8_d128(2048)
    seqs, q_bits, got = _compare(mode, w, w.lens, [2047] * w.batch)
    ref, lo, hi = oracle.decode(mode, q_bits, [s[0] for s in seqs], [s[1] for s in seqs],
                                w.sm_scale, pairs=[(b, h) for b in (0, 9) for h in (0, 1)],
                                bounds=True)
    _gate(got, ref, lo, hi, (mode, "fused append b16 t2048"))


def test_fused_append_skips_empty_and_out_of_capacity():
    """Length 0: nothing stored, output 0.  A length beyond the block table's
    capacity: nothing stored, keys clamped to the capacity."""
    lens = np.array([0, 40, 64], np.int32)
    w = synth.Workload("t", 3, 8, 2, 128, lens, "normal", block_size=16, seed=41)
    cache = make_cache("K8V8", w, capacity=64)   # 4 blocks of 16 per sequence
    seqs = [synth.kv_sequence(w, b) for b in range(3)]
    for b in (1, 2):
        append_seq(cache, b, seqs[b][0][:int(lens[b]) - 1], seqs[b][1][:int(lens[b]) - 1])
    before = _cache_bytes(cache)
    q_bits = synth.q_bf16_bits(w.seed, (3, 8, 128))
    k_new = np.full((3, 2, 128), 3.0, np.float32)
    v_new = np.full((3, 2, 128), -3.0, np.float32)
    k_new[1], v_new[1] = seqs[1][0][39], seqs[1][1][39]
    # sequence 2's device length (65) exceeds the 64-slot capacity and the
    # host's max_seq_len: its new token (position 64) has no slot
    dev_lens = np.array([0, 40, 65], np.int32)
    table = cache.block_table.cpu().numpy()
    check_layout(table, 16, [0, 40, 64])
    max_len = 64
    ws = torch.empty(binding.fp8kv_decode_workspace_bytes(cache, 3, 4, max_len) // 4,
                     device=DEV)
    out = torch.full((3, 8, 128), float("nan"), device=DEV)
    binding.fp8kv_decode_append(cache, torch.from_numpy(k_new).to(DEV),
                                torch.from_numpy(v_new).to(DEV), q_tensor(q_bits), 4,
                                torch.from_numpy(dev_lens).to(DEV), max_len, w.sm_scale, out, ws)
    got = out.cpu().numpy()
    after = _cache_bytes(cache)
    # only sequence 1's slot 39 changed
    ref_cache = make_cache("K8V8", w, capacity=64)
    for b in (1, 2):
        n = int(lens[b]) - 1 + (1 if b == 1 else 0)
        append_seq(ref_cache, b, seqs[b][0][:n], seqs[b][1][:n])
    for x, y in zip(after, _cache_bytes(ref_cache)):
        assert np.array_equal(x, y)
    assert any(not np.array_equal(x, z) for x, z in zip(after, before))
    assert np.all(got[0] == 0)
    keys = [seqs[0][0][:0], seqs[1][0][:40], seqs[2][0][:63]]
    vals = [seqs[0][1][:0], seqs[1][1][:40], seqs[2][1][:63]]
    # sequence 2: keys clamped to the 64-slot capacity; slot 63 was never
    # written (zero codes and scale), so its key is a zero vector with score 0
    keys[2] = np.concatenate([keys[2], np.zeros((1, 2, 128), np.float32)])
    vals[2] = np.concatenate([vals[2], np.zeros((1, 2, 128), np.float32)])
    ref, lo, hi = oracle.decode("K8V8", q_bits[1:], keys[1:], vals[1:], w.sm_scale, bounds=True)
    _gate(got[1:], ref, lo, hi, "fused append guards")


def test_fused_append_invalid_block_is_not_written():
    """The new token's block id is out of range: nothing is stored and the
    key takes no part in the attention."""
    lens = np.array([50, 90], np.int32)
    w = synth.Workload("t", 2, 16, 2, 128, lens, "outliers", block_size=16,
                       shuffle_blocks=True, seed=43)
    cache = make_cache("K8V8", w)
    seqs = [synth.kv_sequence(w, b) for b in range(2)]
    for b in range(2):
        n = int(lens[b]) - 1
        append_seq(cache, b, seqs[b][0][:n], seqs[b][1][:n])
    table = cache.block_table.cpu().numpy().copy()
    table[1, 88 // 16] = -3                # keys 80..89 of sequence 1, incl. the new one
    cache.block_table.copy_(torch.from_numpy(table))
    before = _cache_bytes(cache)
    q_bits = synth.q_bf16_bits(w.seed, (2, 16, 128))
    k_new = np.stack([seqs[b][0][int(lens[b]) - 1] for b in range(2)])
    v_new = np.stack([seqs[b][1][int(lens[b]) - 1] for b in range(2)])
    ws = torch.empty(binding.fp8kv_decode_workspace_bytes(cache, 2, 8, 90) // 4, device=DEV)
    out = torch.full((2, 16, 128), float("nan"), device=DEV)
    binding.fp8kv_decode_append(cache, torch.from_numpy(k_new).to(DEV),
                                torch.from_numpy(v_new).to(DEV), q_tensor(q_bits), 8,
                                torch.from_numpy(lens).to(DEV), 90, w.sm_scale, out, ws)
    got = out.cpu().numpy()
    after = _cache_bytes(cache)
    # only sequence 0's new slot (position 49) differs from before, in K and V
    blk0, slot0 = int(table[0, 49 // 16]), 49 % 16
    for x, y in zip(after[:2], before[:2]):
        diff = np.argwhere(x != y)
        assert diff.size and np.all(diff[:, 0] == blk0) and np.all(diff[:, 1] == slot0)
    keep = [np.r_[0:50], np.r_[0:80]]
    ref, lo, hi = oracle.decode("K8V8", q_bits, [seqs[b][0][keep[b]] for b in range(2)],
                                [seqs[b][1][keep[b]] for b in range(2)], w.sm_scale,
                                bounds=True)
    _gate(got, ref, lo, hi, "fused append, invalid block")


def _split_step(cache, q_bits, lens, group, sm_scale, chunk, k_new=None, v_new=None):
    """Split kernel with an explicit chunk (fused when k_new is given), then
    the merge: the entry points the planner's choice dispatches to."""
    lens = np.asarray(lens, np.int32)
    b, hq, d = q_bits.shape
    max_len = int(lens.max())
    splits = -(-max_len // chunk)
    hkv = cache.num_kv_heads
    pacc = torch.full((b, hkv, splits, group, d), float("nan"), device=DEV)
    pml = torch.full((b, hkv, splits, group, 2), float("nan"), device=DEV)
    out = torch.full((b, hq, d), float("nan"), dtype=torch.float32, device=DEV)
    dl = torch.from_numpy(lens).to(DEV)
    if k_new is None:
        binding.fp8kv_decode_partial(cache, q_tensor(q_bits), group, dl, max_len, sm_scale, chunk,
                                     splits, pacc, pml)
    else:
        binding.fp8kv_decode_append_partial(
            cache, torch.from_numpy(np.ascontiguousarray(k_new)).to(DEV),
            torch.from_numpy(np.ascontiguousarray(v_new)).to(DEV), q_tensor(q_bits), group, dl,
            max_len, sm_scale, chunk, splits, pacc, pml)
    binding.fp8kv_decode_merge(b, hkv, group, d, splits, pacc, pml, out)
    return out.cpu().numpy()


@pytest.mark.parametrize("chunk", [128, 256], ids=["half_tile", "one_tile"])
@pytest.mark.parametrize("layout", ["token", "head"])
@pytest.mark.parametrize("mode", ["K8V8", "K16V8", "BF16", "K8V16"])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: f"hq{s[0]}_hkv{s[1]}_d{s[2]}_bs{s[4]}")
def test_fused_append_each_split_shape(mode, shape, layout, chunk):
    """Both single-pass split variants with the append fused in, whatever the
    planner would pick for the shape: 128-key splits (each wave attends half
    a 64-key tile) and 256-key splits (one tile per wave).  Bit-identical to
    fp8kv_append followed by the plain split kernel with the same chunk, and
    within the oracle gate."""
    hq, hkv, d, lens, bs = shape
    lens = np.array(lens, np.int32)
    w = synth.Workload("t", len(lens), hq, hkv, d, lens, "outliers", block_size=bs,
                       shuffle_blocks=bs > 0, seed=hq * 13 + d + bs + 5)
    seqs = [synth.kv_sequence(w, b) for b in range(w.batch)]
    q_bits = synth.q_bf16_bits(w.seed + 7, (w.batch, w.q_heads, w.head_dim))
    fused, plain = make_cache(mode, w, layout=layout), make_cache(mode, w, layout=layout)
    k_new = np.zeros((w.batch, w.kv_heads, w.head_dim), np.float32)
    v_new = np.zeros_like(k_new)
    for b, (k, v) in enumerate(seqs):
        n = int(lens[b])
        append_seq(fused, b, k[:n - 1], v[:n - 1])
        append_seq(plain, b, k[:n], v[:n])
        k_new[b], v_new[b] = k[n - 1], v[n - 1]
    got = _split_step(fused, q_bits, lens, w.group, w.sm_scale, chunk, k_new, v_new)
    want = _split_step(plain, q_bits, lens, w.group, w.sm_scale, chunk)
    for x, y in zip(_cache_bytes(fused), _cache_bytes(plain)):
        assert np.array_equal(x, y), (mode, chunk, "cache bytes differ")
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), (mode, chunk, "output differs")
    ref, lo, hi = oracle.decode(mode, q_bits, [s[0] for s in seqs], [s[1] for s in seqs],
                                w.sm_scale, bounds=True)
    _gate(got, ref, lo, hi, (mode, "fused append", chunk, shape, layout))
