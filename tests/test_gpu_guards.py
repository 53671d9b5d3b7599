"""The kernels' guards on device-side indices (include/fp8kv.h: an append row
with an out-of-range sequence, position or block id is not written; a length
is clamped to the block-table capacity; a key whose block id is out of range
is not read and takes no part in the attention).

Every case here passes indices that the guards turn into skipped work; the
valid part of each call must still match the oracle exactly as usual.
"""
import numpy as np
import pytest
import torch

import oracle
from fp8_kv_cache_append_amd import binding, synth
from gpu_util import make_cache, read_rows
from test_gpu_decode import _gate

pytestmark = pytest.mark.gpu


def test_append_skips_out_of_range_rows():
    lens = np.array([48, 48], np.int32)
    w = synth.Workload("t", 2, 2, 2, 128, lens, "outliers", block_size=16,
                       shuffle_blocks=True, seed=21)
    cache = make_cache("K8V8", w)
    # block 1 of sequence 1 is marked unused
    table = cache.block_table.cpu().numpy().copy()
    dead = int(table[1, 1])
    table[1, 1] = -1
    cache.block_table.copy_(torch.from_numpy(table))
    n = 6
    k, v = synth.kv_sequence(w, 0, n)
    seq = np.array([0, 5, -1, 1, 1, 0], np.int32)       # 5, -1: no such sequence
    pos = np.array([0, 3, 3, 20, 2, 10 ** 6], np.int32)  # 20 -> unused block; 10**6: no slot
    binding.fp8kv_append(cache, torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda(),
                         torch.from_numpy(seq).cuda(), torch.from_numpy(pos).cuda())
    torch.cuda.synchronize()
    want = oracle.store_rows("K8V8", k, v)
    got0 = read_rows(cache, 0, 1)
    assert np.array_equal(got0["k8"][0], want["k8"][0])       # token 0 -> seq 0 pos 0
    kk = cache.k.cpu().numpy()
    assert np.array_equal(kk[table[1, 0], 2], want["k8"][4])   # token 4 -> seq 1 pos 2
    written = np.zeros(kk.shape[:2], bool)
    written[table[0, 0], 0] = True
    written[table[1, 0], 2] = True
    assert np.all(kk[~written] == 0), "a skipped row was written"
    assert np.all(cache.k[dead].cpu().numpy() == 0)


@pytest.mark.parametrize("mode", ["K8V8", "BF16"])
def test_decode_excludes_keys_of_invalid_blocks(mode):
    lens = np.array([200, 90], np.int32)
    w = synth.Workload("t", 2, 16, 2, 128, lens, "outliers", block_size=16,
                       shuffle_blocks=True, seed=22)
    cache = make_cache(mode, w)
    seqs = [synth.kv_sequence(w, b) for b in range(w.batch)]
    for b, (k, v) in enumerate(seqs):
        n = k.shape[0]
        binding.fp8kv_append(cache, torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda(),
                             torch.full((n,), b, dtype=torch.int32, device="cuda"),
                             torch.arange(n, dtype=torch.int32, device="cuda"))
    table = cache.block_table.cpu().numpy().copy()
    table[0, 3] = -7                     # keys 48..63 of sequence 0
    table[1, 5] = 10 ** 9                # keys 80..89 of sequence 1
    cache.block_table.copy_(torch.from_numpy(table))
    q_bits = synth.q_bf16_bits(w.seed, (w.batch, w.q_heads, w.head_dim))
    q = torch.from_numpy(q_bits.view(np.int16)).cuda().view(torch.bfloat16)
    dev_lens = torch.from_numpy(lens).cuda()
    ws = torch.empty(binding.fp8kv_decode_workspace_bytes(cache, 2, w.group, 200) // 4,
                     device="cuda")
    out = torch.empty((2, w.q_heads, w.head_dim), device="cuda")
    binding.fp8kv_decode(cache, q, w.group, dev_lens, 200, w.sm_scale, out, ws)
    got = out.cpu().numpy()
    keep = [np.r_[0:48, 64:200], np.r_[0:80]]
    ref, lo, hi = oracle.decode(mode, q_bits, [seqs[b][0][keep[b]] for b in range(2)],
                                [seqs[b][1][keep[b]] for b in range(2)], w.sm_scale,
                                bounds=True)
    _gate(got, ref, lo, hi, (mode, "invalid blocks"))


def test_decode_clamps_lengths_to_capacity():
    lens = np.array([64, 64], np.int32)
    w = synth.Workload("t", 2, 8, 1, 64, lens, "normal", block_size=16, seed=23)
    cache = make_cache("K8V8", w)
    seqs = [synth.kv_sequence(w, b) for b in range(w.batch)]
    for b, (k, v) in enumerate(seqs):
        binding.fp8kv_append(cache, torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda(),
                             torch.full((64,), b, dtype=torch.int32, device="cuda"),
                             torch.arange(64, dtype=torch.int32, device="cuda"))
    q_bits = synth.q_bf16_bits(w.seed, (2, 8, 64))
    q = torch.from_numpy(q_bits.view(np.int16)).cuda().view(torch.bfloat16)
    # device lengths beyond the table capacity (4 blocks x 16) and negative
    dev_lens = torch.tensor([10 ** 6, -5], dtype=torch.int32, device="cuda")
    chunk, splits = binding.fp8kv_decode_plan(cache, 2, 8, 64)
    pacc = torch.zeros((2, 1, splits, 8, 64), device="cuda")
    pml = torch.zeros((2, 1, splits, 8, 2), device="cuda")
    binding.fp8kv_decode_partial(cache, q, 8, dev_lens, 64, w.sm_scale, chunk, splits, pacc, pml)
    out = torch.empty((2, 8, 64), device="cuda")
    binding.fp8kv_decode_merge(2, 1, 8, 64, splits, pacc, pml, out)
    got = out.cpu().numpy()
    ref, lo, hi = oracle.decode("K8V8", q_bits[:1], [seqs[0][0]], [seqs[0][1]], w.sm_scale,
                                bounds=True)
    _gate(got[:1], ref, lo, hi, "length clamped to capacity")
    assert np.all(got[1] == 0)           # negative length: no key


def test_prefill_clamps_query_rows_and_skips_invalid_blocks():
    lens = np.array([100], np.int32)
    w = synth.Workload("t", 1, 4, 2, 64, lens, "outliers", block_size=16, seed=24)
    cache = make_cache("K8V8", w)
    k, v = synth.kv_sequence(w, 0)
    binding.fp8kv_append(cache, torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda(),
                         torch.zeros(100, dtype=torch.int32, device="cuda"),
                         torch.arange(100, dtype=torch.int32, device="cuda"))
    table = cache.block_table.cpu().numpy().copy()
    table[0, 2] = -1                     # keys 32..47 are not read
    cache.block_table.copy_(torch.from_numpy(table))
    q_bits = synth.q_bf16_bits(w.seed, (100, 4, 64))
    q = torch.from_numpy(q_bits.view(np.int16)).cuda().view(torch.bfloat16)
    out = torch.full((100, 4, 64), float("nan"), device="cuda")
    # cu_q claims 10**6 queries: rows past total_q (100) must be neither read nor written
    cu = torch.tensor([0, 10 ** 6], dtype=torch.int32, device="cuda")
    binding.fp8kv_prefill(cache, q, 2, cu, torch.zeros(1, dtype=torch.int32, device="cuda"),
                          torch.tensor([100], dtype=torch.int32, device="cuda"), 100,
                          w.sm_scale, out)
    got = out.cpu().numpy()
    keep = np.r_[0:32, 48:100]
    store = oracle.store_rows("K8V8", k[keep], v[keep])
    for i in (0, 31, 40, 47, 48, 99):
        n_valid = int(np.sum(keep <= i))
        for hh in range(4):
            view = {key: np.ascontiguousarray(a[:, hh // 2]) for key, a in store.items()}
            r = oracle.attend_rows("K8V8", q_bits[i, hh][None], view, n_valid, w.sm_scale,
                                   bounds=True)
            _gate(got[i, hh][None], *r, ("prefill guard", i, hh))
