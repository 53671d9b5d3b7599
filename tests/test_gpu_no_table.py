"""A cache passed with no block table (contiguous layout).

With block_table NULL the library takes block b * max_blocks_per_seq + e for
block e of sequence b instead of reading a table.  Each test builds two
caches over the same contiguous layout -- one whose table (holding exactly
those ids) is passed, one passed with no table -- runs the same calls on
both, and requires identical bytes: the cache after the appends and every
output.  The no-table decode output also meets the parity gate against the
oracle.
"""
import numpy as np
import pytest
import torch

import oracle
from fp8_kv_cache_append_amd import binding, synth
from fp8_kv_cache_append_amd.binding import KVCache
from gpu_util import DEV, append_seq, q_tensor
from test_gpu_decode import _gate

pytestmark = pytest.mark.gpu


def _pair(mode, w, capacity, layout="token"):
    bs, table, n_blocks = synth.block_layout(w, capacity)
    assert np.array_equal(table.ravel(), np.arange(table.size)), "layout is not contiguous"
    a = KVCache.allocate(mode, n_blocks, bs, w.kv_heads, w.head_dim, table, DEV, layout=layout)
    b = KVCache.allocate(mode, n_blocks, bs, w.kv_heads, w.head_dim, table, DEV,
                         table_in_memory=False, layout=layout)
    return a, b


def _same_cache(a, b):
    for name in ("k", "v", "k_scale", "v_scale"):
        x, y = getattr(a, name), getattr(b, name)
        assert (x is None) == (y is None)
        if x is not None:
            assert torch.equal(x.view(torch.uint8), y.view(torch.uint8)), name


# (block size, capacity): one block per sequence, and 16-token blocks with
# the same number of blocks for every sequence (ids b * 128 + e)
LAYOUTS = [(0, None), (16, 2048)]


@pytest.mark.parametrize("layout", ["token", "head"])
@pytest.mark.parametrize("mode", ["K8V8", "K16V8", "BF16"])
@pytest.mark.parametrize("bs,capacity", LAYOUTS)
def test_decode_append_without_table(mode, bs, capacity, layout):
    lens = np.array([300, 1, 2048, 777], np.int32)
    w = synth.Workload("t", len(lens), 16, 2, 128, lens, "outliers", block_size=bs, seed=43)
    cache_t, cache_n = _pair(mode, w, capacity, layout)
    seqs = [synth.kv_sequence(w, b) for b in range(w.batch)]
    for cache in (cache_t, cache_n):
        for b, (k, v) in enumerate(seqs):
            append_seq(cache, b, k[:-1], v[:-1])
    torch.cuda.synchronize()
    _same_cache(cache_t, cache_n)
    k_new = torch.from_numpy(np.stack([k[-1] for k, _ in seqs])).to(DEV)
    v_new = torch.from_numpy(np.stack([v[-1] for _, v in seqs])).to(DEV)
    q_bits = synth.q_bf16_bits(w.seed, (w.batch, w.q_heads, w.head_dim))
    q = q_tensor(q_bits)
    lens_t = torch.from_numpy(lens).to(DEV)
    max_len = int(lens.max())
    outs = []
    for cache in (cache_t, cache_n):
        ws_bytes = binding.fp8kv_decode_workspace_bytes(cache, w.batch, w.group, max_len)
        ws = torch.empty(max(ws_bytes // 4, 4), dtype=torch.float32, device=DEV)
        out = torch.full((w.batch, w.q_heads, w.head_dim), float("nan"), device=DEV)
        binding.fp8kv_decode_append(cache, k_new, v_new, q, w.group, lens_t, max_len,
                                    w.sm_scale, out, ws)
        torch.cuda.synchronize()
        outs.append(out.cpu().numpy())
    _same_cache(cache_t, cache_n)
    assert np.array_equal(outs[0].view(np.uint32), outs[1].view(np.uint32))
    ref, lo, hi = oracle.decode(mode, q_bits, [s[0] for s in seqs], [s[1] for s in seqs],
                                w.sm_scale, bounds=True)
    _gate(outs[1], ref, lo, hi, (mode, bs, "no table"))


@pytest.mark.parametrize("d", [128, 64])
@pytest.mark.parametrize("mode", ["K8V8", "K16V8", "K8V16", "BF16"])
@pytest.mark.parametrize("layout", ["token", "head"])
@pytest.mark.parametrize("bs,capacity", LAYOUTS)
def test_prefill_without_table(bs, capacity, layout, mode, d):
    # token-major rows without a table take the linear-offset path (keys read
    # through buffer offsets, zeros past the last key); head-major rows the
    # computed-block path; both must equal the table path bit for bit.  The
    # second sequence's queries start at position 136: its first 136 keys are
    # cached context, and its query tile ends inside a key tile.
    lens = np.array([640, 200], np.int32)
    w = synth.Workload("t", len(lens), 28, 4, d, lens, "normal", block_size=bs,
                       prefill=True, seed=44)
    cache_t, cache_n = _pair(mode, w, capacity, layout)
    seqs = [synth.kv_sequence(w, b) for b in range(w.batch)]
    for cache in (cache_t, cache_n):
        for b, (k, v) in enumerate(seqs):
            append_seq(cache, b, k, v)
    first = np.array([0, 136], np.int32)
    nq = lens - first
    n = int(nq.sum())
    q = q_tensor(synth.q_bf16_bits(w.seed, (n, w.q_heads, w.head_dim)))
    cu = torch.tensor([0, int(nq[0]), n], dtype=torch.int32, device=DEV)
    pos0 = torch.from_numpy(first).to(DEV)
    lens_t = torch.from_numpy(lens).to(DEV)
    outs = []
    for cache in (cache_t, cache_n):
        out = torch.full((n, w.q_heads, w.head_dim), float("nan"), device=DEV)
        binding.fp8kv_prefill(cache, q, w.group, cu, pos0, lens_t, int(nq.max()), w.sm_scale,
                              out)
        torch.cuda.synchronize()
        outs.append(out.cpu().numpy())
    assert not np.any(np.isnan(outs[1]))
    assert np.array_equal(outs[0].view(np.uint32), outs[1].view(np.uint32))
