"""GPU parity of the causal tiled prefill (fp8kv_prefill) against the oracle.

The keys are appended through fp8kv_append first (the store-then-attend path
the FA page's parity test drives), then every query row is compared with the
oracle's attention over its visible keys t <= q_pos0 + i.  Same gate as the
decode tests (see test_gpu_decode.py): contract relative L2 and max abs, the
latter measured outside the interval of valid bf16 roundings of P.
"""
import numpy as np
import pytest
import torch

import oracle
from fp8_kv_cache_append_amd import binding, synth
from fp8_kv_cache_append_amd.binding import KVCache
from gpu_util import append_seq, check_layout, make_cache, q_tensor
from oracle_pool import prefill_full
from test_gpu_decode import _gate

pytestmark = pytest.mark.gpu


def gpu_prefill(cache, q_bits, n_q, q_pos0, seq_lens, group, sm_scale):
    n_q = np.asarray(n_q, np.int32)
    cu = np.concatenate([[0], np.cumsum(n_q)]).astype(np.int32)
    seq_lens = np.asarray(seq_lens, np.int32)
    q_pos0 = np.asarray(q_pos0, np.int32)
    assert q_bits.shape[0] == cu[-1]
    assert np.all(q_pos0 + n_q <= seq_lens) and np.all(q_pos0 >= 0)
    check_layout(cache.block_table.cpu().numpy(), cache.block_size, seq_lens)
    out = torch.full(q_bits.shape, float("nan"), dtype=torch.float32, device="cuda")
    binding.fp8kv_prefill(cache, q_tensor(q_bits), group, torch.from_numpy(cu).cuda(),
                          torch.from_numpy(q_pos0).cuda(), torch.from_numpy(seq_lens).cuda(),
                          int(n_q.max()), sm_scale, out)
    return out.cpu().numpy(), cu


def _case(mode, hq, hkv, d, n_q, q_pos0, seq_lens, bs, seed, rows=None, dist="outliers",
          layout="token"):
    seq_lens = np.asarray(seq_lens, np.int32)
    w = synth.Workload("t", len(seq_lens), hq, hkv, d, seq_lens, dist, block_size=bs,
                       shuffle_blocks=bs > 0, seed=seed)
    cache = make_cache(mode, w, layout=layout)
    seqs = [synth.kv_sequence(w, b) for b in range(w.batch)]
    for b, (k, v) in enumerate(seqs):
        append_seq(cache, b, k, v)
    total = int(np.sum(n_q))
    q_bits = synth.q_bf16_bits(seed, (total, hq, d))
    got, cu = gpu_prefill(cache, q_bits, n_q, q_pos0, seq_lens, hq // hkv, w.sm_scale)
    refs = []
    for b in range(w.batch):
        qb = q_bits[cu[b]:cu[b + 1]]
        r = None if rows is None else rows
        refs.append(oracle.prefill(mode, qb, seqs[b][0], seqs[b][1], int(q_pos0[b]),
                                   w.sm_scale, rows=r, bounds=True))
    ref = np.concatenate([x[0] for x in refs])
    lo = np.concatenate([x[1] for x in refs])
    hi = np.concatenate([x[2] for x in refs])
    return got, ref, lo, hi


CASES = [
    # hq, hkv, d, n_q per seq, q_pos0 per seq, seq_lens, block size
    (4, 2, 64, [100], [0], [100], 16),
    (28, 4, 128, [200], [0], [200], 0),
    (8, 1, 128, [70], [130], [200], 32),                  # chunked prefill after 130 cached
    (16, 2, 128, [1, 64, 65, 130], [0, 10, 0, 3], [1, 74, 65, 133], 16),
    (2, 2, 64, [129], [0], [129], 64),                      # MHA
    (16, 1, 64, [90], [5], [95], 0),                        # GQA 16
    (8, 2, 128, [150], [0], [150], 48),                     # 3 sub-blocks per block
    (4, 1, 64, [40, 200], [100, 0], [140, 200], 80),        # 5 sub-blocks per block
    (4, 1, 128, [300], [0], [300], 256),                    # 16 sub-blocks per block
    (8, 2, 128, [100], [4900], [5000], 16),                 # chunk of a long context
]


@pytest.mark.parametrize("layout", ["token", "head"])
@pytest.mark.parametrize("mode", ["K8V8", "K16V8", "BF16", "K8V16"])
@pytest.mark.parametrize("case", CASES, ids=lambda c: f"hq{c[0]}_hkv{c[1]}_d{c[2]}_n{sum(c[3])}")
def test_prefill_small(mode, case, layout):
    hq, hkv, d, n_q, q_pos0, lens, bs = case
    got, ref, lo, hi = _case(mode, hq, hkv, d, n_q, q_pos0, lens, bs, seed=hq + d,
                             layout=layout)
    _gate(got, ref, lo, hi, (mode, case, layout))


@pytest.mark.timeout(600)
@pytest.mark.parametrize("mode", ["K8V8", "BF16"])
def test_prefill_t2048_gqa7_full(mode):
    """The benchmark's prefill: one sequence of 2048 tokens, 28/4 heads, D
    128, K/V ~ N(0,1), contiguous cache; every one of the 2048 x 28 output
    rows is compared with the oracle (one pool job per query head), with the
    contract's literal figures."""
    w = synth.prefill_gqa7_d128()
    n = int(w.lens[0])
    bs, table, n_blocks = synth.block_layout(w)
    # passed without a table, as the benchmark passes it
    cache = KVCache.allocate(mode, n_blocks, bs, w.kv_heads, w.head_dim, table, "cuda",
                             table_in_memory=False)
    k, v = synth.kv_sequence(w, 0)
    append_seq(cache, 0, k, v)
    q_bits = synth.q_bf16_bits(w.seed, (n, w.q_heads, w.head_dim))
    got, _ = gpu_prefill(cache, q_bits, [n], [0], [n], w.group, w.sm_scale)
    assert not np.any(np.isnan(got))
    ref, lo, hi = prefill_full(mode, q_bits, k, v, 0, w.sm_scale)
    _gate(got, ref, lo, hi, (w.name, mode), literal=True)


@pytest.mark.parametrize("mode", ["K8V8", "BF16", "K8V16"])
def test_prefill_unwritten_slots_hold_nan(mode):
    """Every byte of the cache is 0xFF (NaN in e4m3, bf16 and fp32) before the
    keys are appended, so slots past each sequence's last key hold NaN: keys
    that do not exist must not reach any output."""
    hq, hkv, d, bs = 8, 2, 128, 48
    n_q, q_pos0, lens = [37, 100], [0, 29], [37, 129]
    seq_lens = np.asarray(lens, np.int32)
    w = synth.Workload("t", 2, hq, hkv, d, seq_lens, "outliers", block_size=bs,
                       shuffle_blocks=True, seed=11)
    cache = make_cache(mode, w, capacity=192)
    for x in (cache.k, cache.v, cache.k_scale, cache.v_scale):
        if x is not None:
            x.view(torch.uint8).fill_(0xFF)
    seqs = [synth.kv_sequence(w, b) for b in range(w.batch)]
    for b, (k, v) in enumerate(seqs):
        append_seq(cache, b, k, v)
    q_bits = synth.q_bf16_bits(11, (int(np.sum(n_q)), hq, d))
    got, cu = gpu_prefill(cache, q_bits, n_q, q_pos0, lens, hq // hkv, w.sm_scale)
    assert np.all(np.isfinite(got))
    refs = [oracle.prefill(mode, q_bits[cu[b]:cu[b + 1]], seqs[b][0], seqs[b][1],
                           int(q_pos0[b]), w.sm_scale, bounds=True) for b in range(2)]
    ref, lo, hi = (np.concatenate([x[i] for x in refs]) for i in range(3))
    _gate(got, ref, lo, hi, (mode, "nan-filled"))


def test_prefill_repeat_bitwise_identical():
    """Standalone repeated-run harness (FA page, section 4): LDS double
    buffering must give identical bits run after run."""
    w = synth.prefill_gqa7_d128(tokens=512)
    n = int(w.lens[0])
    cache = make_cache("K8V8", w)
    k, v = synth.kv_sequence(w, 0)
    append_seq(cache, 0, k, v)
    q_bits = synth.q_bf16_bits(w.seed, (n, w.q_heads, w.head_dim))
    first, _ = gpu_prefill(cache, q_bits, [n], [0], [n], w.group, w.sm_scale)
    for _ in range(100):
        again, _ = gpu_prefill(cache, q_bits, [n], [0], [n], w.group, w.sm_scale)
        assert np.array_equal(first.view(np.uint32), again.view(np.uint32))


@pytest.mark.parametrize("mode", ["K8V8", "K16V8"])
def test_prefill_long_paged_two_sequences_sampled_rows(mode):
    """Two sequences of 3000 and 1700 tokens (28/4 heads, D 128) in a paged
    cache with 16-token blocks behind a shuffled table, the second a chunk
    of 900 queries after 800 cached keys: long walks over many tiles in both
    key groups of each work-group.  The oracle checks sampled query rows of
    each sequence (tile edges, chunk edges, the last rows) for all heads."""
    lens = [3000, 1700]
    n_q, q_pos0 = [3000, 900], [0, 800]
    w = synth.Workload("t", 2, 28, 4, 128, np.array(lens, np.int32), "outliers", block_size=16,
                       shuffle_blocks=True, seed=77)
    cache = make_cache(mode, w)
    seqs = [synth.kv_sequence(w, b) for b in range(2)]
    for b, (k, v) in enumerate(seqs):
        append_seq(cache, b, k, v)
    total = int(np.sum(n_q))
    q_bits = synth.q_bf16_bits(77, (total, 28, 128))
    got, cu = gpu_prefill(cache, q_bits, n_q, q_pos0, lens, 7, w.sm_scale)
    rng = np.random.default_rng(8)
    for b in range(2):
        rows = np.unique(np.concatenate([[0, 1, 127, 128, 129, n_q[b] - 129, n_q[b] - 1],
                                         rng.integers(0, n_q[b], 12)]))
        ref, lo, hi = oracle.prefill(mode, q_bits[cu[b]:cu[b + 1]], seqs[b][0], seqs[b][1],
                                     q_pos0[b], w.sm_scale, rows=rows, bounds=True)
        g = got[cu[b]:cu[b + 1]]
        _gate(g[rows], ref[rows], lo[rows], hi[rows], (mode, "long paged", b))
    assert not np.any(np.isnan(got))
