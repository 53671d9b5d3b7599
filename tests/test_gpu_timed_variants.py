"""GPU parity of exactly the kernel variants the benchmark times, at the
benchmark's sizes: bit for bit against append-then-decode, and against the
oracle over every (sequence, KV head) pair.

The split kernel has a variant for splits of several 64-key tiles per wave
(a chunk above 256 keys: each wave streams its tiles through one register
buffer, the next tile's halves loaded behind the current tile's), and for
caches passed without a block table.  The benchmark times the fused-append
form of these: at 8192 keys per sequence (contiguous cache, no table) in
every mode and with narrow QK, and on the ragged batch-64 paged workload
(table) in K8V8, K16V8 and as a pre-bias residual cache.  Every test here
asserts that the plan it runs has chunk >= 512, so that the multi-tile
variant is the one checked, and calls the same entry points the benchmark
calls (fp8kv_decode_append_partial + fp8kv_decode_merge with the plan of
fp8kv_decode_plan; fp8kv_decode_append_q8).

Bit-identity: the fused step must leave the cache byte-identical to one
filled by fp8kv_append alone and return exactly the output of fp8kv_decode
(the same kernel family without the fused append) over that cache.  The
oracle gate is test_gpu_decode._gate with the contract's literal figures
(relative L2 <= 1e-3, max abs <= 5e-3 against the nominal output).
"""
import functools

import numpy as np
import pytest
import torch

from fp8_kv_cache_append_amd import binding, synth
from fp8_kv_cache_append_amd.binding import KVCache
from gpu_util import DEV, q_tensor
from oracle_pool import DecodeOracle, decode_full
from test_gpu_decode import _gate

pytestmark = pytest.mark.gpu


def _cache(mode, w, table_in_memory=True, layout="token"):
    bs, table, n_blocks = synth.block_layout(w)
    return KVCache.allocate(mode, n_blocks, bs, w.kv_heads, w.head_dim, table, DEV,
                            table_in_memory=table_in_memory, layout=layout)


def _append(cache, b, k, v):
    n = k.shape[0]
    if n == 0:
        return
    binding.fp8kv_append(cache, torch.from_numpy(np.ascontiguousarray(k)).to(DEV),
                         torch.from_numpy(np.ascontiguousarray(v)).to(DEV),
                         torch.full((n,), b, dtype=torch.int32, device=DEV),
                         torch.arange(n, dtype=torch.int32, device=DEV))


def _same_cache(a, b, ctx):
    for name in ("k", "v", "k_scale", "v_scale"):
        x, y = getattr(a, name), getattr(b, name)
        assert (x is None) == (y is None), (ctx, name)
        if x is not None:
            assert torch.equal(x.view(torch.uint8), y.view(torch.uint8)), (ctx, name, "differs")


def _plan(cache, w):
    chunk, splits = binding.fp8kv_decode_plan(cache, w.batch, w.group, w.max_len)
    print(f"{w.name}: plan chunk={chunk} splits={splits}", flush=True)
    assert chunk >= 512, ("the multi-tile variant is not the one planned", chunk)
    return chunk, splits


def _bench_step(cache, w, k_new, v_new, q, lens):
    """The benchmark's step: fused split kernel with the plan, then merge."""
    chunk, splits = _plan(cache, w)
    g, d = w.group, w.head_dim
    pacc = torch.full((w.batch, w.kv_heads, splits, g, d), float("nan"), device=DEV)
    pml = torch.full((w.batch, w.kv_heads, splits, g, 2), float("nan"), device=DEV)
    out = torch.full((w.batch, w.q_heads, d), float("nan"), device=DEV)
    binding.fp8kv_decode_append_partial(cache, k_new, v_new, q, g, lens, w.max_len, w.sm_scale,
                                        chunk, splits, pacc, pml)
    binding.fp8kv_decode_merge(w.batch, w.kv_heads, g, d, splits, pacc, pml, out)
    torch.cuda.synchronize()
    return out


def _plain_decode(cache, w, q, lens, q8=False):
    ws = torch.empty(binding.fp8kv_decode_workspace_bytes(cache, w.batch, w.group, w.max_len)
                     // 4 + 4, device=DEV)
    out = torch.full((w.batch, w.q_heads, w.head_dim), float("nan"), device=DEV)
    fn = binding.fp8kv_decode_q8 if q8 else binding.fp8kv_decode
    fn(cache, q, w.group, lens, w.max_len, w.sm_scale, out, ws)
    torch.cuda.synchronize()
    return out


# ------------------------------------------------- B16, 16q/2kv, 8192 keys

W8192 = synth.decode_b16_gqa8_d128(8192)   # the benchmark's context-sweep workload


@functools.lru_cache(maxsize=1)
def _seqs8192():
    return [synth.kv_sequence(W8192, b) for b in range(W8192.batch)]


@functools.lru_cache(maxsize=8)
def _oracle8192(mode, q8=False):
    seqs = _seqs8192()
    q_bits = synth.q_bf16_bits(W8192.seed, (W8192.batch, W8192.q_heads, W8192.head_dim))
    ref = decode_full(mode, q_bits, [s[0] for s in seqs], [s[1] for s in seqs],
                      W8192.sm_scale, q8=q8)
    unr = None
    if q8:
        unr = decode_full(mode, q_bits, [s[0] for s in seqs], [s[1] for s in seqs],
                          W8192.sm_scale, round_p=False, q8=True)[0]
    return ref, unr


def _fused_and_plain(mode, w, seqs, table_in_memory, layout="token"):
    fused = _cache(mode, w, table_in_memory, layout)
    plain = _cache(mode, w, table_in_memory, layout)
    for b, (k, v) in enumerate(seqs):
        _append(fused, b, k[:-1], v[:-1])
        _append(plain, b, k, v)
    k_new = torch.from_numpy(np.stack([k[-1] for k, _ in seqs])).to(DEV)
    v_new = torch.from_numpy(np.stack([v[-1] for _, v in seqs])).to(DEV)
    return fused, plain, k_new, v_new


@pytest.mark.parametrize("layout", ["token", "head"])
@pytest.mark.parametrize("table_in_memory", [False, True], ids=["no_table", "table"])
@pytest.mark.parametrize("mode", ["K8V8", "K16V8", "BF16", "K8V16"])
def test_fused_multi_tile_b16_t8192(mode, table_in_memory, layout):
    w = W8192
    seqs = _seqs8192()
    fused, plain, k_new, v_new = _fused_and_plain(mode, w, seqs, table_in_memory, layout)
    q_bits = synth.q_bf16_bits(w.seed, (w.batch, w.q_heads, w.head_dim))
    q = q_tensor(q_bits)
    lens = torch.from_numpy(w.lens).to(DEV)
    got = _bench_step(fused, w, k_new, v_new, q, lens)
    want = _plain_decode(plain, w, q, lens)
    ctx = (w.name, mode, "table" if table_in_memory else "no table", layout)
    _same_cache(fused, plain, ctx)
    assert torch.equal(got.view(torch.int32), want.view(torch.int32)), (ctx, "output differs")
    # the public fused entry point is the same two kernels
    again = torch.full_like(got, float("nan"))
    ws = torch.empty(binding.fp8kv_decode_workspace_bytes(plain, w.batch, w.group, w.max_len)
                     // 4 + 4, device=DEV)
    binding.fp8kv_decode_append(plain, k_new, v_new, q, w.group, lens, w.max_len, w.sm_scale,
                                again, ws)
    torch.cuda.synchronize()
    assert torch.equal(again.view(torch.int32), want.view(torch.int32)), ctx
    (ref, lo, hi), _ = _oracle8192(mode)
    _gate(got.cpu().numpy(), ref, lo, hi, ctx, literal=True)


@pytest.mark.parametrize("layout", ["token", "head"])
@pytest.mark.parametrize("mode", ["K8V8", "K8V16"])
def test_fused_narrow_qk_multi_tile_b16_t8192(mode, layout):
    """fp8kv_decode_append_q8 (the benchmark's narrow_qk leg) at 8192 keys:
    bit-identical to fp8kv_append + fp8kv_decode_q8, and the narrow-QK gate
    (test_gpu_decode_q8) against the oracle's narrow path in full."""
    w = W8192
    seqs = _seqs8192()
    fused, plain, k_new, v_new = _fused_and_plain(mode, w, seqs, False, layout)
    _plan(fused, w)
    q_bits = synth.q_bf16_bits(w.seed, (w.batch, w.q_heads, w.head_dim))
    q = q_tensor(q_bits)
    lens = torch.from_numpy(w.lens).to(DEV)
    ws = torch.empty(binding.fp8kv_decode_workspace_bytes(fused, w.batch, w.group, w.max_len)
                     // 4 + 4, device=DEV)
    got = torch.full((w.batch, w.q_heads, w.head_dim), float("nan"), device=DEV)
    binding.fp8kv_decode_append_q8(fused, k_new, v_new, q, w.group, lens, w.max_len,
                                   w.sm_scale, got, ws)
    want = _plain_decode(plain, w, q, lens, q8=True)
    ctx = (w.name, mode, "narrow QK", layout)
    _same_cache(fused, plain, ctx)
    assert torch.equal(got.view(torch.int32), want.view(torch.int32)), (ctx, "output differs")
    (ref, lo, hi), unr = _oracle8192(mode, q8=True)
    bar = 1e-3 + 2.0 * float(np.linalg.norm(ref - unr) / np.linalg.norm(ref))
    print(f"{ctx}: narrow bar rel_l2 <= {bar:.2e}", flush=True)
    _gate(got.cpu().numpy(), ref, lo, hi, ctx, expect_rel=bar, gate_rel=bar)


# ------------------------------------------- ragged batch 64, paged 16, full

@pytest.mark.timeout(900)
@pytest.mark.parametrize("layout", ["token", "head"])
@pytest.mark.parametrize("variant", ["K8V8", "K16V8", "K8V8_pre_bias"])
def test_ragged_b64_paged_fused_full(variant, layout):
    """The benchmark's ragged legs: 64 sequences of 1024-32768 keys, 32q/8kv,
    16-token blocks behind a shuffled table, biased keys; the fused split
    kernel with the plan (chunk 1024) and the merge.  Every (sequence, KV
    head) pair of the output is compared with the oracle.  The pre-bias
    variant stores the keys' residuals with the exact bias in the
    descriptor."""
    mode = variant.split("_")[0]
    pre_bias = variant.endswith("pre_bias")
    w = synth.decode_b64_gqa4_ragged_paged()
    q_bits = synth.q_bf16_bits(w.seed, (w.batch, w.q_heads, w.head_dim))
    fused, plain = _cache(mode, w, layout=layout), _cache(mode, w, layout=layout)
    bias = None
    if pre_bias:
        bias = synth.kv_sequence_prebias(w, 0)[2]
        for c in (fused, plain):
            c.k_bias = torch.from_numpy(bias).to(DEV)
    orc = DecodeOracle(mode, q_bits, w.sm_scale, w.kv_heads, k_bias=bias)
    k_new = np.zeros((w.batch, w.kv_heads, w.head_dim), np.float32)
    v_new = np.zeros_like(k_new)
    for b in range(w.batch):
        if pre_bias:
            k, v, _ = synth.kv_sequence_prebias(w, b)
        else:
            k, v = synth.kv_sequence(w, b)
        _append(fused, b, k[:-1], v[:-1])
        _append(plain, b, k, v)
        k_new[b], v_new[b] = k[-1], v[-1]
        orc.submit(b, k, v)          # the oracle runs while the GPU cache fills
        del k, v
    q = q_tensor(q_bits)
    lens = torch.from_numpy(w.lens).to(DEV)
    got = _bench_step(fused, w, torch.from_numpy(k_new).to(DEV), torch.from_numpy(v_new).to(DEV),
                      q, lens)
    want = _plain_decode(plain, w, q, lens)
    ctx = (w.name, variant, layout)
    _same_cache(fused, plain, ctx)
    assert torch.equal(got.view(torch.int32), want.view(torch.int32)), (ctx, "output differs")
    del fused, plain
    torch.cuda.empty_cache()
    ref, lo, hi = orc.result()
    _gate(got.cpu().numpy(), ref, lo, hi, ctx, literal=True)
