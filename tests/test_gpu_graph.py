"""The entry points under HIP graph capture.

The library allocates nothing, never synchronises and records no memset, so
a caller may capture its calls in a graph (the benchmark times its steps
that way).  Each test captures a call sequence once, then replays the graph
several times with the program's own eager work and synchronisations in
between, and checks every replay bit for bit against the same calls made
eagerly on the same inputs.
"""
import numpy as np
import pytest
import torch

import oracle
from fp8_kv_cache_append_amd import binding, synth
from gpu_util import DEV, append_seq, make_cache, q_tensor
from test_gpu_decode import _gate

pytestmark = pytest.mark.gpu

REPLAYS = 4


def _bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy().view(np.uint32).copy()


def _eager_noise(n: int) -> None:
    """Unrelated eager work between replays (allocations, kernels, a sync)."""
    x = torch.randn(4096 + n, device=DEV)
    y = (x * 3.0 + 1.0).sum()
    torch.cuda.synchronize()
    assert torch.isfinite(y)


def _decode_setup(mode: str):
    lens = np.array([300, 1, 2048, 777], np.int32)
    w = synth.Workload("t", len(lens), 16, 2, 128, lens, "outliers", block_size=16,
                       shuffle_blocks=True, seed=41)
    cache = make_cache(mode, w)
    seqs = [synth.kv_sequence(w, b) for b in range(w.batch)]
    for b, (k, v) in enumerate(seqs):
        append_seq(cache, b, k[:-1], v[:-1])   # the last key comes with the step
    k_new = torch.from_numpy(np.stack([k[-1] for k, _ in seqs])).to(DEV)
    v_new = torch.from_numpy(np.stack([v[-1] for _, v in seqs])).to(DEV)
    q_bits = synth.q_bf16_bits(w.seed, (w.batch, w.q_heads, w.head_dim))
    lens_t = torch.from_numpy(lens).to(DEV)
    max_len = int(lens.max())
    ws_bytes = binding.fp8kv_decode_workspace_bytes(cache, w.batch, w.group, max_len)
    ws = torch.empty(max(ws_bytes // 4, 4), dtype=torch.float32, device=DEV)
    return w, cache, seqs, k_new, v_new, q_bits, lens_t, max_len, ws


@pytest.mark.parametrize("mode", ["K8V8", "K16V8", "BF16"])
def test_decode_append_step_in_graph(mode):
    w, cache, seqs, k_new, v_new, q_bits, lens_t, max_len, ws = _decode_setup(mode)
    q = q_tensor(q_bits)
    out = torch.full((w.batch, w.q_heads, w.head_dim), float("nan"), device=DEV)

    def step():
        binding.fp8kv_decode_append(cache, k_new, v_new, q, w.group, lens_t, max_len,
                                    w.sm_scale, out, ws)

    step()   # eager (also warms up before capture)
    torch.cuda.synchronize()
    eager = _bits(out)
    ref, lo, hi = oracle.decode(mode, q_bits, [s[0] for s in seqs], [s[1] for s in seqs],
                                w.sm_scale, bounds=True)
    _gate(out.cpu().numpy(), ref, lo, hi, (mode, "eager step"))

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for r in range(REPLAYS):
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(_bits(out), eager), (mode, "replay", r)
        _eager_noise(r)


def test_three_kernel_step_in_graph():
    """fp8kv_append, then fp8kv_decode_partial and fp8kv_decode_merge, in one
    graph; replays rewrite the same cache bytes and produce the same output."""
    mode = "K8V8"
    w, cache, seqs, k_new, v_new, q_bits, lens_t, max_len, ws = _decode_setup(mode)
    q = q_tensor(q_bits)
    seq_idx = torch.arange(w.batch, dtype=torch.int32, device=DEV)
    pos = lens_t - 1
    chunk = 256
    splits = -(-max_len // chunk)
    pacc = torch.empty((w.batch, w.kv_heads, splits, w.group, w.head_dim), device=DEV)
    pml = torch.empty((w.batch, w.kv_heads, splits, w.group, 2), device=DEV)
    out = torch.full((w.batch, w.q_heads, w.head_dim), float("nan"), device=DEV)

    def step():
        binding.fp8kv_append(cache, k_new, v_new, seq_idx, pos)
        binding.fp8kv_decode_partial(cache, q, w.group, lens_t, max_len, w.sm_scale, chunk,
                                     splits, pacc, pml)
        binding.fp8kv_decode_merge(w.batch, w.kv_heads, w.group, w.head_dim, splits, pacc,
                                   pml, out)

    step()
    torch.cuda.synchronize()
    eager = _bits(out)
    k_eager = cache.k.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for r in range(REPLAYS):
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(_bits(out), eager), ("replay", r)
        assert torch.equal(cache.k, k_eager), ("cache bytes", r)
        _eager_noise(r)


def test_prefill_in_graph():
    w = synth.prefill_gqa7_d128(tokens=640)
    n = int(w.lens[0])
    cache = make_cache("K8V8", w)
    k, v = synth.kv_sequence(w, 0)
    append_seq(cache, 0, k, v)
    q = q_tensor(synth.q_bf16_bits(w.seed, (n, w.q_heads, w.head_dim)))
    cu = torch.tensor([0, n], dtype=torch.int32, device=DEV)
    pos0 = torch.zeros(1, dtype=torch.int32, device=DEV)
    lens = torch.tensor([n], dtype=torch.int32, device=DEV)
    out = torch.full((n, w.q_heads, w.head_dim), float("nan"), device=DEV)

    def call():
        binding.fp8kv_prefill(cache, q, w.group, cu, pos0, lens, n, w.sm_scale, out)

    call()
    torch.cuda.synchronize()
    eager = _bits(out)
    assert not np.any(np.isnan(out.cpu().numpy()))
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for r in range(REPLAYS):
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(_bits(out), eager), ("replay", r)
        _eager_noise(r)
