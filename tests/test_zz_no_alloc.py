"""fp8kv_decode_noalloc: fp8kv_decode with the split partials in the
library's own device scratch instead of a caller workspace.  Through the C
ABI, on two calls in a row (the second smaller, so it runs over what the
first left in the scratch) and against fp8kv_decode on the same inputs: the
same kernels and plan, so the outputs must be bit-identical; both also meet
the oracle gate.  A request whose partials exceed the scratch is refused
with FP8KV_ERR_TOO_LARGE before anything is enqueued."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from fp8_kv_cache_append_amd import binding, synth
from gpu_util import DEV, append_seq, decode, make_cache, q_tensor
from test_gpu_decode import _gate

pytestmark = pytest.mark.gpu


def _noalloc(cache, q_bits, lens, group, sm_scale):
    lens = np.asarray(lens, np.int32)
    b, hq, d = q_bits.shape
    out = torch.full((b, hq, d), float("nan"), dtype=torch.float32, device=DEV)
    binding.fp8kv_decode_noalloc(cache, q_tensor(q_bits), group, torch.from_numpy(lens).to(DEV),
                                 int(lens.max()), sm_scale, out)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def _case(mode, w):
    seqs = [synth.kv_sequence(w, b) for b in range(w.batch)]
    cache = make_cache(mode, w)
    for b, (k, v) in enumerate(seqs):
        append_seq(cache, b, k, v)
    q_bits = synth.q_bf16_bits(w.seed, (w.batch, w.q_heads, w.head_dim))
    return cache, seqs, q_bits


@pytest.mark.parametrize("mode", ["K8V8", "K16V8"])
def test_noalloc_matches_workspace_decode_twice(mode):
    big = synth.Workload("t", 16, 16, 2, 128, np.array([2048, 1, 700, 4096] * 4, np.int32),
                         "outliers", block_size=16, shuffle_blocks=True, seed=91)
    small = synth.Workload("t", 3, 8, 2, 64, np.array([300, 0, 65], np.int32), "outliers",
                           seed=92)
    for w in (big, small):       # the second call is smaller than the first
        cache, seqs, q_bits = _case(mode, w)
        got = _noalloc(cache, q_bits, w.lens, w.group, w.sm_scale)
        want = decode(cache, q_bits, w.lens, w.group, w.sm_scale)
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), (mode, w.batch)
        ref, lo, hi = oracle.decode(mode, q_bits, [s[0] for s in seqs], [s[1] for s in seqs],
                                    w.sm_scale, bounds=True)
        _gate(got, ref, lo, hi, (mode, "noalloc", w.batch))
        assert np.all(got[w.lens == 0] == 0)


def test_noalloc_refuses_requests_beyond_its_scratch():
    w = synth.Workload("t", 2, 16, 2, 128, np.array([64, 64], np.int32), "normal", seed=3)
    cache = make_cache("K8V8", w)
    d = cache.desc()
    lib = binding.lib()
    need = lib.fp8kv_decode_workspace_bytes(ctypes.byref(d), 2, 8, 64)
    assert 0 < need <= 64 << 20
    # a paged cache of 2^20 keys per sequence x 64 sequences x 8 KV heads
    huge = binding.CacheDesc(0, 1, 16, 8, 128, 1 << 16, 64, d.k, d.v, d.k_scale, d.v_scale,
                             d.block_table, None, None)
    assert lib.fp8kv_decode_workspace_bytes(ctypes.byref(huge), 64, 4, 1 << 20) > 64 << 20
    out = torch.empty((64, 32, 128), device=DEV)
    st = lib.fp8kv_decode_noalloc(ctypes.byref(huge), d.k, 4, d.block_table, 64, 1 << 20, 0.1,
                                  out.data_ptr(), None)
    assert st == binding.FP8KV_ERR_TOO_LARGE
    assert "scratch" in binding.strerror(st)
