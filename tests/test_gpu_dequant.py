"""GPU parity of the unfused control (fp8kv_dequantize): a stored cache
converted to bf16, bit-exact against the oracle's bf16(fp32(value * scale)),
and attention on the converted cache against the oracle's BF16 mode."""
import numpy as np
import pytest
import torch

import oracle
from fp8_kv_cache_append_amd import binding, synth
from fp8_kv_cache_append_amd.binding import KVCache
from gpu_util import DEV, append_seq, decode, make_cache
from test_gpu_decode import _gate

pytestmark = pytest.mark.gpu


def _bf16_cache_like(src: KVCache) -> KVCache:
    return KVCache.allocate("BF16", int(src.k.shape[0]), src.block_size, src.num_kv_heads,
                            src.head_dim, src.block_table.cpu().numpy(), DEV,
                            layout=src.layout)


def _bits(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("layout", ["token", "head"])
@pytest.mark.parametrize("mode", ["K8V8", "K16V8", "K8V16", "BF16"])
@pytest.mark.parametrize("d", [64, 128])
def test_dequantize_bit_exact_and_attention(mode, d, layout):
    lens = np.array([100, 37], np.int32)
    w = synth.Workload("t", 2, 8, 2, d, lens, "outliers", block_size=16,
                       shuffle_blocks=True, seed=91 + d)
    src = make_cache(mode, w, layout=layout)
    seqs = [synth.kv_sequence(w, b) for b in range(2)]
    for b, (k, v) in enumerate(seqs):
        append_seq(src, b, k, v)
    dst = _bf16_cache_like(src)
    dst.k.fill_(float("nan"))
    dst.v.fill_(float("nan"))
    binding.fp8kv_dequantize(src, dst)
    torch.cuda.synchronize()
    # expected: the oracle's stores of the same rows, converted by the oracle
    table = src.block_table.cpu().numpy()

    def at(x, b, t):  # rows of sequence b's tokens t: [slot][head] or [head][slot]
        blk, slot = table[b, t // 16], t % 16
        return (blk, slot) if layout == "token" else (blk, slice(None), slot)

    want_k = np.zeros(dst.k.shape, np.uint16)
    want_v = np.zeros(dst.v.shape, np.uint16)
    for b, (k, v) in enumerate(seqs):
        st = oracle.store_rows(mode, k, v)
        kb = oracle.dequantize_rows(st["k8"], st["ks"]) if "k8" in st else st["k16"]
        vb = oracle.dequantize_rows(st["v8"], st["vs"]) if "v8" in st else st["v16"]
        t = np.arange(k.shape[0])
        want_k[at(want_k, b, t)] = kb
        want_v[at(want_v, b, t)] = vb
    assert np.array_equal(_bits(dst.k), want_k)
    assert np.array_equal(_bits(dst.v), want_v)
    # attention over the converted cache = the oracle's BF16 mode on those values
    q_bits = synth.q_bf16_bits(w.seed, (2, 8, d))
    got = decode(dst, q_bits, lens, w.group, w.sm_scale)
    keys, vals = [], []
    for b in range(2):
        t = np.arange(int(lens[b]))
        keys.append(oracle.bf16_value(want_k[at(want_k, b, t)]).astype(np.float32))
        vals.append(oracle.bf16_value(want_v[at(want_v, b, t)]).astype(np.float32))
    ref, lo, hi = oracle.decode("BF16", q_bits, keys, vals, w.sm_scale, bounds=True)
    _gate(got, ref, lo, hi, (mode, d, "dequantized"))
