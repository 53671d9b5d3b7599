"""Seeded synthetic inputs for the decode and prefill workloads.

This module only draws random numbers and builds index structures (lengths,
block tables).  It holds none of the quantisation or attention arithmetic, so
the GPU path and the CPU oracle can both be fed from it without sharing any of
the method.

Every stream is counter-based: ``numpy.random.default_rng([seed, tag, i])``
for a fixed integer tag per quantity and the sequence (or block) index ``i``,
so one sequence can be regenerated without drawing the others.

Value distributions of the workloads:

* ``normal``   K, V ~ N(0, 1).
* ``outliers`` K, V ~ N(0, 1); each element independently multiplied by 10
  with probability 0.02.
* ``bias``     keys ~ N(0, 1) plus 20 on 8 of the D channels (the same 8
  channels, drawn once from the seed, for every head and token); V ~ N(0, 1).

Q is N(0, 1) rounded to bf16 (round-to-nearest-even, done by torch on the
CPU: an input format, not a step of the method).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

_TAG = {"q": 1, "k": 2, "v": 3, "k_out": 4, "v_out": 5, "bias": 6,
        "lens": 7, "blocks": 8}


def rng(seed: int, tag: str, index: int = 0) -> np.random.Generator:
    return np.random.default_rng([int(seed), _TAG[tag], int(index)])


@dataclass
class Workload:
    """One decode or prefill workload."""
    name: str
    batch: int
    q_heads: int
    kv_heads: int
    head_dim: int
    lens: np.ndarray              # int32 [batch]: keys per sequence
    dist: str = "normal"          # normal | outliers | bias
    block_size: int = 0           # 0: contiguous cache, one block per sequence
    shuffle_blocks: bool = False
    modes: tuple = ("K8V8",)
    prefill: bool = False
    seed: int = 0
    extra: dict = field(default_factory=dict)

    @property
    def group(self) -> int:
        return self.q_heads // self.kv_heads

    @property
    def sm_scale(self) -> float:
        return float(1.0 / np.sqrt(self.head_dim))

    @property
    def max_len(self) -> int:
        return int(self.lens.max()) if self.batch else 0


def decode_b1_gqa4_d64(seed: int = 1) -> Workload:
    """Decode, batch 1, 4 query / 1 KV head, head_dim 64, 128 keys, N(0,1)."""
    return Workload("decode_b1_hq4_hkv1_d64_t128", 1, 4, 1, 64,
                    np.full(1, 128, np.int32), "normal", seed=seed)


def decode_b16_gqa8_d128(tokens: int = 2048, seed: int = 2) -> Workload:
    """Decode, batch 16, 16 query / 2 KV heads, head_dim 128, ``tokens`` keys
    per sequence, N(0,1) with 2 % x10 outliers, contiguous cache."""
    return Workload(f"decode_b16_hq16_hkv2_d128_t{int(tokens)}", 16, 16, 2, 128,
                    np.full(16, int(tokens), np.int32), "outliers",
                    modes=("K8V8", "K16V8", "BF16"), seed=seed)


def decode_b64_gqa4_ragged_paged(seed: int = 4) -> Workload:
    """Decode, batch 64, 32 query / 8 KV heads, head_dim 128, lengths uniform
    in [1024, 32768], 16-token blocks behind a shuffled table, keys biased by
    +20 on 8 channels."""
    lens = rng(seed, "lens").integers(1024, 32768, size=64, endpoint=True)
    return Workload("decode_b64_hq32_hkv8_d128_ragged_paged16", 64, 32, 8, 128,
                    lens.astype(np.int32), "bias", block_size=16,
                    shuffle_blocks=True, modes=("K8V8", "K16V8"), seed=seed)


def prefill_gqa7_d128(tokens: int = 2048, seed: int = 5) -> Workload:
    """Causal prefill of one sequence, 28 query / 4 KV heads, head_dim 128."""
    return Workload(f"prefill_b1_t{tokens}_hq28_hkv4_d128", 1, 28, 4, 128,
                    np.full(1, tokens, np.int32), "normal", prefill=True, seed=seed)


def q_bf16_bits(seed: int, shape, index: int = 0) -> np.ndarray:
    """N(0, 1) queries rounded to bf16, as uint16 bit patterns."""
    import torch
    x = rng(seed, "q", index).standard_normal(size=shape, dtype=np.float32)
    t = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16)
    return t.numpy().view(np.uint16).copy()


def bias_channels(seed: int, head_dim: int) -> np.ndarray:
    return np.sort(rng(seed, "bias").choice(head_dim, size=8, replace=False))


def kv_sequence(w: Workload, b: int, n: int | None = None):
    """fp32 K and V of sequence ``b``: arrays [n, kv_heads, head_dim]."""
    n = int(w.lens[b]) if n is None else int(n)
    shape = (n, w.kv_heads, w.head_dim)
    k = rng(w.seed, "k", b).standard_normal(size=shape, dtype=np.float32)
    v = rng(w.seed, "v", b).standard_normal(size=shape, dtype=np.float32)
    if w.dist == "outliers":
        k[rng(w.seed, "k_out", b).random(size=shape) < 0.02] *= np.float32(10.0)
        v[rng(w.seed, "v_out", b).random(size=shape) < 0.02] *= np.float32(10.0)
    elif w.dist == "bias":
        k[:, :, bias_channels(w.seed, w.head_dim)] += np.float32(20.0)
    elif w.dist != "normal":
        raise ValueError(w.dist)
    return k, v


def kv_sequence_prebias(w: Workload, b: int):
    """The ``bias`` workload split into its parts: the token-varying
    residual of K (the N(0, 1) draw of kv_sequence, before the bias is
    added), V, and the fixed K bias, fp32 [kv_heads, head_dim] (20 on the 8
    seeded channels of every head, 0 elsewhere).  kv_sequence's K is the
    fp32 sum of the first and the last."""
    if w.dist != "bias":
        raise ValueError("pre-bias parts exist for the bias workload only")
    n = int(w.lens[b])
    shape = (n, w.kv_heads, w.head_dim)
    k = rng(w.seed, "k", b).standard_normal(size=shape, dtype=np.float32)
    v = rng(w.seed, "v", b).standard_normal(size=shape, dtype=np.float32)
    bias = np.zeros((w.kv_heads, w.head_dim), np.float32)
    bias[:, bias_channels(w.seed, w.head_dim)] = np.float32(20.0)
    return k, v, bias


def block_layout(w: Workload, capacity: int | None = None):
    """Block size, block table [batch, max_blocks] int32 and block count.

    Contiguous: one block of ``capacity`` (default max_len, rounded up to a
    multiple of 16) tokens per sequence and block_table[b] = [b].  Paged: ceil(len_b / block_size)
    blocks per sequence, numbered 0..n-1 in order or by a seeded random
    permutation; unused table entries are -1.
    """
    if w.block_size == 0:
        cap = w.max_len if capacity is None else int(capacity)
        cap = max(16, -(-cap // 16) * 16)  # block sizes are multiples of 16
        table = np.arange(w.batch, dtype=np.int32).reshape(w.batch, 1)
        return cap, table, w.batch
    bs = w.block_size
    cap = w.lens if capacity is None else np.maximum(w.lens, capacity)
    per = (np.asarray(cap, np.int64) + bs - 1) // bs
    n_blocks = int(per.sum())
    ids = np.arange(n_blocks, dtype=np.int32)
    if w.shuffle_blocks:
        ids = rng(w.seed, "blocks").permutation(n_blocks).astype(np.int32)
    width = int(per.max()) if w.batch else 1
    table = np.full((w.batch, max(width, 1)), -1, dtype=np.int32)
    start = 0
    for b in range(w.batch):
        table[b, :per[b]] = ids[start:start + per[b]]
        start += int(per[b])
    return bs, table, n_blocks


def kv_sequence_device(w: Workload, b: int, device="cuda", residual: bool = False):
    """fp32 K and V of sequence ``b`` drawn on the device (torch's seeded
    generator): the same distributions as kv_sequence, other values.  For
    benchmark caches of gigabytes, where host generation would dominate.
    residual=True (bias workload): K without its bias, the rows a pre-bias
    cache stores; the bias is kv_sequence_prebias's."""
    import torch
    n = int(w.lens[b])
    g = torch.Generator(device=device)
    g.manual_seed((int(w.seed) * 1_000_003 + int(b)) * 7 + 1)
    shape = (n, w.kv_heads, w.head_dim)
    k = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    v = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if w.dist == "outliers":
        k = torch.where(torch.rand(shape, generator=g, device=device) < 0.02, k * 10.0, k)
        v = torch.where(torch.rand(shape, generator=g, device=device) < 0.02, v * 10.0, v)
    elif w.dist == "bias":
        if not residual:
            ch = torch.from_numpy(bias_channels(w.seed, w.head_dim)).to(device)
            k[:, :, ch] += 20.0
    elif w.dist != "normal":
        raise ValueError(w.dist)
    return k, v
