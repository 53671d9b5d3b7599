"""Benchmark: KV-cache GB/s (% of 8 TB/s) and us per decode step, K8V8 vs
K16V8 vs BF16, on one MI355X.

Step: one decode step of batch 16, 16 query / 2 KV heads (GQA 8), head_dim
128, 2048 keys per sequence (e4m3 K/V, N(0,1) with 2 % x10 outliers),
through the library's entry point fp8kv_decode_append, which launches
  the split kernel, which also quantises and stores each sequence's new
    token (position 2047) and attends it (fp8kv_decode_append_partial);
  the merge kernel (fp8kv_decode_merge), unless the plan has one split of
    at most 256 keys, whose output the split kernel writes itself.
The same step as three kernels (fp8kv_append, fp8kv_decode_partial,
fp8kv_decode_merge) is timed too and reported as unfused_step_us, and the
unfused control -- append, the whole cache dequantised to bf16 in HBM
(fp8kv_dequantize), BF16 split + merge on the copy -- as
dequant_then_bf16_step_us.

Protocol.  The headline value is K8V8 KV bytes per step / time per step,
HBM-cold: the step rotates over 64 copies of the cache (> 1 GB, larger than
the 256 MB Infinity Cache), so no copy is cache-resident when it is read.
Steps are replayed from HIP graphs of one rotation (and of the remainder),
so exactly --warmup untimed steps run, then exactly --steps timed steps
between two events with a synchronisation on both sides (no host launch
cost inside the timed region).  Then each step form (fused step, split
kernel alone, three-kernel step, narrow QK, unfused control) is replayed a
number of whole rotations, each between its own events, for the median and
10th / 90th percentiles of the per-replay means; the roofline's duration is
the split kernel's median.  Per-kernel durations also come from HIP event
pairs around each kernel of one eager rotation, enqueued behind a replay.
Before anything is timed, every timed output is checked on sampled rows
against a plain torch / numpy fp64 reference computed from the cache bytes
(reference_rows; parity against the oracle is the test suite's), and the
headline step's output against the oracle's own output of the same step in
the CPU-baseline leg.

Narrow QK (fp8kv_decode_append_q8: Q quantised to e4m3 in the split kernel,
fp8 QK) is timed on the same rotation for the e4m3-K modes
(narrow_qk_step_us), with its output's relative L2 against the bf16-Q step
(narrow_qk_vs_bf16q_rel_l2: the Q rounding's cost).

Extra fields: the K16V8 and BF16 controls (same protocol); two floors for
one launch moving the step's KV bytes under the same rotation -- a device
copy (read + write, copy_floor_same_bytes) and a plain streaming read
(read_floor_same_bytes); the bulk append kernel's rate (append_bulk: 1M
rows into a paged K8V8 cache); the op-level error of each quantised cache
(fp8_vs_bf16_rel_l2: the step's output against the BF16-cache step's on the
same inputs); the L2/MALL-warm rate (one copy, labelled); the causal prefill
of 2048 tokens (28/4 heads; K8V8 and the BF16 cache as its matrix-core
control); the batch-1 4q/1kv D64 128-key step; the context sweep of the
headline shape at 77/512/2048/8192 keys in all four modes (K8V16 isolates
the K side) with the K8V8-vs-K16V8 break-even and the per-side savings
against BF16; a GQA-group sweep (G 1/4/8/16 at 8192 keys) and a batch sweep
(1/4/16/64 at 2048 keys), K8V8 against BF16; the ragged batch-64 paged
workload (32q/8kv, lengths 1024..32768, K8V8, K16V8 and K8V8 as a pre-bias
residual cache with the exact key bias, in the head-major layout, and K8V8
token-major beside them) and a page-size sweep (16/32/64/256 tokens) on its
first 16 sequences; block-scaled K (MXK8V8) against per-row
K8V8 with bf16 Q and with fp8 QK (block_scaled_k); the roofline of the split
kernel and the CPU oracle as a baseline.  Rotations of the sweeps hold at
least 1 GiB of cache (fewer copies only where a copy is tiny, labelled).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
BF16_MFMA_PEAK_TFLOPS = 2500.0
ROW_BYTES = {"K8V8": lambda d: 2 * d + 8, "K16V8": lambda d: 3 * d + 4, "BF16": lambda d: 4 * d,
             "K8V16": lambda d: 3 * d + 4}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_split_k8v8_b16_t2048_traffic.json")
KERNEL_SOURCES = ["fp8_kv_cache_append_amd/csrc/decode.hip",
                  "fp8_kv_cache_append_amd/csrc/device.h",
                  "fp8_kv_cache_append_amd/csrc/launch.h"]


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def pctl(samples_ms) -> dict:
    """Median and 10th / 90th percentiles of per-replay mean times, in us."""
    x = np.asarray(samples_ms, np.float64) * 1e3
    return {"median": float(np.median(x)), "p10": float(np.percentile(x, 10)),
            "p90": float(np.percentile(x, 90)), "replays": int(x.size)}


class GraphTimer:
    """HIP graphs of consecutive calls fn(0), fn(1), ... over a rotation of
    `copies` inputs: one graph of a whole rotation, and one of the remainder,
    so that exactly n calls can be replayed (no host launch cost inside a
    timed region; HIP cannot time events recorded inside a graph)."""

    def __init__(self, torch, fn, copies: int):
        self.torch, self.fn, self.copies = torch, fn, copies
        self.graphs = {}

    def graph(self, n: int):
        if n not in self.graphs:
            torch = self.torch
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for i in range(n):
                    self.fn(i)
            torch.cuda.synchronize()
            self.graphs[n] = g
        return self.graphs[n]

    def run(self, n_calls: int) -> None:
        """Enqueue exactly n_calls calls (whole rotations, then the rest)."""
        full, rest = divmod(int(n_calls), self.copies)
        for _ in range(full):
            self.graph(self.copies).replay()
        if rest:
            self.graph(rest).replay()

    def time(self, n_calls: int) -> float:
        """ms per call over exactly n_calls calls, between two events, with a
        synchronisation on both sides."""
        torch = self.torch
        self.graph(self.copies)
        if n_calls % self.copies:
            self.graph(n_calls % self.copies)
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0.record()
        self.run(n_calls)
        t1.record()
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) / n_calls

    def samples(self, replays: int) -> list:
        """Mean ms per call of each of `replays` whole-rotation replays, each
        between its own pair of events."""
        torch = self.torch
        g = self.graph(self.copies)
        g.replay()
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(replays)]
        for a, b in ev:
            a.record()
            g.replay()
            b.record()
        torch.cuda.synchronize()
        return [a.elapsed_time(b) / self.copies for a, b in ev]


# ---------------------------------------------------------------------------
# Sanity check of what is timed: a plain torch / numpy fp64 reference of the
# attention on sampled rows, computed from the cache bytes the kernels read
# (e4m3 codes decoded through torch's float8_e4m3fn type).  It is independent
# of the HIP kernels and of the oracle (parity against the oracle is the test
# suite's job); a timed kernel whose output strays from it beyond the
# contract's figures is reported as not validated.

LOG2E = 1.4426950408889634
_E4M3 = None


def _e4m3_values():
    global _E4M3
    if _E4M3 is None:
        import torch
        _E4M3 = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(
            torch.float8_e4m3fn).double().numpy()
    return _E4M3


def _bf16_round(x):
    """fp64 -> fp32 -> bf16 (nearest even, torch) -> fp64."""
    import torch
    return torch.from_numpy(np.asarray(x, np.float64)).float().to(torch.bfloat16).double().numpy()


def _e4m3_round(x32):
    import torch
    return _e4m3_values()[torch.from_numpy(np.asarray(x32, np.float32)).to(
        torch.float8_e4m3fn).view(torch.uint8).numpy().astype(np.int64)]


def _cache_rows(cache, b, h, n):
    """fp64 K, V [n, D] and the per-token factors ks, vs [n] of (sequence b,
    KV head h), read back from the cache through its block table."""
    import torch
    bs = cache.block_size
    table = cache.block_table[b].cpu().numpy()
    t = np.arange(n)
    blk = torch.from_numpy(table[t // bs].astype(np.int64)).to(cache.k.device)
    slot = torch.from_numpy((t % bs).astype(np.int64)).to(cache.k.device)
    tab = _e4m3_values()

    def row(x):  # rows of a block: [slot][head] or [head][slot]
        return x[blk, slot, h] if cache.layout == "token" else x[blk, h, slot]

    def side(x):
        r = row(x).cpu()
        if r.dtype == torch.uint8:
            return tab[r.numpy().astype(np.int64)]
        return r.double().numpy()

    k, v = side(cache.k), side(cache.v)
    if cache.k_exp is not None:   # block-scaled K: 2^(E - 127) per 32 values
        e = row(cache.k_exp).cpu().numpy().astype(np.float64)
        k = k * np.repeat(np.exp2(e - 127.0), 32, axis=1)
    ks = row(cache.k_scale).cpu().double().numpy() if cache.k_scale is not None else np.ones(n)
    vs = row(cache.v_scale).cpu().double().numpy() if cache.v_scale is not None else np.ones(n)
    return k, v, ks, vs


def _query_values(qrows, narrow, mx):
    """bf16 query rows as fp64 values and their per-row factor; narrow QK:
    the rows quantised by the cache-row rule (per row, or per 32 values with
    a power-of-two scale for block-scaled K)."""
    q = qrows.astype(np.float64)
    if not narrow:
        return q, np.ones(q.shape[0])
    if mx:
        blocks = q.reshape(q.shape[0], -1, 32)
        s = (np.abs(blocks).max(axis=2).astype(np.float32) / np.float32(448.0)).astype(np.float64)
        m, e = np.frexp(np.maximum(s, 2.0 ** -126))
        e = np.clip(np.where(m == 0.5, e - 1, e), -126, 127).astype(np.float64)
        codes = _e4m3_round((blocks / np.exp2(e)[..., None]).astype(np.float32))
        return (codes * np.exp2(e)[..., None]).reshape(q.shape), np.ones(q.shape[0])
    qs = (np.abs(q).max(axis=1).astype(np.float32) / np.float32(448.0)).astype(np.float64)
    safe = np.where(qs > 0, qs, 1.0)
    codes = _e4m3_round((q.astype(np.float32) / safe[:, None].astype(np.float32)))
    return np.where(qs[:, None] > 0, codes, 0.0), qs


def reference_rows(cache, q_bits, group, sm_scale, items, narrow=False):
    """items: (b, h, n_keys per query row of the head group, output row
    index); returns fp64 [len(items), G, D] of the two-pass attention with
    the integer log2 reference and bf16 P (v_scale folded in)."""
    c = float(np.float32(np.float64(np.float32(sm_scale)) * LOG2E))
    mx = cache.k_exp is not None
    out = []
    for b, h, n_keys, qi in items:
        n = int(max(n_keys))
        k, v, ks, vs = _cache_rows(cache, b, h, n)
        rows = q_bits[qi][h * group:(h + 1) * group].astype(np.uint32) << 16
        q, qf = _query_values(rows.view(np.float32), narrow, mx)
        s = (q @ k.T) * ks[None, :] * qf[:, None]
        if cache.k_bias is not None:
            s = s + (q @ cache.k_bias[h].cpu().double().numpy())[:, None]
        s = s * c
        mask = np.arange(n)[None, :] < np.asarray(n_keys)[:, None]
        s = np.where(mask, s, -np.inf)
        m = np.ceil(s.max(axis=1, keepdims=True))
        p = np.where(mask, np.exp2(s - m), 0.0)
        w = _bf16_round(p * vs[None, :])
        out.append((w @ v) / p.sum(axis=1, keepdims=True))
    return np.stack(out)


def check_rows(got_rows, ref_rows, gate_rel=1e-3, gate_abs=5e-3) -> dict:
    got = np.asarray(got_rows, np.float64)
    ref = np.asarray(ref_rows, np.float64)
    rel = float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300))
    mab = float(np.max(np.abs(got - ref))) if got.size else 0.0
    return {"validated": bool(rel <= gate_rel and mab <= gate_abs and np.all(np.isfinite(got))),
            "rel_l2": rel, "max_abs": mab, "gate_rel_l2": gate_rel, "gate_max_abs": gate_abs}


def validate_decode(cache, q, out, lens, group, sm_scale, pairs, narrow=False):
    """The decode output `out` (device [B, Hq, D]) of sampled (sequence, KV
    head) pairs against reference_rows."""
    q_bits = q.view(__import__("torch").int16).cpu().numpy().view(np.uint16)
    lens = np.asarray(lens)
    items = [(b, h, np.full(group, int(lens[b])), b) for b, h in pairs]
    ref = reference_rows(cache, q_bits, group, sm_scale, items, narrow)
    o = out.cpu().numpy()
    got = np.stack([o[b, h * group:(h + 1) * group] for b, h in pairs])
    if narrow:
        # the fp8 matrix instruction sums its products only to ~2^-12 of their
        # absolute sum, so narrow-QK scores carry that noise, and through
        # rows that weigh two keys (x10 outlier values) an output can move by
        # ~0.1; its figure is the relative L2 (the test suite gates it inside
        # the oracle's rounding interval)
        r = check_rows(got, ref, gate_rel=5e-3, gate_abs=float("inf"))
    else:
        r = check_rows(got, ref)
    r["sample"] = f"{len(pairs)} (sequence, KV head) pairs, all their query heads"
    return r


class DecodeBench:
    """Rotating copies of one decode workload plus the graph of one rotation."""

    def __init__(self, mode: str, w, copies: int, warm: bool = False, layout: str = "token"):
        import torch
        from fp8_kv_cache_append_amd import binding, synth
        from fp8_kv_cache_append_amd.binding import KVCache

        self.torch, self.binding = torch, binding
        self.mode, self.w, self.copies, self.warm = mode, w, copies, warm
        dev = "cuda"
        n = int(w.lens[0])
        bs, table, n_blocks = synth.block_layout(w)
        # a contiguous cache is passed without a table (the library computes the ids)
        mem_table = w.block_size != 0
        base = KVCache.allocate(mode, n_blocks, bs, w.kv_heads, w.head_dim, table, dev,
                                table_in_memory=mem_table, layout=layout)
        last_k, last_v = [], []
        for b in range(w.batch):
            k, v = synth.kv_sequence(w, b)
            binding.fp8kv_append(base, torch.from_numpy(k).to(dev), torch.from_numpy(v).to(dev),
                                 torch.full((n,), b, dtype=torch.int32, device=dev),
                                 torch.arange(n, dtype=torch.int32, device=dev))
            last_k.append(k[-1])
            last_v.append(v[-1])
        n_copies = 1 if warm else copies
        self.caches = [base] + [KVCache(mode, base.k.clone(), base.v.clone(),
                                        None if base.k_scale is None else base.k_scale.clone(),
                                        None if base.v_scale is None else base.v_scale.clone(),
                                        base.block_table, table_in_memory=mem_table,
                                        layout=base.layout)
                                for _ in range(n_copies - 1)]
        # the new token of each sequence, appended at its last position
        self.k_new = torch.from_numpy(np.stack(last_k)).to(dev)
        self.v_new = torch.from_numpy(np.stack(last_v)).to(dev)
        self.seq_idx = torch.arange(w.batch, dtype=torch.int32, device=dev)
        self.pos = torch.full((w.batch,), n - 1, dtype=torch.int32, device=dev)
        q_bits = synth.q_bf16_bits(w.seed, (w.batch, w.q_heads, w.head_dim))
        self.q = torch.from_numpy(q_bits.view(np.int16)).to(dev).view(torch.bfloat16)
        self.lens = torch.from_numpy(w.lens.astype(np.int32)).to(dev)
        self.max_len = n
        self.chunk, self.splits = binding.fp8kv_decode_plan(base, w.batch, w.group, n)
        g, d = w.group, w.head_dim
        self.pacc = torch.empty((w.batch, w.kv_heads, self.splits, g, d), device=dev)
        self.pml = torch.empty((w.batch, w.kv_heads, self.splits, g, 2), device=dev)
        self.out = torch.empty((w.batch, w.q_heads, d), device=dev)
        self.kv_bytes = int(w.lens.sum()) * w.kv_heads * ROW_BYTES[mode](d)
        # narrow QK (Q quantised to e4m3 in the kernel): e4m3-K modes only
        self.narrow = mode in ("K8V8", "K8V16")
        ws_bytes = binding.fp8kv_decode_workspace_bytes(base, w.batch, g, n)
        self.ws = torch.empty(ws_bytes // 4 + 4, device=dev)
        if self.narrow:
            self.out_q8 = torch.empty_like(self.out)
        self.graph = None
        self.dq = None
        if mode == "K8V8":
            # the unfused control: the cache dequantised to bf16 in HBM, then
            # the BF16 kernels on the copy
            self.dq = KVCache.allocate("BF16", n_blocks, bs, w.kv_heads, d, table, dev,
                                       table_in_memory=mem_table, layout=layout)
            self.dq_chunk, self.dq_splits = binding.fp8kv_decode_plan(self.dq, w.batch, g, n)
            self.dq_pacc = torch.empty((w.batch, w.kv_heads, self.dq_splits, g, d), device=dev)
            self.dq_pml = torch.empty((w.batch, w.kv_heads, self.dq_splits, g, 2), device=dev)

    def split(self, i: int):
        """The step's first kernel: fused append of the new token + split
        partials."""
        w = self.w
        self.binding.fp8kv_decode_append_partial(
            self.caches[i % len(self.caches)], self.k_new, self.v_new, self.q, w.group,
            self.lens, self.max_len, w.sm_scale, self.chunk, self.splits, self.pacc, self.pml)

    def step(self, i: int, ev=None):
        """One decode step through fp8kv_decode_append: append each
        sequence's new token (fused into the split kernel), split partials,
        merge (none for a plan of one split).  With events (kernel_events):
        the split and merge kernels through their own entry points, an event
        pair around each."""
        b, w = self.binding, self.w
        if ev is None:
            b.fp8kv_decode_append(self.caches[i % len(self.caches)], self.k_new, self.v_new,
                                  self.q, w.group, self.lens, self.max_len, w.sm_scale,
                                  self.out, self.ws)
            return
        ev[0].record()
        self.split(i)
        ev[1].record()
        b.fp8kv_decode_merge(w.batch, w.kv_heads, w.group, w.head_dim, self.splits,
                             self.pacc, self.pml, self.out)
        ev[2].record()

    def step_q8(self, i: int):
        """The same step with narrow QK (fp8kv_decode_append_q8: the same two
        kernels, Q quantised in the split kernel, fp8 QK)."""
        w = self.w
        self.binding.fp8kv_decode_append_q8(
            self.caches[i % len(self.caches)], self.k_new, self.v_new, self.q, w.group,
            self.lens, self.max_len, w.sm_scale, self.out_q8, self.ws)

    def step_unfused(self, i: int):
        """The same step as three kernels: append, split, merge."""
        b, w = self.binding, self.w
        c = self.caches[i % len(self.caches)]
        b.fp8kv_append(c, self.k_new, self.v_new, self.seq_idx, self.pos)
        b.fp8kv_decode_partial(c, self.q, w.group, self.lens, self.max_len, w.sm_scale,
                               self.chunk, self.splits, self.pacc, self.pml)
        b.fp8kv_decode_merge(w.batch, w.kv_heads, w.group, w.head_dim, self.splits,
                             self.pacc, self.pml, self.out)

    def step_unfused_dequant(self, i: int):
        """The unfused control's step: append, dequantise the whole cache to
        bf16, BF16 split + merge over the copy."""
        b, w = self.binding, self.w
        c = self.caches[i % len(self.caches)]
        b.fp8kv_append(c, self.k_new, self.v_new, self.seq_idx, self.pos)
        b.fp8kv_dequantize(c, self.dq)
        b.fp8kv_decode_partial(self.dq, self.q, w.group, self.lens, self.max_len, w.sm_scale,
                               self.dq_chunk, self.dq_splits, self.dq_pacc, self.dq_pml)
        b.fp8kv_decode_merge(w.batch, w.kv_heads, w.group, w.head_dim, self.dq_splits,
                             self.dq_pacc, self.dq_pml, self.out)

    def capture(self):
        """Eager calls first (the library's one-time device check), then a
        graph timer per step form; graphs are captured on first use."""
        torch = self.torch
        self.step(0)
        self.step_unfused(0)
        torch.cuda.synchronize()
        T = lambda fn: GraphTimer(torch, fn, self.copies)
        self.t_step, self.t_split, self.t_unfused = T(self.step), T(self.split), T(self.step_unfused)
        self.t_q8 = self.t_dq = None
        if self.narrow:
            self.step_q8(0)
            self.t_q8 = T(self.step_q8)
        if self.dq is not None:
            self.step_unfused_dequant(0)
            self.t_dq = T(self.step_unfused_dequant)
        torch.cuda.synchronize()

    def kernel_events(self):
        """One rotation launched eagerly with an event pair around every
        kernel on the launch stream, enqueued while the GPU is still busy
        with a whole-rotation replay, so no host launch gap falls inside a
        pair: each pair brackets exactly one kernel.  Mean durations (ms) of
        the split kernel (with the fused append) and the merge kernel."""
        torch = self.torch
        torch.cuda.synchronize()
        self.t_step.graph(self.copies).replay()
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)]
              for _ in range(self.copies)]
        for i in range(self.copies):
            self.step(i, ev[i])
        torch.cuda.synchronize()
        spl = [ev[i][0].elapsed_time(ev[i][1]) for i in range(self.copies)]
        mrg = [ev[i][1].elapsed_time(ev[i][2]) for i in range(self.copies)]
        return float(np.mean(spl)), float(np.mean(mrg))

    def sample_pairs(self, n=4):
        """(sequence, KV head) pairs for the sanity check: first, last and
        spread sequences, every KV head in turn."""
        bsz, hkv = self.w.batch, self.w.kv_heads
        seqs = sorted({0, bsz - 1, bsz // 2, bsz // 3})[:n]
        return [(b, (i * 3 + 1) % hkv) for i, b in enumerate(seqs)] + [(0, 0)]

    def validate(self):
        """The fused step's output on copy 0 (and the narrow-QK step's)
        against the torch reference on sampled rows."""
        w, torch = self.w, self.torch
        self.step(0)
        torch.cuda.synchronize()
        pairs = self.sample_pairs()
        res = validate_decode(self.caches[0], self.q, self.out, w.lens, w.group, w.sm_scale, pairs)
        if self.narrow:
            self.step_q8(0)
            torch.cuda.synchronize()
            res["narrow_qk"] = validate_decode(self.caches[0], self.q, self.out_q8, w.lens,
                                               w.group, w.sm_scale, pairs, narrow=True)
            res["validated"] = res["validated"] and res["narrow_qk"]["validated"]
        return res


def step_output(bench):
    """The output of one decode step on the bench's first cache copy (fp64,
    on the device): every mode's bench holds the same seeded inputs."""
    bench.step(0)
    bench.torch.cuda.synchronize()
    return bench.out.double().clone()


def cold_copies(mode, w, at_least=64, total=1 << 30, cap=2048) -> int:
    """Copies in a rotation whose caches total at least 1 GiB (larger than
    the 256 MB Infinity Cache and the eight 4 MB L2s), so that no copy is
    resident when it is read again; capped for tiny workloads (then the
    rotation is cache-resident and the figure is labelled so)."""
    kv = int(w.lens.sum()) * w.kv_heads * ROW_BYTES[mode](w.head_dim)
    return int(min(cap, max(at_least, math.ceil(total / max(kv, 1)))))


def bench_decode(mode, w, steps, warmup, copies, replays=8, layout="token"):
    """Warm up with exactly `warmup` steps, time exactly `steps` steps (the
    headline figures), then `replays` whole-rotation replays of each step
    form, each between its own events, for the median and 10th / 90th
    percentiles.  The outputs are checked before any timing."""
    bench = DecodeBench(mode, w, copies, layout=layout)
    bench.capture()
    valid = bench.validate()
    bench.t_step.run(warmup)
    step_ms = bench.t_step.time(steps)
    spl, mrg = bench.kernel_events()
    st = {name: pctl(t.samples(replays)) for name, t in
          (("step", bench.t_step), ("split", bench.t_split), ("unfused", bench.t_unfused),
           ("narrow_qk", bench.t_q8), ("dequant_then_bf16", bench.t_dq)) if t is not None}
    q8_err = None
    if bench.t_q8 is not None:
        # narrow against bf16-Q outputs of the same step on the same cache
        bench.step(0)
        bench.step_q8(0)
        bench.torch.cuda.synchronize()
        a = bench.out_q8.double()
        r = bench.out.double()
        q8_err = float(((a - r).norm() / r.norm()).item())
    res = {"ms_per_step": step_ms, "steps": int(steps), "warmup": int(warmup),
           "kv_bytes": bench.kv_bytes,
           "kv_gbs": bench.kv_bytes / (step_ms * 1e-3) / 1e9,
           "kernel_us_event_pairs": {"split_with_append": spl * 1e3, "merge": mrg * 1e3},
           "split_us": st["split"]["median"],
           "step_us_stats": st["step"], "split_us_stats": st["split"],
           "unfused_step_us": st["unfused"]["median"],
           "dequant_then_bf16_step_us": st["dequant_then_bf16"]["median"]
           if "dequant_then_bf16" in st else None,
           "narrow_qk_step_us": st["narrow_qk"]["median"] if "narrow_qk" in st else None,
           "narrow_qk_vs_bf16q_rel_l2": q8_err,
           "validation": valid, "layout": layout,
           "split_plan": {"chunk_tokens": bench.chunk, "n_splits": bench.splits}}
    res["pct_roofline"] = 100.0 * res["kv_gbs"] / HBM_PEAK_GBS
    return res, bench


def bench_sweep(steps, warmup, copies, head):
    """The context sweep of the B16 16q/2kv D128 shape at 77, 512, 2048 and
    8192 keys, all four modes, HBM-cold as the headline; the K8V8-vs-K16V8
    break-even is the first length where the K8V8 step is faster (linear
    interpolation of the step time over the swept lengths)."""
    from fp8_kv_cache_append_amd import synth

    table = {}
    for tokens in (77, 512, 2048, 8192):
        w = synth.decode_b16_gqa8_d128(tokens)
        row = {}
        for mode in ("K8V8", "K16V8", "BF16", "K8V16"):
            if tokens == 2048 and mode == "K8V8":
                r = head
            else:
                r, _ = bench_decode(mode, w, steps, warmup, cold_copies(mode, w, copies))
            row[mode] = {"us_per_step": r["ms_per_step"] * 1e3, "split_us": r["split_us"],
                         "kv_gbs": r["kv_gbs"], "pct_roofline": r["pct_roofline"],
                         "step_us_p10_p90": [r["step_us_stats"]["p10"], r["step_us_stats"]["p90"]],
                         "unfused_step_us": r["unfused_step_us"],
                         "narrow_qk_step_us": r["narrow_qk_step_us"],
                         "validated": r["validation"]["validated"],
                         "copies": cold_copies(mode, w, copies)}
        row["K8V8_speedup_vs_K16V8"] = row["K16V8"]["us_per_step"] / row["K8V8"]["us_per_step"]
        row["K8V8_speedup_vs_BF16"] = row["BF16"]["us_per_step"] / row["K8V8"]["us_per_step"]
        # time the BF16 control saves by storing one side in e4m3 ("Account
        # for V preparation"): K side alone (K8V16), V side alone (K16V8),
        # both (K8V8); the fraction hidden is the both-sides saving over the
        # sum of the single-side ones
        t_bf16 = row["BF16"]["us_per_step"]
        sav_k = t_bf16 - row["K8V16"]["us_per_step"]
        sav_v = t_bf16 - row["K16V8"]["us_per_step"]
        sav_kv = t_bf16 - row["K8V8"]["us_per_step"]
        row["saving_us"] = {"K_only": sav_k, "V_only": sav_v, "K_and_V": sav_kv}
        table[str(tokens)] = row
    lens = [77, 512, 2048, 8192]
    diff = [table[str(t)]["K16V8"]["us_per_step"] - table[str(t)]["K8V8"]["us_per_step"]
            for t in lens]
    be = None
    if diff[0] > 0:
        be = f"<= {lens[0]}"
    else:
        for i in range(1, len(lens)):
            if diff[i] > 0:
                t0, t1, d0, d1 = lens[i - 1], lens[i], diff[i - 1], diff[i]
                be = round(t0 + (t1 - t0) * (-d0) / (d1 - d0))
                break
    return {"tokens": table, "k8v8_vs_k16v8_break_even_tokens": be}


def _row(r):
    return {"us_per_step": r["ms_per_step"] * 1e3, "split_us": r["split_us"],
            "kv_gbs": r["kv_gbs"], "pct_roofline": r["pct_roofline"],
            "step_us_p10_p90": [r["step_us_stats"]["p10"], r["step_us_stats"]["p90"]],
            "validated": r["validation"]["validated"], "split_plan": r["split_plan"]}


def bench_gqa_sweep(steps, warmup, tokens=8192):
    """GQA group sweep: batch 16, 2 KV heads, head_dim 128, 8192 keys, query
    heads 2G for G = 1, 4, 8, 16; K8V8 and the BF16 control, HBM-cold."""
    from fp8_kv_cache_append_amd import synth

    res = {}
    for g in (1, 4, 8, 16):
        w = synth.Workload(f"decode_b16_hq{2 * g}_hkv2_d128_t{tokens}", 16, 2 * g, 2, 128,
                           np.full(16, tokens, np.int32), "outliers", seed=2)
        row = {}
        for mode in ("K8V8", "BF16"):
            r, _ = bench_decode(mode, w, steps, warmup, cold_copies(mode, w))
            row[mode] = _row(r)
        row["K8V8_speedup_vs_BF16"] = row["BF16"]["us_per_step"] / row["K8V8"]["us_per_step"]
        res[str(g)] = row
    return {"workload": f"decode_b16_hkv2_d128_t{tokens}, query heads 2G", "group": res}


def bench_batch_sweep(steps, warmup, tokens=2048):
    """Batch sweep of the 16q/2kv D128 shape at 2048 keys: batch 1, 4, 16,
    64; K8V8 and the BF16 control, HBM-cold."""
    from fp8_kv_cache_append_amd import synth

    res = {}
    for bsz in (1, 4, 16, 64):
        w = synth.Workload(f"decode_b{bsz}_hq16_hkv2_d128_t{tokens}", bsz, 16, 2, 128,
                           np.full(bsz, tokens, np.int32), "outliers", seed=2)
        row = {}
        for mode in ("K8V8", "BF16"):
            r, _ = bench_decode(mode, w, steps, warmup, cold_copies(mode, w))
            row[mode] = _row(r)
        row["K8V8_speedup_vs_BF16"] = row["BF16"]["us_per_step"] / row["K8V8"]["us_per_step"]
        res[str(bsz)] = row
    return {"workload": f"decode_hq16_hkv2_d128_t{tokens}", "batch": res}


def bench_small(steps, warmup):
    """Batch 1, 4 query / 1 KV head, head_dim 64, 128 keys, K8V8: 17 KB of
    cache per step, so even a rotation of 2048 copies (36 MB) stays in the
    Infinity Cache; the step is launch- and latency-bound."""
    from fp8_kv_cache_append_amd import synth

    w = synth.decode_b1_gqa4_d64()
    copies = cold_copies("K8V8", w)
    r, _ = bench_decode("K8V8", w, steps, warmup, copies)
    out = _row(r)
    out.update({"workload": w.name, "copies": copies,
                "cache_state": f"rotation of {copies} copies ({copies * r['kv_bytes'] / 1e6:.0f} MB)"
                               ", Infinity-Cache resident"})
    return out


def bench_read_floor(nbytes: int, copies: int = 64, replays: int = 10):
    """A plain streaming read of nbytes (the step's KV bytes) per launch, one
    buffer per launch of a 64-buffer rotation (HBM-cold like the headline),
    back to back in a HIP graph: what a single launch reading this many
    bytes reaches on this device (launch, ramp and drain included).  The
    fastest of a few grid sizes is the floor."""
    import ctypes
    import torch

    lib = ctypes.CDLL(os.path.join(ROOT, "tests", "hw", "libstream_read.so"))
    lib.stream_read_launch.restype = ctypes.c_int
    lib.stream_read_launch.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p,
                                       ctypes.c_int, ctypes.c_void_p]
    n = (int(nbytes) + 15) // 16 * 16
    bufs = [torch.empty(n, dtype=torch.uint8, device="cuda").fill_(i % 251)
            for i in range(copies)]
    sink = torch.empty(8192, dtype=torch.int32, device="cuda")
    res = {}
    for blocks in (1024, 2048, 4096, 8192):
        def launch(i, blocks=blocks):
            st = lib.stream_read_launch(bufs[i].data_ptr(), n, sink.data_ptr(), blocks,
                                        torch.cuda.current_stream().cuda_stream)
            assert st == 0, st
        launch(0)
        t = GraphTimer(torch, launch, copies)
        t.run(copies)
        res[str(blocks)] = pctl(t.samples(replays))["median"]
        del t
    best = min(res, key=res.get)
    us = res[best]
    del bufs
    return {"bytes_read": n, "us_per_launch": us, "read_gbs": n / (us * 1e-6) / 1e9,
            "pct_of_8tbs": 100.0 * n / (us * 1e-6) / 1e9 / HBM_PEAK_GBS,
            "work_groups": int(best), "us_by_work_groups": res}


def bench_block_scaled(steps, copies):
    """Block-scaled K (MXK8V8) against per-row K8V8 on the B16 T2048 shape,
    HBM-cold like the headline: fp8kv_decode (bf16 Q) and fp8kv_decode_q8
    (fp8 QK: per-row Q scale on K8V8, block-scaled QK on MXK8V8), two kernels
    each (split + merge; block-scaled K takes no fused append).  Errors are
    each output's relative L2 against the BF16 cache's, GPU against GPU."""
    import torch
    from fp8_kv_cache_append_amd import binding, synth
    from fp8_kv_cache_append_amd.binding import KVCache

    dev = "cuda"
    w = synth.decode_b16_gqa8_d128(2048)
    n = int(w.lens[0])
    bs, table, n_blocks = synth.block_layout(w)
    q_bits = synth.q_bf16_bits(w.seed, (w.batch, w.q_heads, w.head_dim))
    q = torch.from_numpy(q_bits.view(np.int16)).to(dev).view(torch.bfloat16)
    lens = torch.from_numpy(w.lens.astype(np.int32)).to(dev)
    ref_out = torch.empty((w.batch, w.q_heads, w.head_dim), device=dev)
    res = {}
    bases = {}
    for mode in ("BF16", "K8V8", "MXK8V8"):
        c = KVCache.allocate(mode, n_blocks, bs, w.kv_heads, w.head_dim, table, dev,
                             table_in_memory=False)   # contiguous
        for b in range(w.batch):
            k, v = synth.kv_sequence(w, b)
            binding.fp8kv_append(c, torch.from_numpy(k).to(dev), torch.from_numpy(v).to(dev),
                                 torch.full((n,), b, dtype=torch.int32, device=dev),
                                 torch.arange(n, dtype=torch.int32, device=dev))
        bases[mode] = c
    ws = torch.empty(binding.fp8kv_decode_workspace_bytes(bases["K8V8"], w.batch, w.group, n)
                     // 4 + 4, device=dev)
    binding.fp8kv_decode(bases["BF16"], q, w.group, lens, n, w.sm_scale, ref_out, ws)
    torch.cuda.synchronize()
    for mode in ("K8V8", "MXK8V8"):
        base = bases[mode]
        caches = [base] + [KVCache(mode, base.k.clone(), base.v.clone(),
                                   None if base.k_scale is None else base.k_scale.clone(),
                                   base.v_scale.clone(), base.block_table, None,
                                   None if base.k_exp is None else base.k_exp.clone(),
                                   False, base.layout)
                           for _ in range(copies - 1)]
        out = torch.empty_like(ref_out)
        for name, fn in (("bf16_q", binding.fp8kv_decode), ("fp8_qk", binding.fp8kv_decode_q8)):
            def step(i):
                fn(caches[i % copies], q, w.group, lens, n, w.sm_scale, out, ws)
            step(0)
            torch.cuda.synchronize()
            err = float(((out.double() - ref_out.double()).norm() / ref_out.double().norm()).item())
            valid = validate_decode(caches[0], q, out, w.lens, w.group, w.sm_scale,
                                    [(0, 0), (7, 1), (15, 0)], narrow=(name == "fp8_qk"))
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for i in range(copies):
                    step(i)
            g.replay()
            torch.cuda.synchronize()
            reps = max(1, math.ceil(steps / copies))
            t0 = torch.cuda.Event(enable_timing=True)
            t1 = torch.cuda.Event(enable_timing=True)
            t0.record()
            for _ in range(reps):
                g.replay()
            t1.record()
            torch.cuda.synchronize()
            res[f"{mode}_{name}"] = {"us_per_step": t0.elapsed_time(t1) * 1e3 / (reps * copies),
                                     "rel_l2_vs_bf16_cache": err,
                                     "validated": valid["validated"]}
        del caches
        torch.cuda.empty_cache()
    return {"workload": w.name + " (decode without append)", **res}


def bench_ragged(mode, replays=20, steps=8, pre_bias=False, w=None, layout="token"):
    """Batch 64, 32q/8kv, D128, lengths uniform in [1024, 32768], paged
    16-token blocks behind a shuffled table, biased keys (or workload w of
    that kind).  The cache (2.3 GB K8V8, 3.4 GB K16V8) is far larger than the
    Infinity Cache, so one copy is HBM-cold.  Filled from device-generated
    K/V of the same distributions.  pre_bias: the cache stores the keys'
    pre-bias residuals with the exact bias in the descriptor (decode adds
    q . b to the scores).  The step's output is checked on sampled pairs
    before timing."""
    import torch
    from fp8_kv_cache_append_amd import binding, synth
    from fp8_kv_cache_append_amd.binding import KVCache

    dev = "cuda"
    # the earlier legs' rotating copies go back to the device first, so the
    # 2-3 GB cache is allocated fresh rather than from fragmented cached blocks
    import gc
    gc.collect()
    torch.cuda.empty_cache()
    w = synth.decode_b64_gqa4_ragged_paged() if w is None else w
    bs, table, n_blocks = synth.block_layout(w)
    cache = KVCache.allocate(mode, n_blocks, bs, w.kv_heads, w.head_dim, table, dev,
                             layout=layout)
    if pre_bias:
        cache.k_bias = torch.from_numpy(synth.kv_sequence_prebias(w, 0)[2]).to(dev)
    k_last, v_last = [], []
    for b in range(w.batch):
        n = int(w.lens[b])
        k, v = synth.kv_sequence_device(w, b, dev, residual=pre_bias)
        seq = torch.full((n,), b, dtype=torch.int32, device=dev)
        pos = torch.arange(n, dtype=torch.int32, device=dev)
        binding.fp8kv_append(cache, k, v, seq, pos)
        k_last.append(k[-1].clone())
        v_last.append(v[-1].clone())
        torch.cuda.synchronize()
        del k, v, seq, pos
    k_new, v_new = torch.stack(k_last).contiguous(), torch.stack(v_last).contiguous()
    q_bits = synth.q_bf16_bits(w.seed, (w.batch, w.q_heads, w.head_dim))
    q = torch.from_numpy(q_bits.view(np.int16)).to(dev).view(torch.bfloat16)
    lens = torch.from_numpy(w.lens.astype(np.int32)).to(dev)
    max_len = int(w.lens.max())
    chunk, splits = binding.fp8kv_decode_plan(cache, w.batch, w.group, max_len)
    pacc = torch.empty((w.batch, w.kv_heads, splits, w.group, w.head_dim), device=dev)
    pml = torch.empty((w.batch, w.kv_heads, splits, w.group, 2), device=dev)
    out = torch.empty((w.batch, w.q_heads, w.head_dim), device=dev)

    def split(i=0):
        binding.fp8kv_decode_append_partial(cache, k_new, v_new, q, w.group, lens, max_len,
                                            w.sm_scale, chunk, splits, pacc, pml)

    def step(i=0):
        split()
        binding.fp8kv_decode_merge(w.batch, w.kv_heads, w.group, w.head_dim, splits, pacc,
                                   pml, out)

    step()
    torch.cuda.synchronize()
    order = np.argsort(w.lens)
    pairs = [(int(order[0]), 0), (int(order[-1]), w.kv_heads - 1),
             (int(order[len(order) // 2]), w.kv_heads // 2)]
    valid = validate_decode(cache, q, out, w.lens, w.group, w.sm_scale, pairs)
    t_step, t_split = GraphTimer(torch, step, steps), GraphTimer(torch, split, steps)
    t_step.run(steps)
    step_st, split_st = pctl(t_step.samples(replays)), pctl(t_split.samples(replays))
    step_us, split_us = step_st["median"], split_st["median"]
    kv_bytes = int(w.lens.sum()) * w.kv_heads * ROW_BYTES[mode](w.head_dim)
    return {"workload": w.name, "mode": mode + ("_pre_bias" if pre_bias else ""),
            "layout": layout, "us_per_step": step_us, "split_us": split_us,
            "step_us_stats": step_st, "split_us_stats": split_st,
            "kv_bytes": kv_bytes, "kv_gbs": kv_bytes / (step_us * 1e-6) / 1e9,
            "split_kv_gbs": kv_bytes / (split_us * 1e-6) / 1e9,
            "pct_roofline": 100.0 * kv_bytes / (step_us * 1e-6) / 1e9 / HBM_PEAK_GBS,
            "split_pct_roofline": 100.0 * kv_bytes / (split_us * 1e-6) / 1e9 / HBM_PEAK_GBS,
            "validation": valid,
            "split_plan": {"chunk_tokens": chunk, "n_splits": splits}}


def bench_page_sizes(replays=10, steps=8):
    """Page-size sweep on a subset of the ragged workload: its first 16
    sequences (same lengths, distributions and heads), K8V8, head-major
    blocks of 16, 32, 64 and 256 tokens behind a shuffled table."""
    from fp8_kv_cache_append_amd import synth

    base = synth.decode_b64_gqa4_ragged_paged()
    res = {}
    for bs in (16, 32, 64, 256):
        w = synth.Workload(f"decode_b16_hq32_hkv8_d128_ragged_paged{bs}", 16, 32, 8, 128,
                           base.lens[:16].copy(), "bias", block_size=bs, shuffle_blocks=True,
                           seed=base.seed)
        r = bench_ragged("K8V8", replays, steps, w=w, layout="head")
        res[str(bs)] = {k: r[k] for k in ("us_per_step", "split_us", "kv_gbs", "pct_roofline",
                                           "split_pct_roofline", "split_plan")}
        res[str(bs)]["validated"] = r["validation"]["validated"]
    return {"workload": "first 16 sequences of the ragged batch, K8V8", "block_size": res}


def bench_warm(mode, w, steps, copies):
    """The same graph of steps on one copy of the cache: L2/MALL-warm,
    labelled as such (it can exceed the HBM rate)."""
    bench = DecodeBench(mode, w, copies, warm=True)
    bench.capture()
    bench.t_step.run(2 * copies)
    step_ms = bench.t_step.time(steps)
    return {"ms_per_step": step_ms, "steps": int(steps),
            "kv_gbs": bench.kv_bytes / (step_ms * 1e-3) / 1e9,
            "split_us": pctl(bench.t_split.samples(4))["median"]}


def bench_copy_floor(nbytes: int, copies: int = 64, replays: int = 20):
    """Context for the roofline at this size: a device-to-device copy of
    nbytes (the step's KV bytes), one per buffer pair of a 64-pair rotation
    (HBM-cold like the headline), back to back in a HIP graph.  It reads and
    writes nbytes each, so it bounds from below what one launch moving this
    many bytes costs on this stack (launch, ramp and drain included)."""
    import torch

    n = int(nbytes)
    src = [torch.empty(n, dtype=torch.uint8, device="cuda").fill_(i % 251) for i in range(copies)]
    dst = [torch.empty(n, dtype=torch.uint8, device="cuda") for _ in range(copies)]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(copies):
            dst[i].copy_(src[i])
    g.replay()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(replays):
        g.replay()
    t1.record()
    torch.cuda.synchronize()
    us = t0.elapsed_time(t1) * 1e3 / (replays * copies)
    ok = all(torch.equal(dst[i][:4096], src[i][:4096]) for i in (0, copies - 1))
    del src, dst, g
    return {"bytes_read": n, "bytes_written": n, "us_per_copy": us,
            "read_plus_write_gbs": 2 * n / (us * 1e-6) / 1e9, "checked": ok}


def bench_append_bulk(n_tok: int = 131072, replays: int = 10):
    """Bulk append (fp8kv_append) of n_tok new tokens x 8 KV heads x head_dim
    128 into a paged K8V8 cache with 16-token blocks behind a shuffled table
    (the ragged batch's cache format): per (token, KV head) row the kernel
    reads 8 * 128 B of fp32 K and V and writes 264 B of codes and scales.
    Eight calls on rotating inputs and caches, back to back in a graph."""
    import torch
    from fp8_kv_cache_append_amd import binding
    from fp8_kv_cache_append_amd.binding import KVCache

    hkv, d, bs, copies = 8, 128, 16, 8
    n_blocks = n_tok // bs
    table = np.random.default_rng(4).permutation(n_blocks).astype(np.int32).reshape(1, -1)
    caches = [KVCache.allocate("K8V8", n_blocks, bs, hkv, d, table, "cuda") for _ in range(copies)]
    gen = torch.Generator(device="cuda").manual_seed(4)
    ks = [torch.randn((n_tok, hkv, d), device="cuda", generator=gen) for _ in range(copies)]
    vs = [torch.randn((n_tok, hkv, d), device="cuda", generator=gen) for _ in range(copies)]
    seq = torch.zeros(n_tok, dtype=torch.int32, device="cuda")
    pos = torch.arange(n_tok, dtype=torch.int32, device="cuda")

    def call(i):
        binding.fp8kv_append(caches[i], ks[i], vs[i], seq, pos)

    for i in range(copies):
        call(i)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(copies):
            call(i)
    g.replay()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(replays):
        g.replay()
    t1.record()
    torch.cuda.synchronize()
    us = t0.elapsed_time(t1) * 1e3 / (replays * copies)
    rows = n_tok * hkv
    alg = rows * (8 * d + ROW_BYTES["K8V8"](d))
    res = {"workload": f"append_k8v8_{n_tok}tok_hkv{hkv}_d{d}_paged{bs}", "rows": rows,
           "us": us, "algorithmic_bytes": alg, "gbs": alg / (us * 1e-6) / 1e9,
           "pct_roofline": 100.0 * alg / (us * 1e-6) / 1e9 / HBM_PEAK_GBS}
    del caches, ks, vs, g
    return res


def bench_prefill(reps=200, mode="K8V8", layout="token"):
    import torch
    from fp8_kv_cache_append_amd import binding, synth
    from fp8_kv_cache_append_amd.binding import KVCache

    w = synth.prefill_gqa7_d128()
    n = int(w.lens[0])
    bs, table, n_blocks = synth.block_layout(w)
    cache = KVCache.allocate(mode, n_blocks, bs, w.kv_heads, w.head_dim, table, "cuda",
                             table_in_memory=False, layout=layout)   # contiguous
    k, v = synth.kv_sequence(w, 0)
    binding.fp8kv_append(cache, torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda(),
                         torch.zeros(n, dtype=torch.int32, device="cuda"),
                         torch.arange(n, dtype=torch.int32, device="cuda"))
    q_bits = synth.q_bf16_bits(w.seed, (n, w.q_heads, w.head_dim))
    q = torch.from_numpy(q_bits.view(np.int16)).cuda().view(torch.bfloat16)
    cu = torch.tensor([0, n], dtype=torch.int32, device="cuda")
    pos0 = torch.zeros(1, dtype=torch.int32, device="cuda")
    lens = torch.tensor([n], dtype=torch.int32, device="cuda")
    out = torch.empty((n, w.q_heads, w.head_dim), device="cuda")

    def call():
        binding.fp8kv_prefill(cache, q, w.group, cu, pos0, lens, n, w.sm_scale, out)

    for _ in range(5):
        call()
    # launches back to back in one graph, timed between two events around
    # its replays: no host launch cost inside the timed region
    per_graph = 10
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(per_graph):
            call()
    g.replay()
    torch.cuda.synchronize()
    samples = []
    for _ in range(max(1, reps // per_graph)):
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record()
        g.replay()
        t1.record()
        torch.cuda.synchronize()
        samples.append(t0.elapsed_time(t1) / per_graph)
    us = float(np.median(samples)) * 1e3
    flops = 4.0 * w.q_heads * w.head_dim * (n * (n + 1) / 2)
    # sanity check of the timed output on sampled query rows, every head
    call()
    torch.cuda.synchronize()
    rows = [0, 63, 64, 1000, 2047]
    g = w.group
    items = [(0, hk, np.full(g, i + 1), i) for i in rows for hk in range(w.kv_heads)]
    ref = reference_rows(cache, q_bits, g, w.sm_scale, items)
    o = out.cpu().numpy()
    got = np.stack([o[i, hk * g:(hk + 1) * g] for i in rows for hk in range(w.kv_heads)])
    valid = check_rows(got, ref)
    valid["sample"] = f"query rows {rows}, all heads"
    return {"workload": w.name, "mode": mode, "us": us, "tflops": flops / (us * 1e-6) / 1e12,
            "pct_mfma_peak": 100.0 * flops / (us * 1e-6) / 1e12 / BF16_MFMA_PEAK_TFLOPS,
            "us_stats": {"median": us, "p10": float(np.percentile(samples, 10)) * 1e3,
                         "p90": float(np.percentile(samples, 90)) * 1e3,
                         "replays": len(samples), "launches_per_replay": per_graph},
            "validation": valid, "algorithmic_gflop": flops / 1e9}


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def cpu_baseline(w, min_seconds=8.0):
    """The oracle as it stands on whole decode steps of the same workload:
    quantise the new tokens, then attend every (sequence, KV head).  The
    cache is quantised once beforehand (not timed).  Timed twice: on one
    thread, and with the (sequence, KV head) units spread over the host's
    cores (up to 16, the box's share) by a thread pool -- the oracle's C
    calls release the interpreter lock, and the units share nothing.
    Returns the record and the oracle's output of the step (fp64 [B, Hq,
    D]), which the caller compares with the GPU step's."""
    import os
    from concurrent.futures import ThreadPoolExecutor

    import oracle
    from fp8_kv_cache_append_amd import synth

    g, n = w.group, int(w.lens[0])
    q_bits = synth.q_bf16_bits(w.seed, (w.batch, w.q_heads, w.head_dim))
    stores, news = [], []
    for b in range(w.batch):
        k, v = synth.kv_sequence(w, b)
        stores.append(oracle.store_rows("K8V8", k, v))
        news.append((k[-1:], v[-1:]))
    units = [(b, h) for b in range(w.batch) for h in range(w.kv_heads)]
    result = np.full((w.batch, w.q_heads, w.head_dim), np.nan)

    def unit(bh):
        b, h = bh
        view = {key: np.ascontiguousarray(a[:, h]) for key, a in stores[b].items()}
        result[b, h * g:(h + 1) * g] = oracle.attend_rows(
            "K8V8", q_bits[b, h * g:(h + 1) * g], view, n, w.sm_scale)

    def run(workers):
        steps, t0 = 0, time.perf_counter()
        with ThreadPoolExecutor(max_workers=workers) as pool:
            while True:
                for b in range(w.batch):
                    oracle.store_rows("K8V8", *news[b])
                if workers == 1:
                    for u in units:
                        unit(u)
                else:
                    list(pool.map(unit, units))
                steps += 1
                el = time.perf_counter() - t0
                if el >= min_seconds:
                    return steps, el

    kv_bytes = int(w.lens.sum()) * w.kv_heads * ROW_BYTES["K8V8"](w.head_dim)
    workers = max(1, min(16, os.cpu_count() or 1))
    res = {}
    for nw in sorted({1, workers}):
        steps, el = run(nw)
        res[nw] = {"value": kv_bytes * steps / el / 1e9, "unit": "GB/s", "cores": nw,
                   "kind": "oracle", "ms_per_step": el / steps * 1e3,
                   "sample": f"{steps} full decode steps of the benchmark workload "
                             f"(16 seqs x 2 KV heads x {n} keys, K8V8), {el:.1f} s on "
                             f"{nw} thread{'s' if nw > 1 else ''}"}
    out = dict(res[workers])
    out["cpu_model"] = cpu_model()
    out["host_cpus"] = os.cpu_count()
    if workers > 1:
        out["single_thread"] = res[1]
    return out, result


def traffic_for(kernel_hash: str, split_launches_bytes_hint=None):
    """HBM bytes per split-kernel launch from the committed counter summary,
    or None when it is missing or was taken on different kernel source."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_hash") != kernel_hash:
        return None
    return rec.get("bytes_per_launch")


def _validated_flags(x):
    """Every "validated" flag anywhere in the record."""
    if isinstance(x, dict):
        for k, v in x.items():
            if k == "validated" and isinstance(v, bool):
                yield v
            else:
                yield from _validated_flags(v)
    elif isinstance(x, list):
        for v in x:
            yield from _validated_flags(v)


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=6400,
                    help="decode steps timed for the headline (exactly this many)")
    ap.add_argument("--warmup", type=int, default=640,
                    help="untimed decode steps before them (exactly this many)")
    ap.add_argument("--copies", type=int, default=64,
                    help="cache copies in the headline's rotation (64: 1.1 GB, HBM-cold)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="K8V8 decode only (for profiling runs)")
    ap.add_argument("--prefill-only", action="store_true",
                    help="only the causal prefill of 2048 tokens (for profiling runs)")
    ap.add_argument("--ragged-only", action="store_true",
                    help="only the ragged batch-64 paged K8V8 decode (for profiling runs)")
    ap.add_argument("--append-only", action="store_true",
                    help="only the bulk append of 1 M rows (for profiling runs)")
    ap.add_argument("--tokens", type=int, default=2048,
                    help="cached tokens of the headline shape (2048; other lengths only "
                         "for profiling runs with --no-extras)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: every box here has one, and the decode path "
              "has no cross-GPU step.", file=sys.stderr)
        sys.exit(2)
    if args.steps < 1 or args.warmup < 0 or args.copies < 1:
        print("--steps >= 1, --warmup >= 0, --copies >= 1", file=sys.stderr)
        sys.exit(2)
    if args.tokens != 2048 and not args.no_extras:
        print("--tokens other than 2048 needs --no-extras", file=sys.stderr)
        sys.exit(2)

    import torch
    from fp8_kv_cache_append_amd import binding, synth

    binding.lib()
    torch.cuda.set_device(0)
    t_start = time.perf_counter()

    def leg(name, fn, *a, **k):
        t0 = time.perf_counter()
        r = fn(*a, **k)
        print(f"[bench] {name}: {time.perf_counter() - t0:.1f} s", file=sys.stderr, flush=True)
        return r

    if args.ragged_only:
        print(json.dumps({"ragged_b64_paged": bench_ragged("K8V8", replays=4, steps=4,
                                                           layout="head")}), flush=True)
        return
    if args.prefill_only:
        print(json.dumps({"prefill": bench_prefill()}), flush=True)
        return
    if args.append_only:
        print(json.dumps({"append_bulk": bench_append_bulk()}), flush=True)
        return

    w = synth.decode_b16_gqa8_d128(args.tokens)
    head, hb = leg("headline K8V8", bench_decode, "K8V8", w, args.steps, args.warmup,
                   args.copies, replays=16)
    split_us = head["split_us"]
    achieved = head["kv_bytes"] / (split_us * 1e-6) / 1e9
    khash = kernel_source_hash()
    traffic = traffic_for(khash)
    gpu_out = step_output(hb)
    extras = {}
    if not args.no_extras:
        sw, ww = max(640, args.steps // 4), max(64, args.warmup // 4)
        outs = {"K8V8": gpu_out}
        for mode in ("K16V8", "BF16"):
            r, bb = leg(f"headline {mode}", bench_decode, mode, w, args.steps, args.warmup,
                        args.copies)
            extras[mode] = r
            outs[mode] = step_output(bb)
            del bb
        ref = outs["BF16"]
        extras["fp8_vs_bf16"] = {
            m: float(((outs[m] - ref).norm() / ref.norm()).item()) for m in ("K8V8", "K16V8")}
        del hb
        extras["K8V8_warm"] = leg("warm", bench_warm, "K8V8", w, args.steps, args.copies)
        extras["copy_floor"] = leg("copy floor", bench_copy_floor, head["kv_bytes"])
        extras["read_floor"] = leg("read floor", bench_read_floor, head["kv_bytes"])
        extras["append_bulk"] = leg("append bulk", bench_append_bulk)
        extras["prefill"] = leg("prefill K8V8", bench_prefill)
        extras["prefill_bf16"] = leg("prefill BF16", bench_prefill, mode="BF16")
        extras["small"] = leg("config 1", bench_small, sw, ww)
        extras["sweep"] = leg("context sweep", bench_sweep, sw, ww, args.copies, head)
        extras["gqa"] = leg("GQA sweep", bench_gqa_sweep, sw, ww)
        extras["batch"] = leg("batch sweep", bench_batch_sweep, sw, ww)
        # the paged batch's page-internal order is free: head-major, the order
        # the split kernel reads; token-major reported beside it
        extras["ragged"] = {m: leg(f"ragged {m}", bench_ragged, m, layout="head")
                            for m in ("K8V8", "K16V8")}
        extras["ragged"]["K8V8_pre_bias"] = leg("ragged pre-bias", bench_ragged, "K8V8",
                                                pre_bias=True, layout="head")
        extras["ragged"]["K8V8_token_major"] = leg("ragged token-major", bench_ragged, "K8V8",
                                                   layout="token")
        extras["page_sizes"] = leg("page sizes", bench_page_sizes)
        extras["block_scaled"] = leg("block-scaled K", bench_block_scaled, sw, args.copies)
    cpu = None
    if not args.no_cpu_baseline:
        cpu, orc = leg("cpu baseline", cpu_baseline, w)
        # the oracle's own output of the step (this leg) against the GPU's
        got = gpu_out.cpu().numpy()
        cpu["oracle_vs_gpu_step"] = {
            "rel_l2": float(np.linalg.norm(got - orc) / np.linalg.norm(orc)),
            "max_abs": float(np.max(np.abs(got - orc)))}

    rec = {
        "metric": "KV-cache GB/s (% of 8 TB/s) and us/decode step, K8/V8 vs K16/V8 vs BF16",
        "value": head["kv_gbs"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": head["steps"],
        "warmup": head["warmup"],
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"decode_b16_hq16_hkv2_d128_t{args.tokens}_k8v8_hbm_cold",
                   "batch": w.batch, "q_heads": w.q_heads, "kv_heads": w.kv_heads,
                   "head_dim": w.head_dim, "cached_tokens": int(w.lens[0]),
                   "kv_format": "e4m3 + fp32 scale per (token, KV head)",
                   "cache_state": f"HBM-cold, rotating {args.copies} copies",
                   "step": "split kernel with the append of 1 token/seq fused in + "
                           "merge kernel",
                   "split_plan": head["split_plan"]},
        "us_per_step": head["ms_per_step"] * 1e3,
        "pct_roofline": head["pct_roofline"],
        "step_us_stats": head["step_us_stats"],
        "split_us": head["split_us"],
        "split_us_stats": head["split_us_stats"],
        "kernel_us_event_pairs": head["kernel_us_event_pairs"],
        "unfused_step_us": head["unfused_step_us"],
        "dequant_then_bf16_step_us": head["dequant_then_bf16_step_us"],
        "narrow_qk_step_us": head["narrow_qk_step_us"],
        "narrow_qk_vs_bf16q_rel_l2": head["narrow_qk_vs_bf16q_rel_l2"],
        "validation": head["validation"],
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "kernel": "decode_partial_kernel<K8V8,128,append,one tile per wave>",
                     "bytes_per_launch": head["kv_bytes"],
                     "duration_us": "median of per-replay means (split_us_stats)",
                     "kernel_source_hash": khash},
        "cpu_baseline": cpu,
    }
    if extras:
        keys = ("ms_per_step", "kv_gbs", "pct_roofline", "split_us", "kernel_us_event_pairs",
                "unfused_step_us", "step_us_stats")
        rec["modes"] = {"K8V8": {k: head[k] for k in keys}}
        for mode in ("K16V8", "BF16"):
            rec["modes"][mode] = {k: extras[mode][k] for k in keys}
            rec["modes"][mode]["validated"] = extras[mode]["validation"]["validated"]
        rec["speedup_vs_bf16"] = extras["BF16"]["ms_per_step"] / head["ms_per_step"]
        rec["speedup_vs_k16v8"] = extras["K16V8"]["ms_per_step"] / head["ms_per_step"]
        # op-level error of the quantised caches: the GPU step's output
        # against the BF16-cache step's on the same inputs (relative L2)
        rec["fp8_vs_bf16_rel_l2"] = extras["fp8_vs_bf16"]
        rec["warm_l2_mall"] = extras["K8V8_warm"]
        rec["copy_floor_same_bytes"] = extras["copy_floor"]
        rec["read_floor_same_bytes"] = extras["read_floor"]
        rec["append_bulk"] = extras["append_bulk"]
        rec["prefill"] = extras["prefill"]
        rec["prefill_bf16_control"] = extras["prefill_bf16"]
        rec["decode_b1_hq4_hkv1_d64_t128"] = extras["small"]
        rec["context_sweep"] = extras["sweep"]
        rec["gqa_sweep"] = extras["gqa"]
        rec["batch_sweep"] = extras["batch"]
        rec["ragged_b64_paged"] = extras["ragged"]
        rec["page_size_sweep"] = extras["page_sizes"]
        rec["block_scaled_k"] = extras["block_scaled"]
        rec["all_timed_outputs_validated"] = bool(all(_validated_flags(rec)))
    rec["bench_wall_s"] = time.perf_counter() - t_start
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
