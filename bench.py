"""Benchmark: KV-cache GB/s (% of 8 TB/s) and us per decode step, K8V8 vs
K16V8 vs BF16, on one MI355X.

Step: one decode step of batch 16, 16 query / 2 KV heads (GQA 8), head_dim
128, 2048 keys per sequence (e4m3 K/V, N(0,1) with 2 % x10 outliers):
  fp8kv_decode_append_partial: the split kernel, which also quantises and
    stores each sequence's new token (position 2047) and attends it;
  fp8kv_decode_merge: the merge kernel.
The same step as three kernels (fp8kv_append, fp8kv_decode_partial,
fp8kv_decode_merge) is timed too and reported as unfused_step_us, and the
unfused control -- append, the whole cache dequantised to bf16 in HBM
(fp8kv_dequantize), BF16 split + merge on the copy -- as
dequant_then_bf16_step_us.
The headline value is K8V8 KV bytes per step / time per step, HBM-cold: the
step rotates over 64 copies of the cache (> 1 GB, larger than the 256 MB
Infinity Cache), so no copy is cache-resident when it is read.  All steps of
one rotation are captured in a HIP graph (no host launch cost inside the
timed region).  Per-kernel durations come from HIP event pairs around each
kernel of one more rotation, launched on the same stream right behind the
timed replays (see DecodeBench.run).

Narrow QK (fp8kv_decode_append_q8: Q quantised to e4m3 in the split kernel,
fp8 QK) is timed on the same rotation for the e4m3-K modes
(narrow_qk_step_us), with its output's relative L2 against the bf16-Q step
(narrow_qk_vs_bf16q_rel_l2: the Q rounding's cost).

Extra fields: the K16V8 and BF16 controls (same protocol), a device copy of
the step's KV bytes under the same protocol (copy_floor_same_bytes: what one
launch moving this many bytes costs here), the bulk append kernel's rate
(append_bulk: 1M rows into a paged K8V8 cache), the op-level error
of each quantised cache (fp8_vs_bf16_rel_l2: the step's output against the
BF16-cache step's on the same inputs), the L2/MALL-warm
rate (one copy, labelled), the causal prefill of 2048 tokens (28/4 heads;
K8V8 and the BF16 cache as its matrix-core control),
the context sweep of the same shape at 77/512/2048/8192 keys in all four
modes (K8V16 isolates the K side) with the K8V8-vs-K16V8 break-even and the
per-side savings against BF16, the ragged batch-64 paged workload
(32q/8kv, lengths 1024..32768, K8V8, K16V8 and K8V8 as a pre-bias residual
cache with the exact key bias), block-scaled K (MXK8V8) against per-row
K8V8 with bf16 Q and with fp8 QK (block_scaled_k), the roofline of the split
kernel and the CPU oracle as a baseline.
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
                  "fp8_kv_cache_append_amd/csrc/device.h"]


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


class DecodeBench:
    """Rotating copies of one decode workload plus the graph of one rotation."""

    def __init__(self, mode: str, w, copies: int, warm: bool = False):
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
                                table_in_memory=mem_table)
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
                                        base.block_table, table_in_memory=mem_table)
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
        if self.narrow:
            ws_bytes = binding.fp8kv_decode_workspace_bytes(base, w.batch, g, n)
            self.ws = torch.empty(ws_bytes // 4 + 4, device=dev)
            self.out_q8 = torch.empty_like(self.out)
        self.graph = None
        self.dq = None
        if mode == "K8V8":
            # the unfused control: the cache dequantised to bf16 in HBM, then
            # the BF16 kernels on the copy
            self.dq = KVCache.allocate("BF16", n_blocks, bs, w.kv_heads, d, table, dev,
                                       table_in_memory=mem_table)
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
        """One decode step: append each sequence's new token (fused into the
        split kernel), split partials, merge."""
        b, w = self.binding, self.w
        if ev: ev[0].record()
        self.split(i)
        if ev: ev[1].record()
        b.fp8kv_decode_merge(w.batch, w.kv_heads, w.group, w.head_dim, self.splits,
                             self.pacc, self.pml, self.out)
        if ev: ev[2].record()

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

    def _graph(self, fn):
        torch = self.torch
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(self.copies):
                fn(i)
        torch.cuda.synchronize()
        return g

    def capture(self):
        torch = self.torch
        self.step(0)  # eager calls first: the library's one-time device check
        self.step_unfused(0)
        torch.cuda.synchronize()
        self.graph = self._graph(self.step)
        self.split_graph = self._graph(self.split)
        self.unfused_graph = self._graph(self.step_unfused)
        self.q8_graph = None
        if self.narrow:
            self.step_q8(0)
            torch.cuda.synchronize()
            self.q8_graph = self._graph(self.step_q8)
        self.dq_graph = None
        if self.dq is not None:
            self.step_unfused_dequant(0)
            torch.cuda.synchronize()
            self.dq_graph = self._graph(self.step_unfused_dequant)

    def graph_avg_ms(self, graph, replays: int) -> float:
        """Average time of one rotation entry of `graph` (ms), back to back."""
        torch = self.torch
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        graph.replay()
        torch.cuda.synchronize()
        t0.record()
        for _ in range(replays):
            graph.replay()
        t1.record()
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) / (replays * self.copies)

    def split_avg_ms(self, replays: int) -> float:
        """Average duration of one split-kernel launch: the split kernel alone
        over the rotation, back to back in a graph, between two events."""
        return self.graph_avg_ms(self.split_graph, replays)

    def run(self, replays: int, kernel_events: bool = False):
        """Replay the rotation `replays` times between two events (ms).

        With kernel_events, one more rotation is then launched eagerly with an
        event pair around every kernel on the launch stream.  It is enqueued
        while the GPU is still busy with the replays, so no host launch gap
        falls inside a pair: each pair brackets exactly one kernel."""
        torch = self.torch
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0.record()
        for _ in range(replays):
            self.graph.replay()
        t1.record()
        ev = None
        if kernel_events:
            ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)]
                  for _ in range(self.copies)]
            for i in range(self.copies):
                self.step(i, ev[i])
        torch.cuda.synchronize()
        self.events = ev
        return t0.elapsed_time(t1)  # ms

    def kernel_ms(self):
        """Mean per-launch durations (ms) of the split kernel (with the fused
        append) and the merge kernel."""
        ev = self.events
        spl = [ev[i][0].elapsed_time(ev[i][1]) for i in range(self.copies)]
        mrg = [ev[i][1].elapsed_time(ev[i][2]) for i in range(self.copies)]
        return float(np.mean(spl)), float(np.mean(mrg))


def step_output(bench):
    """The output of one decode step on the bench's first cache copy (fp64,
    on the device): every mode's bench holds the same seeded inputs."""
    bench.step(0)
    bench.torch.cuda.synchronize()
    return bench.out.double().clone()


def bench_decode(mode, w, steps, warmup, copies):
    bench = DecodeBench(mode, w, copies)
    bench.capture()
    reps = max(1, math.ceil(steps / copies))
    bench.run(max(1, math.ceil(warmup / copies)))
    ms = bench.run(reps, kernel_events=True)
    n_steps = reps * copies
    spl, mrg = bench.kernel_ms()
    split_avg = bench.split_avg_ms(reps)
    unfused = bench.graph_avg_ms(bench.unfused_graph, reps)
    dq = bench.graph_avg_ms(bench.dq_graph, reps) if bench.dq_graph is not None else None
    q8 = bench.graph_avg_ms(bench.q8_graph, reps) if bench.q8_graph is not None else None
    q8_err = None
    if q8 is not None:
        # narrow against bf16-Q outputs of the same step on the same cache
        bench.step(0)
        bench.step_q8(0)
        bench.torch.cuda.synchronize()
        a = bench.out_q8.double()
        r = bench.out.double()
        q8_err = float(((a - r).norm() / r.norm()).item())
    step_ms = ms / n_steps
    res = {"ms_per_step": step_ms, "steps": n_steps, "kv_bytes": bench.kv_bytes,
           "kv_gbs": bench.kv_bytes / (step_ms * 1e-3) / 1e9,
           "kernel_us_event_pairs": {"split_with_append": spl * 1e3, "merge": mrg * 1e3},
           "split_us": split_avg * 1e3,
           "unfused_step_us": unfused * 1e3,
           "dequant_then_bf16_step_us": None if dq is None else dq * 1e3,
           "narrow_qk_step_us": None if q8 is None else q8 * 1e3,
           "narrow_qk_vs_bf16q_rel_l2": q8_err,
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
                r, _ = bench_decode(mode, w, steps, warmup, copies)
            row[mode] = {"us_per_step": r["ms_per_step"] * 1e3, "split_us": r["split_us"],
                         "kv_gbs": r["kv_gbs"], "pct_roofline": r["pct_roofline"],
                         "unfused_step_us": r["unfused_step_us"],
                         "narrow_qk_step_us": r["narrow_qk_step_us"]}
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
                                   False)
                           for _ in range(copies - 1)]
        out = torch.empty_like(ref_out)
        for name, fn in (("bf16_q", binding.fp8kv_decode), ("fp8_qk", binding.fp8kv_decode_q8)):
            def step(i):
                fn(caches[i % copies], q, w.group, lens, n, w.sm_scale, out, ws)
            step(0)
            torch.cuda.synchronize()
            err = float(((out.double() - ref_out.double()).norm() / ref_out.double().norm()).item())
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
                                     "rel_l2_vs_bf16_cache": err}
        del caches
        torch.cuda.empty_cache()
    return {"workload": w.name + " (decode without append)", **res}


def bench_ragged(mode, replays=20, steps=8, pre_bias=False):
    """Batch 64, 32q/8kv, D128, lengths uniform in [1024, 32768], paged
    16-token blocks behind a shuffled table, biased keys.  The cache (2.3 GB
    K8V8, 3.4 GB K16V8) is far larger than the Infinity Cache, so one copy is
    HBM-cold.  Filled from device-generated K/V of the same distributions.
    pre_bias: the cache stores the keys' pre-bias residuals with the exact
    bias in the descriptor (decode adds q . b to the scores)."""
    import torch
    from fp8_kv_cache_append_amd import binding, synth
    from fp8_kv_cache_append_amd.binding import KVCache

    dev = "cuda"
    # the earlier legs' rotating copies go back to the device first, so the
    # 2-3 GB cache is allocated fresh rather than from fragmented cached blocks
    import gc
    gc.collect()
    torch.cuda.empty_cache()
    w = synth.decode_b64_gqa4_ragged_paged()
    bs, table, n_blocks = synth.block_layout(w)
    cache = KVCache.allocate(mode, n_blocks, bs, w.kv_heads, w.head_dim, table, dev)
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

    def split():
        binding.fp8kv_decode_append_partial(cache, k_new, v_new, q, w.group, lens, max_len,
                                            w.sm_scale, chunk, splits, pacc, pml)

    def step():
        split()
        binding.fp8kv_decode_merge(w.batch, w.kv_heads, w.group, w.head_dim, splits, pacc,
                                   pml, out)

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(steps):
                fn()
        g.replay()
        torch.cuda.synchronize()
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record()
        for _ in range(replays):
            g.replay()
        t1.record()
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) * 1e3 / (replays * steps)

    step_us, split_us = timed(step), timed(split)
    kv_bytes = int(w.lens.sum()) * w.kv_heads * ROW_BYTES[mode](w.head_dim)
    return {"workload": w.name, "mode": mode + ("_pre_bias" if pre_bias else ""),
            "us_per_step": step_us, "split_us": split_us,
            "kv_bytes": kv_bytes, "kv_gbs": kv_bytes / (step_us * 1e-6) / 1e9,
            "split_kv_gbs": kv_bytes / (split_us * 1e-6) / 1e9,
            "pct_roofline": 100.0 * kv_bytes / (step_us * 1e-6) / 1e9 / HBM_PEAK_GBS,
            "split_plan": {"chunk_tokens": chunk, "n_splits": splits}}


def bench_warm(mode, w, steps, copies):
    """The same graph of steps on one copy of the cache: L2/MALL-warm,
    labelled as such (it can exceed the HBM rate)."""
    bench = DecodeBench(mode, w, copies, warm=True)
    bench.capture()
    bench.run(2)
    reps = max(1, math.ceil(steps / copies))
    ms = bench.run(reps)
    step_ms = ms / (reps * copies)
    return {"ms_per_step": step_ms, "kv_gbs": bench.kv_bytes / (step_ms * 1e-3) / 1e9,
            "split_us": bench.split_avg_ms(reps) * 1e3}


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


def bench_prefill(reps=200, mode="K8V8"):
    import torch
    from fp8_kv_cache_append_amd import binding, synth
    from fp8_kv_cache_append_amd.binding import KVCache

    w = synth.prefill_gqa7_d128()
    n = int(w.lens[0])
    bs, table, n_blocks = synth.block_layout(w)
    cache = KVCache.allocate(mode, n_blocks, bs, w.kv_heads, w.head_dim, table, "cuda",
                             table_in_memory=False)   # contiguous
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
    return {"workload": w.name, "mode": mode, "us": us, "tflops": flops / (us * 1e-6) / 1e12,
            "pct_mfma_peak": 100.0 * flops / (us * 1e-6) / 1e12 / BF16_MFMA_PEAK_TFLOPS,
            "algorithmic_gflop": flops / 1e9}


def cpu_baseline(w, min_seconds=8.0):
    """The oracle as it stands on whole decode steps of the same workload:
    quantise the new tokens, then attend every (sequence, KV head).  The
    cache is quantised once beforehand (not timed).  Timed twice: on one
    thread, and with the (sequence, KV head) units spread over the host's
    cores (up to 16, the box's share) by a thread pool -- the oracle's C
    calls release the interpreter lock, and the units share nothing."""
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

    def unit(bh):
        b, h = bh
        view = {key: np.ascontiguousarray(a[:, h]) for key, a in stores[b].items()}
        oracle.attend_rows("K8V8", q_bits[b, h * g:(h + 1) * g], view, n, w.sm_scale)

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
    if workers > 1:
        out["single_thread"] = res[1]
    return out


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


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=6400)
    ap.add_argument("--warmup", type=int, default=640)
    ap.add_argument("--copies", type=int, default=64)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="K8V8 decode only (for profiling runs)")
    ap.add_argument("--prefill-only", action="store_true",
                    help="only the causal prefill of 2048 tokens (for profiling runs)")
    ap.add_argument("--ragged-only", action="store_true",
                    help="only the ragged batch-64 paged K8V8 decode (for profiling runs)")
    args = ap.parse_args()
    if args.ragged_only:
        import torch
        from fp8_kv_cache_append_amd import binding

        binding.lib()
        torch.cuda.set_device(0)
        print(json.dumps({"ragged_b64_paged": bench_ragged("K8V8", replays=4, steps=4)}),
              flush=True)
        return
    if args.prefill_only:
        import torch
        from fp8_kv_cache_append_amd import binding

        binding.lib()
        torch.cuda.set_device(0)
        print(json.dumps({"prefill": bench_prefill()}), flush=True)
        return
    if args.gpus != 1:
        print("bench.py measures one GPU: every box here has one, and the decode path "
              "has no cross-GPU step.", file=sys.stderr)
        sys.exit(2)

    import torch
    from fp8_kv_cache_append_amd import binding, synth

    binding.lib()
    torch.cuda.set_device(0)
    w = synth.decode_b16_gqa8_d128(2048)
    head, hb = bench_decode("K8V8", w, args.steps, args.warmup, args.copies)
    split_us = head["split_us"]
    achieved = head["kv_bytes"] / (split_us * 1e-6) / 1e9
    khash = kernel_source_hash()
    traffic = traffic_for(khash)
    extras = {}
    if not args.no_extras:
        outs = {"K8V8": step_output(hb)}
        for mode in ("K16V8", "BF16"):
            r, bb = bench_decode(mode, w, args.steps, args.warmup, args.copies)
            extras[mode] = r
            outs[mode] = step_output(bb)
            del bb
        ref = outs["BF16"]
        extras["fp8_vs_bf16"] = {
            m: float(((outs[m] - ref).norm() / ref.norm()).item()) for m in ("K8V8", "K16V8")}
        extras["K8V8_warm"] = bench_warm("K8V8", w, args.steps, args.copies)
        extras["copy_floor"] = bench_copy_floor(head["kv_bytes"])
        extras["append_bulk"] = bench_append_bulk()
        extras["prefill"] = bench_prefill()
        extras["prefill_bf16"] = bench_prefill(mode="BF16")
        extras["sweep"] = bench_sweep(max(640, args.steps // 4), max(64, args.warmup // 4),
                                      args.copies, head)
        extras["ragged"] = {m: bench_ragged(m) for m in ("K8V8", "K16V8")}
        extras["ragged"]["K8V8_pre_bias"] = bench_ragged("K8V8", pre_bias=True)
        extras["block_scaled"] = bench_block_scaled(max(640, args.steps // 4), args.copies)
    cpu = None if args.no_cpu_baseline else cpu_baseline(w)

    rec = {
        "metric": "KV-cache GB/s (% of 8 TB/s) and us/decode step, K8/V8 vs K16/V8 vs BF16",
        "value": head["kv_gbs"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": head["steps"],
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "decode_b16_hq16_hkv2_d128_t2048_k8v8_hbm_cold",
                   "batch": w.batch, "q_heads": w.q_heads, "kv_heads": w.kv_heads,
                   "head_dim": w.head_dim, "cached_tokens": int(w.lens[0]),
                   "kv_format": "e4m3 + fp32 scale per (token, KV head)",
                   "cache_state": f"HBM-cold, rotating {args.copies} copies",
                   "step": "split kernel with the append of 1 token/seq fused in + "
                           "merge kernel",
                   "split_plan": head["split_plan"]},
        "us_per_step": head["ms_per_step"] * 1e3,
        "pct_roofline": head["pct_roofline"],
        "split_us": head["split_us"],
        "kernel_us_event_pairs": head["kernel_us_event_pairs"],
        "unfused_step_us": head["unfused_step_us"],
        "dequant_then_bf16_step_us": head["dequant_then_bf16_step_us"],
        "narrow_qk_step_us": head["narrow_qk_step_us"],
        "narrow_qk_vs_bf16q_rel_l2": head["narrow_qk_vs_bf16q_rel_l2"],
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "kernel": "decode_partial_kernel<K8V8,128,append,one tile per wave>",
                     "bytes_per_launch": head["kv_bytes"],
                     "kernel_source_hash": khash},
        "cpu_baseline": cpu,
    }
    if extras:
        keys = ("ms_per_step", "kv_gbs", "pct_roofline", "split_us", "kernel_us_event_pairs",
                "unfused_step_us")
        rec["modes"] = {"K8V8": {k: head[k] for k in keys}}
        for mode in ("K16V8", "BF16"):
            rec["modes"][mode] = {k: extras[mode][k] for k in keys}
        rec["speedup_vs_bf16"] = extras["BF16"]["ms_per_step"] / head["ms_per_step"]
        rec["speedup_vs_k16v8"] = extras["K16V8"]["ms_per_step"] / head["ms_per_step"]
        # op-level error of the quantised caches: the GPU step's output
        # against the BF16-cache step's on the same inputs (relative L2)
        rec["fp8_vs_bf16_rel_l2"] = extras["fp8_vs_bf16"]
        rec["warm_l2_mall"] = extras["K8V8_warm"]
        rec["copy_floor_same_bytes"] = extras["copy_floor"]
        rec["append_bulk"] = extras["append_bulk"]
        rec["prefill"] = extras["prefill"]
        rec["prefill_bf16_control"] = extras["prefill_bf16"]
        rec["context_sweep"] = extras["sweep"]
        rec["ragged_b64_paged"] = extras["ragged"]
        rec["block_scaled_k"] = extras["block_scaled"]
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
