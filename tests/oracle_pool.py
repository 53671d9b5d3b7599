"""The oracle over a thread pool, for full-size comparisons.

The oracle's C calls release the interpreter lock (ctypes) and its
(sequence, KV head) and (query head) units share nothing, so workloads of
gigabytes can be checked in full on the host's cores.  Nothing here changes
what the oracle computes: every unit is oracle.store_rows +
oracle.attend_rows as they stand; this module only schedules them.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

import oracle

# the GPU machine's CPU share is 16 threads; fewer where the host has fewer cores
WORKERS = max(1, min(16, os.cpu_count() or 1))


class DecodeOracle:
    """Decode attention of whole sequences, one pool job per sequence.

    submit(b, k, v) queues sequence b (fp32 K/V [n, Hkv, D]; for a pre-bias
    cache the residual rows) as soon as its data exists, so the oracle runs
    while the caller fills the GPU cache; result() waits and returns
    (out, lo, hi), fp64 [B, Hq, D] (NaN for sequences never submitted).
    q8: the narrow QK path (queries quantised by oracle.quantize_q).
    """

    def __init__(self, mode, q_bits, sm_scale, kv_heads, round_p=True, q8=False, k_bias=None):
        self.mode, self.sm_scale, self.round_p = mode, float(sm_scale), round_p
        self.q_bits = np.asarray(q_bits, np.uint16)
        self.batch, hq, self.d = self.q_bits.shape
        self.hkv = int(kv_heads)
        self.g = hq // self.hkv
        self.k_bias = k_bias
        self.q8 = None
        if q8:
            self.q8 = oracle.quantize_q(self.q_bits)
        self.pool = ThreadPoolExecutor(WORKERS)
        self.futs = {}

    def _sequence(self, b, k, v):
        store = oracle.store_rows(self.mode, k, v)
        n = int(k.shape[0])
        res = []
        for h in range(self.hkv):
            sl = slice(h * self.g, (h + 1) * self.g)
            view = {key: np.ascontiguousarray(a[:, h]) for key, a in store.items()}
            rq8 = None if self.q8 is None else (self.q8[0][b, sl], self.q8[1][b, sl])
            res.append(oracle.attend_rows(
                self.mode, self.q_bits[b, sl], view, n, self.sm_scale, self.round_p,
                bounds=self.round_p, q8=rq8,
                k_bias=None if self.k_bias is None else self.k_bias[h]))
        return res

    def submit(self, b, k, v):
        self.futs[b] = self.pool.submit(self._sequence, b, k, v)

    def result(self):
        out = np.full((self.batch, self.hkv * self.g, self.d), np.nan)
        lo, hi = out.copy(), out.copy()
        for b, f in self.futs.items():
            for h, r in enumerate(f.result()):
                sl = slice(h * self.g, (h + 1) * self.g)
                if self.round_p:
                    out[b, sl], lo[b, sl], hi[b, sl] = r
                else:
                    out[b, sl] = lo[b, sl] = hi[b, sl] = r
        self.pool.shutdown()
        return out, lo, hi


def decode_full(mode, q_bits, k_seqs, v_seqs, sm_scale, round_p=True, q8=False,
                k_bias=None):
    """oracle.decode(..., bounds=True) over every (sequence, KV head) pair,
    spread over the pool."""
    hkv = k_seqs[0].shape[1]
    o = DecodeOracle(mode, q_bits, sm_scale, hkv, round_p=round_p, q8=q8, k_bias=k_bias)
    for b, (k, v) in enumerate(zip(k_seqs, v_seqs)):
        o.submit(b, k, v)
    return o.result()


def prefill_full(mode, q_bits, k, v, q_pos0, sm_scale, rows=None):
    """oracle.prefill(..., bounds=True) with one pool job per query head."""
    q_bits = np.asarray(q_bits, np.uint16)
    lq, hq, d = q_bits.shape
    lkv, hkv = k.shape[0], k.shape[1]
    g = hq // hkv
    rows = np.arange(lq) if rows is None else np.asarray(rows, np.int64)
    store = oracle.store_rows(mode, k, v)
    views = [{key: np.ascontiguousarray(a[:, hk]) for key, a in store.items()}
             for hk in range(hkv)]
    n_valid = np.minimum(q_pos0 + rows + 1, lkv).astype(np.int32)

    def head(hh):
        return oracle.attend_rows(mode, q_bits[rows, hh], views[hh // g], n_valid, sm_scale,
                                  bounds=True)

    out = np.full((lq, hq, d), np.nan)
    lo, hi = out.copy(), out.copy()
    with ThreadPoolExecutor(WORKERS) as pool:
        for hh, (o, l, h) in enumerate(pool.map(head, range(hq))):
            out[rows, hh], lo[rows, hh], hi[rows, hh] = o, l, h
    return out, lo, hi
