"""The thread-pool driver of the oracle (tests/oracle_pool.py) schedules the
oracle's own calls and nothing else: on small workloads its results equal
oracle.decode / oracle.prefill exactly, element for element."""
import numpy as np

import oracle
from fp8_kv_cache_append_amd import synth
from oracle_pool import decode_full, prefill_full


def test_decode_full_equals_oracle_decode():
    lens = np.array([40, 1, 130], np.int32)
    w = synth.Workload("t", 3, 8, 2, 64, lens, "outliers", seed=5)
    seqs = [synth.kv_sequence(w, b) for b in range(w.batch)]
    q_bits = synth.q_bf16_bits(w.seed, (w.batch, w.q_heads, w.head_dim))
    for mode, q8 in (("K8V8", False), ("K16V8", False), ("K8V8", True)):
        got = decode_full(mode, q_bits, [s[0] for s in seqs], [s[1] for s in seqs],
                          w.sm_scale, q8=q8)
        want = oracle.decode(mode, q_bits, [s[0] for s in seqs], [s[1] for s in seqs],
                             w.sm_scale, bounds=True, q8=q8)
        for a, b in zip(got, want):
            assert np.array_equal(a, b), mode
        unr = decode_full(mode, q_bits, [s[0] for s in seqs], [s[1] for s in seqs],
                          w.sm_scale, round_p=False, q8=q8)[0]
        assert np.array_equal(unr, oracle.decode(mode, q_bits, [s[0] for s in seqs],
                                                 [s[1] for s in seqs], w.sm_scale,
                                                 round_p=False, q8=q8))


def test_decode_full_with_bias_equals_oracle_decode():
    lens = np.array([50, 17], np.int32)
    w = synth.Workload("t", 2, 8, 2, 128, lens, "bias", seed=6)
    parts = [synth.kv_sequence_prebias(w, b) for b in range(w.batch)]
    q_bits = synth.q_bf16_bits(w.seed, (w.batch, w.q_heads, w.head_dim))
    bias = parts[0][2]
    got = decode_full("K8V8", q_bits, [p[0] for p in parts], [p[1] for p in parts],
                      w.sm_scale, k_bias=bias)
    want = oracle.decode("K8V8", q_bits, [p[0] for p in parts], [p[1] for p in parts],
                         w.sm_scale, bounds=True, k_bias=bias)
    for a, b in zip(got, want):
        assert np.array_equal(a, b)


def test_prefill_full_equals_oracle_prefill():
    w = synth.Workload("t", 1, 8, 2, 64, np.array([70], np.int32), "normal", seed=7)
    k, v = synth.kv_sequence(w, 0)
    q_bits = synth.q_bf16_bits(w.seed, (60, w.q_heads, w.head_dim))
    got = prefill_full("K8V8", q_bits, k, v, 10, w.sm_scale)
    want = oracle.prefill("K8V8", q_bits, k, v, 10, w.sm_scale, bounds=True)
    for a, b in zip(got, want):
        assert np.array_equal(a, b)
