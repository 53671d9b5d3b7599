"""numpy marshalling around the plain-C oracle (oracle.c).

TEST INFRASTRUCTURE ONLY.  The oracle states, slowly and plainly, what the GPU
library computes; only the test suite, the smoke check and the CPU-baseline
leg of the benchmark may import it.  It never imports the GPU package and the
GPU package never imports it.  See oracle.h for the pages and sections each
step follows and for the readings taken where the pages are silent.

Conventions
-----------
* Modes: ``K8V8`` (K and V e4m3 + fp32 scale per (token, KV head)),
  ``K16V8`` (K bf16, V e4m3 + scale), ``BF16`` (K and V bf16).
* bf16 values travel as ``uint16`` bit patterns; e4m3 codes as ``uint8``.
* Query head ``h`` reads KV head ``h // G`` (GQA slicing of the FA page,
  section 3.1).
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liboracle.so")

MODES = {"K8V8": 0, "K16V8": 1, "BF16": 2, "K8V16": 3, "MXK8V8": 4}
K_E4M3 = ("K8V8", "K8V16", "MXK8V8")   # modes whose K side is e4m3 codes
V_E4M3 = ("K8V8", "K16V8", "MXK8V8")   # modes whose V side is e4m3 codes + scale
K_MX = ("MXK8V8",)                       # K codes with one E8M0 scale per 32 values

_lib = None


def lib() -> ctypes.CDLL:
    """Load liboracle.so, compiling it with gcc first if it is absent."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            from oracle.build import build
            build()
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.c_void_p
        L.orc_e4m3_value.restype = ctypes.c_double
        L.orc_e4m3_value.argtypes = [ctypes.c_uint8]
        L.orc_e4m3_encode.restype = ctypes.c_uint8
        L.orc_e4m3_encode.argtypes = [ctypes.c_float]
        L.orc_bf16_round.restype = ctypes.c_uint16
        L.orc_bf16_round.argtypes = [ctypes.c_double]
        L.orc_bf16_value.restype = ctypes.c_double
        L.orc_bf16_value.argtypes = [ctypes.c_uint16]
        L.orc_e4m3_encode_array.restype = None
        L.orc_e4m3_encode_array.argtypes = [P, P, ctypes.c_size_t]
        L.orc_bf16_round_array_f32.restype = None
        L.orc_bf16_round_array_f32.argtypes = [P, P, ctypes.c_size_t]
        L.orc_quantize_rows.restype = None
        L.orc_quantize_rows.argtypes = [P, ctypes.c_int64, ctypes.c_int, P, P]
        L.orc_dequantize_rows.restype = None
        L.orc_dequantize_rows.argtypes = [P, P, ctypes.c_int64, ctypes.c_int, P]
        L.orc_attend_rows.restype = None
        L.orc_attend_rows.argtypes = [
            ctypes.c_int, ctypes.c_int, ctypes.c_int, P, ctypes.c_int,
            P, P, P, P, P, P, P, ctypes.c_float, ctypes.c_int, P, P, P]
        L.orc_attend_rows_online.restype = None
        L.orc_attend_rows_online.argtypes = [
            ctypes.c_int, ctypes.c_int, ctypes.c_int, P, ctypes.c_int,
            P, P, P, P, P, P, P, ctypes.c_float, ctypes.c_int,
            ctypes.c_int, ctypes.c_int, P, P, P, P]
        L.orc_attend_rows_ex.restype = None
        L.orc_attend_rows_ex.argtypes = [
            ctypes.c_int, ctypes.c_int, ctypes.c_int, P, P, P, P, P, ctypes.c_int,
            P, P, P, P, P, P, P, P, ctypes.c_float, ctypes.c_int, P, P, P]
        L.orc_attend_rows_online_ex.restype = None
        L.orc_attend_rows_online_ex.argtypes = [
            ctypes.c_int, ctypes.c_int, ctypes.c_int, P, P, P, P, P, ctypes.c_int,
            P, P, P, P, P, P, P, P, ctypes.c_float, ctypes.c_int,
            ctypes.c_int, ctypes.c_int, P, P, P, P]
        L.orc_mx_exponent.restype = ctypes.c_int
        L.orc_mx_exponent.argtypes = [ctypes.c_float]
        L.orc_quantize_rows_mx.restype = None
        L.orc_quantize_rows_mx.argtypes = [P, ctypes.c_int64, ctypes.c_int, P, P]
        L.orc_attend_rows_q8.restype = None
        L.orc_attend_rows_q8.argtypes = [
            ctypes.c_int, ctypes.c_int, ctypes.c_int, P, P, ctypes.c_int,
            P, P, P, P, P, P, P, ctypes.c_float, ctypes.c_int, P, P, P]
        L.orc_attend_rows_online_q8.restype = None
        L.orc_attend_rows_online_q8.argtypes = [
            ctypes.c_int, ctypes.c_int, ctypes.c_int, P, P, ctypes.c_int,
            P, P, P, P, P, P, P, ctypes.c_float, ctypes.c_int,
            ctypes.c_int, ctypes.c_int, P, P, P, P]
        _lib = L
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return None if a is None else np.ascontiguousarray(a, dtype=dtype)


# ---------------------------------------------------------------- formats

def e4m3_value(codes) -> np.ndarray:
    """fp64 value of each e4m3 code (NaN for 0x7F and 0xFF)."""
    codes = np.asarray(codes, dtype=np.uint8)
    table = np.array([lib().orc_e4m3_value(c) for c in range(256)])
    return table[codes]


def e4m3_encode(y) -> np.ndarray:
    """Saturating round-to-nearest-even e4m3 code of each fp32 value."""
    y = _c(y, np.float32)
    out = np.empty(y.shape, dtype=np.uint8)
    lib().orc_e4m3_encode_array(_ptr(y), _ptr(out), y.size)
    return out


def bf16_round_f32(x) -> np.ndarray:
    """Round-to-nearest-even bf16 bit pattern of each fp32 value."""
    x = _c(x, np.float32)
    out = np.empty(x.shape, dtype=np.uint16)
    lib().orc_bf16_round_array_f32(_ptr(x), _ptr(out), x.size)
    return out


def bf16_round(x: float) -> int:
    """Round-to-nearest-even bf16 bit pattern of one fp64 value."""
    return int(lib().orc_bf16_round(float(x)))


def bf16_value(bits) -> np.ndarray:
    """fp64 value of bf16 bit patterns (bf16 is the top half of an fp32)."""
    bits = np.asarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


# ---------------------------------------------------------------- append

def quantize_rows(x):
    """Per-row e4m3 quantisation over the last axis.

    Returns (codes uint8 [..., D], scales fp32 [...]) with
    scale = fp32(amax / 448) and code = e4m3(fp32(x / scale)).
    """
    x = _c(x, np.float32)
    d = x.shape[-1]
    n = x.size // d if d else 0
    codes = np.empty(x.shape, dtype=np.uint8)
    scales = np.empty(x.shape[:-1], dtype=np.float32)
    lib().orc_quantize_rows(_ptr(x), n, d, _ptr(codes), _ptr(scales))
    return codes, scales


def dequantize_rows(codes, scales):
    """bf16 bits of bf16(fp32(value(code) * scale)) per element (the unfused
    control's conversion); codes uint8 [..., D], scales fp32 [...]."""
    codes = _c(codes, np.uint8)
    scales = _c(scales, np.float32)
    d = codes.shape[-1]
    n = codes.size // d if d else 0
    assert scales.shape == codes.shape[:-1]
    out = np.empty(codes.shape, dtype=np.uint16)
    lib().orc_dequantize_rows(_ptr(codes), _ptr(scales), n, d, _ptr(out))
    return out


def quantize_rows_mx(x):
    """Block-scaled (MX) quantisation over the last axis (a multiple of 32):
    returns (codes uint8 [..., D], exps uint8 [..., D/32]) with exps = E + 127,
    E = ceil(log2(fp32(amax of the block / 448))) clamped to [-126, 127],
    codes = e4m3(x / 2^E)."""
    x = _c(x, np.float32)
    d = x.shape[-1]
    assert d % 32 == 0
    n = x.size // d if d else 0
    codes = np.empty(x.shape, dtype=np.uint8)
    exps = np.empty(x.shape[:-1] + (d // 32,), dtype=np.uint8)
    lib().orc_quantize_rows_mx(_ptr(x), n, d, _ptr(codes), _ptr(exps))
    return codes, exps


def mx_exponent(amax: float) -> int:
    return int(lib().orc_mx_exponent(float(amax)))


def quantize_q_mx(q_bits):
    """Block-scaled QK: the bf16 query rows quantised by the MX rule."""
    return quantize_rows_mx(bf16_value(q_bits).astype(np.float32))


def quantize_q(q_bits):
    """Narrow QK: the bf16 query rows quantised once per decode step like
    cache rows (hardware notes, "Operating model" path 2).  q_bits uint16
    [..., D]; returns (codes uint8 [..., D], q_scale fp32 [...])."""
    q = bf16_value(q_bits).astype(np.float32)   # exact: bf16 is an fp32 prefix
    return quantize_rows(q)


def store_rows(mode: str, k, v) -> dict:
    """What the cache holds for fp32 K and V rows in the given mode.

    Keys: k8/ks (K8V8, K8V16), k8/kx (MXK8V8), k16 (K16V8, BF16), v8/vs
    (K8V8, K16V8, MXK8V8), v16 (BF16, K8V16).
    """
    if mode not in MODES:
        raise ValueError(mode)
    out = {}
    if mode in K_MX:
        out["k8"], out["kx"] = quantize_rows_mx(k)
    elif mode in K_E4M3:
        out["k8"], out["ks"] = quantize_rows(k)
    else:
        out["k16"] = bf16_round_f32(k)
    if mode in V_E4M3:
        out["v8"], out["vs"] = quantize_rows(v)
    else:
        out["v16"] = bf16_round_f32(v)
    return out


# ---------------------------------------------------------------- attention

def _head_view(store: dict, h: int) -> dict:
    """Slice one KV head out of [T, Hkv, D] / [T, Hkv] stores."""
    out = {}
    for key, arr in store.items():
        out[key] = np.ascontiguousarray(arr[:, h])
    return out


def _kv_args(kv: dict):
    return (_ptr(_c(kv.get("k8"), np.uint8)), _ptr(_c(kv.get("kx"), np.uint8)),
            _ptr(_c(kv.get("k16"), np.uint16)),
            _ptr(_c(kv.get("ks"), np.float32)), _ptr(_c(kv.get("v8"), np.uint8)),
            _ptr(_c(kv.get("v16"), np.uint16)), _ptr(_c(kv.get("vs"), np.float32)))


def attend_rows(mode: str, q_bits, kv: dict, n_valid, sm_scale: float,
                round_p: bool = True, bounds: bool = False, q8=None, k_bias=None):
    """Two-pass attention of query rows q_bits [R, D] against one KV head.

    kv holds the stores of that head ([T, D] and [T]); n_valid[r] keys are
    visible to row r.  Returns fp64 [R, D]; with bounds=True returns
    (out, lo, hi) where [lo, hi] holds every output reachable by rounding an
    ambiguous P (one within fp32 noise of a bf16 midpoint) either way.
    q8 = (codes uint8 [R, D], q_scale fp32 [R]): narrow QK on these query
    codes instead of q_bits (which may then be None); (codes, None, exps
    uint8 [R, D/32]): block-scaled (MX) query rows.  k_bias (fp32 [D]):
    the head's exact K bias; kv then holds the pre-bias residual rows.
    """
    q16, qc, qs, qx, r, d = _query_args(q_bits, q8)
    n_valid = _c(np.broadcast_to(np.asarray(n_valid), (r,)), np.int32)
    n_keys = _n_keys(kv)
    kb = _bias_arg(k_bias, d)
    out = np.empty((r, d), dtype=np.float64)
    lo = np.empty((r, d), dtype=np.float64) if bounds else None
    hi = np.empty((r, d), dtype=np.float64) if bounds else None
    lib().orc_attend_rows_ex(MODES[mode], d, r, _ptr(q16), _ptr(qc), _ptr(qs), _ptr(qx),
                             _ptr(kb), n_keys, *_kv_args(kv), _ptr(n_valid), float(sm_scale),
                             int(bool(round_p)), _ptr(out), _ptr(lo), _ptr(hi))
    return (out, lo, hi) if bounds else out


def _query_args(q_bits, q8):
    if q8 is None:
        q16 = _c(q_bits, np.uint16)
        return (q16, None, None, None) + q16.shape
    qc = _c(q8[0], np.uint8)
    if len(q8) == 3 and q8[1] is None:      # block-scaled rows
        qx = _c(q8[2], np.uint8)
        assert qx.shape == (qc.shape[0], qc.shape[1] // 32)
        return (None, qc, None, qx) + qc.shape
    qs = _c(q8[1], np.float32)
    assert qs.shape == qc.shape[:1]
    return (None, qc, qs, None) + qc.shape


def _bias_arg(k_bias, d):
    if k_bias is None:
        return None
    kb = _c(k_bias, np.float32)
    assert kb.shape == (d,), kb.shape
    return kb


def attend_rows_online(mode: str, q_bits, kv: dict, n_valid, sm_scale: float,
                       tile: int, split: int, round_p: bool = True, q8=None, k_bias=None):
    """Online (tiled, split, merged) attention; see orc_attend_rows_online.

    Returns (out [R, D], part_acc [S, R, D], part_l [S, R], part_m [S, R]).
    q8 and k_bias as for attend_rows.
    """
    q16, qc, qs, qx, r, d = _query_args(q_bits, q8)
    kb = _bias_arg(k_bias, d)
    n_valid = _c(np.broadcast_to(np.asarray(n_valid), (r,)), np.int32)
    n_keys = _n_keys(kv)
    n_splits = -(-n_keys // split) if n_keys else 0
    out = np.empty((r, d), dtype=np.float64)
    pacc = np.empty((max(n_splits, 1), r, d), dtype=np.float64)
    pl = np.empty((max(n_splits, 1), r), dtype=np.float64)
    pm = np.empty((max(n_splits, 1), r), dtype=np.float64)
    lib().orc_attend_rows_online_ex(
        MODES[mode], d, r, _ptr(q16), _ptr(qc), _ptr(qs), _ptr(qx), _ptr(kb), n_keys,
        *_kv_args(kv),
        _ptr(n_valid), float(sm_scale), int(bool(round_p)), int(tile), int(split),
        _ptr(pacc), _ptr(pl), _ptr(pm), _ptr(out))
    return out, pacc[:n_splits], pl[:n_splits], pm[:n_splits]


def _n_keys(kv: dict) -> int:
    for key in ("k8", "k16"):
        if kv.get(key) is not None:
            return int(kv[key].shape[0])
    raise ValueError("kv store holds no keys")


def decode(mode: str, q_bits, k_seqs, v_seqs, sm_scale: float,
           pairs=None, round_p: bool = True, bounds: bool = False, q8: bool = False,
           k_bias=None):
    """Decode attention from the fp32 K/V of each sequence.

    q_bits  bf16 bits [B, Hq, D]
    k_seqs  list of B fp32 arrays [len_b, Hkv, D] (v_seqs alike)
    pairs   optional iterable of (b, kv_head) to compute; other rows are NaN
    q8      narrow QK: Q quantised once (quantize_q; quantize_q_mx for the
            block-scaled MXK8V8 cache), scores on its codes
    k_bias  exact K bias fp32 [Hkv, D]: k_seqs are then the pre-bias
            residuals (stored quantised) and each key is residual + bias
    Returns fp64 [B, Hq, D] (with bounds=True: (out, lo, hi), see
    attend_rows).  The oracle quantises each sequence itself.
    """
    q_bits = np.asarray(q_bits, dtype=np.uint16)
    b_n, hq, d = q_bits.shape
    qc, qs, qx = None, None, None
    if q8 and mode in K_MX:
        qc, qx = quantize_q_mx(q_bits)
    elif q8:
        qc, qs = quantize_q(q_bits)
    out = np.full((b_n, hq, d), np.nan)
    lo, hi = out.copy(), out.copy()
    if b_n == 0:
        return (out, lo, hi) if bounds else out
    hkv = k_seqs[0].shape[1] if len(k_seqs) else 1
    g = hq // hkv
    if pairs is None:
        pairs = [(b, h) for b in range(b_n) for h in range(hkv)]
    by_seq = {}
    for b, h in pairs:
        by_seq.setdefault(b, []).append(h)
    for b, heads in by_seq.items():
        n = k_seqs[b].shape[0]
        store = store_rows(mode, k_seqs[b], v_seqs[b])
        for h in heads:
            rows = q_bits[b, h * g:(h + 1) * g]
            sl = slice(h * g, (h + 1) * g)
            rq8 = None
            if q8:
                rq8 = (qc[b, sl], None, qx[b, sl]) if qx is not None else (qc[b, sl], qs[b, sl])
            res = attend_rows(mode, rows, _head_view(store, h), n, sm_scale, round_p, bounds,
                              q8=rq8, k_bias=None if k_bias is None else k_bias[h])
            if bounds:
                out[b, sl], lo[b, sl], hi[b, sl] = res
            else:
                out[b, sl] = res
    return (out, lo, hi) if bounds else out


def prefill(mode: str, q_bits, k, v, q_pos0: int, sm_scale: float,
            rows=None, round_p: bool = True, bounds: bool = False):
    """Causal prefill of one sequence.

    q_bits  bf16 bits [Lq, Hq, D]; query i sits at position q_pos0 + i
    k, v    fp32 [Lkv, Hkv, D], every key of the sequence (positions 0..Lkv-1)
    rows    optional query indices to compute; other rows are NaN
    Key t is visible to query i when t <= q_pos0 + i (FA page, section 3.1).
    Returns fp64 [Lq, Hq, D] (with bounds=True: (out, lo, hi), see
    attend_rows).
    """
    q_bits = np.asarray(q_bits, dtype=np.uint16)
    lq, hq, d = q_bits.shape
    lkv, hkv = k.shape[0], k.shape[1]
    g = hq // hkv
    out = np.full((lq, hq, d), np.nan)
    lo, hi = out.copy(), out.copy()
    if rows is None:
        rows = np.arange(lq)
    rows = np.asarray(rows, dtype=np.int64)
    store = store_rows(mode, k, v)
    n_valid = np.minimum(q_pos0 + rows + 1, lkv).astype(np.int32)
    for hk in range(hkv):
        view = _head_view(store, hk)
        for hh in range(hk * g, (hk + 1) * g):
            res = attend_rows(mode, q_bits[rows, hh], view, n_valid, sm_scale, round_p, bounds)
            if bounds:
                out[rows, hh], lo[rows, hh], hi[rows, hh] = res
            else:
                out[rows, hh] = res
    return (out, lo, hi) if bounds else out


# ---------------------------------------------------------------- metrics

def rel_l2(a, ref) -> float:
    """||a - ref||_2 / ||ref||_2 over the whole tensor (0 when both are 0)."""
    a = np.asarray(a, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    num = np.sqrt(np.sum((a - ref) ** 2))
    den = np.sqrt(np.sum(ref ** 2))
    if den == 0.0:
        return 0.0 if num == 0.0 else float("inf")
    return float(num / den)


def max_abs(a, ref) -> float:
    a = np.asarray(a, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.max(np.abs(a - ref))) if a.size else 0.0


def fp8_kv_error(q_bits, k_seqs, v_seqs, sm_scale: float, mode: str = "K8V8",
                 pairs=None) -> float:
    """Relative L2 of a quantised mode's output against the BF16 mode on the
    same inputs (the op-level error the fp8-kv-cache page asks to report)."""
    a = decode(mode, q_bits, k_seqs, v_seqs, sm_scale, pairs)
    r = decode("BF16", q_bits, k_seqs, v_seqs, sm_scale, pairs)
    m = ~np.isnan(r)
    return rel_l2(a[m], r[m])
