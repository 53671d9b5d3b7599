"""Python binding of the fp8kv C ABI (include/fp8kv.h).

Argument marshalling only: torch tensors supply device memory and the current
HIP stream; every computation runs in the HIP kernels of libfp8kv.so.  There
is no fallback: if the library is missing or the call fails, an exception is
raised.  Function names and argument order follow the C ABI.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libfp8kv.so")

MODES = {"K8V8": 0, "K16V8": 1, "BF16": 2, "K8V16": 3, "MXK8V8": 4}
K_E4M3 = ("K8V8", "K8V16", "MXK8V8")  # K side: uint8 e4m3 codes (else bf16)
V_E4M3 = ("K8V8", "K16V8", "MXK8V8")  # V side: uint8 e4m3 codes + fp32 scale (else bf16)
K_MX = ("MXK8V8",)                     # K codes with an E8M0 byte per 32 values (k_exp)

LAYOUTS = {"token": 0, "head": 1}   # row order in a block: [slot][head] or [head][slot]

FP8KV_OK = 0
FP8KV_ERR_INVALID = -1
FP8KV_ERR_WORKSPACE = -2
FP8KV_ERR_LAUNCH = -3
FP8KV_ERR_UNSUPPORTED = -4
FP8KV_ERR_TOO_LARGE = -5

# Every symbol include/fp8kv.h declares.
EXPORTS = ("fp8kv_append", "fp8kv_decode_plan", "fp8kv_decode_workspace_bytes",
           "fp8kv_decode_partial", "fp8kv_decode_merge", "fp8kv_decode",
           "fp8kv_decode_append", "fp8kv_decode_append_partial", "fp8kv_decode_q8",
           "fp8kv_decode_append_q8", "fp8kv_prefill", "fp8kv_dequantize", "fp8kv_strerror",
           "fp8kv_decode_noalloc")


class Fp8kvError(RuntimeError):
    def __init__(self, status: int, call: str):
        self.status = status
        super().__init__(f"{call}: {strerror(status)} ({status})")


class CacheDesc(ctypes.Structure):
    """Mirror of struct fp8kv_cache."""
    _fields_ = [("mode", ctypes.c_int32), ("num_blocks", ctypes.c_int32),
                ("block_size", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("max_blocks_per_seq", ctypes.c_int32),
                ("num_seqs", ctypes.c_int32), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("k_scale", ctypes.c_void_p), ("v_scale", ctypes.c_void_p),
                ("block_table", ctypes.c_void_p), ("k_bias", ctypes.c_void_p),
                ("k_exp", ctypes.c_void_p), ("layout", ctypes.c_int32)]


_lib = None


def lib() -> ctypes.CDLL:
    """Load libfp8kv.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "fp8_kv_cache_append_amd/build.py (no CPU fallback exists)")
        L = ctypes.CDLL(LIB_PATH)
        P, I32, F = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float
        C = ctypes.POINTER(CacheDesc)
        sig = {
            "fp8kv_append": (ctypes.c_int, [C, P, P, P, P, I32, P]),
            "fp8kv_decode_plan": (ctypes.c_int, [C, I32, I32, I32, ctypes.POINTER(I32),
                                                 ctypes.POINTER(I32)]),
            "fp8kv_decode_workspace_bytes": (ctypes.c_size_t, [C, I32, I32, I32]),
            "fp8kv_decode_partial": (ctypes.c_int, [C, P, I32, P, I32, I32, F, I32, I32,
                                                    P, P, P]),
            "fp8kv_decode_merge": (ctypes.c_int, [I32, I32, I32, I32, I32, P, P, P, P]),
            "fp8kv_decode": (ctypes.c_int, [C, P, I32, P, I32, I32, F, P, P,
                                            ctypes.c_size_t, P]),
            "fp8kv_decode_append": (ctypes.c_int, [C, P, P, P, I32, P, I32, I32, F, P, P,
                                                   ctypes.c_size_t, P]),
            "fp8kv_decode_q8": (ctypes.c_int, [C, P, I32, P, I32, I32, F, P, P,
                                               ctypes.c_size_t, P]),
            "fp8kv_decode_append_q8": (ctypes.c_int, [C, P, P, P, I32, P, I32, I32, F, P, P,
                                                      ctypes.c_size_t, P]),
            "fp8kv_decode_append_partial": (ctypes.c_int, [C, P, P, P, I32, P, I32, I32, F,
                                                           I32, I32, P, P, P]),
            "fp8kv_prefill": (ctypes.c_int, [C, P, I32, P, P, P, I32, I32, I32, F, P, P]),
            "fp8kv_dequantize": (ctypes.c_int, [C, C, P]),
            "fp8kv_decode_noalloc": (ctypes.c_int, [C, P, I32, P, I32, I32, F, P, P]),
            "fp8kv_strerror": (ctypes.c_char_p, [ctypes.c_int]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype, fn.argtypes = res, args
        _lib = L
    return _lib


def strerror(status: int) -> str:
    return lib().fp8kv_strerror(int(status)).decode()


def _check(status: int, call: str) -> None:
    if status != FP8KV_OK:
        raise Fp8kvError(status, call)


def _ptr(t):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        return t  # a raw integer address, passed through
    if not t.is_contiguous():
        raise ValueError("tensors passed to fp8kv must be contiguous")
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


@dataclass
class KVCache:
    """A paged cache in device memory plus its C descriptor.

    layout "token" (rows of a block in [slot][head] order) or "head"
    ([head][slot]); with R the block's rows in that order, shaped
    (block_size, Hkv) or (Hkv, block_size):
    k, v: uint8 (e4m3 codes) or bfloat16 [num_blocks, *R, D];
    k_scale, v_scale: float32 [num_blocks, *R] for an e4m3 side, else None;
    k_exp: uint8 [num_blocks, *R, D / 32] for block-scaled K, else None;
    block_table: int32 [batch, max_blocks_per_seq]; with table_in_memory False
    the descriptor passes no table and the library computes the contiguous
    ids b * max_blocks_per_seq + e (block_table then only gives the shape);
    k_bias: float32 [Hkv, D] for a pre-bias residual cache (the stored K rows
    are residuals, the key is residual + k_bias), else None.
    """
    mode: str
    k: torch.Tensor
    v: torch.Tensor
    k_scale: torch.Tensor | None
    v_scale: torch.Tensor | None
    block_table: torch.Tensor
    k_bias: torch.Tensor | None = None
    k_exp: torch.Tensor | None = None
    table_in_memory: bool = True   # False: pass no table (contiguous layout)
    layout: str = "token"

    @classmethod
    def allocate(cls, mode: str, num_blocks: int, block_size: int, num_kv_heads: int,
                 head_dim: int, block_table, device="cuda",
                 table_in_memory: bool = True, layout: str = "token") -> "KVCache":
        if layout not in LAYOUTS:
            raise ValueError(layout)
        rows = (block_size, num_kv_heads) if layout == "token" else (num_kv_heads, block_size)
        shape = (num_blocks, *rows, head_dim)
        k8, v8, kmx = mode in K_E4M3, mode in V_E4M3, mode in K_MX
        k = torch.zeros(shape, dtype=torch.uint8 if k8 else torch.bfloat16, device=device)
        v = torch.zeros(shape, dtype=torch.uint8 if v8 else torch.bfloat16, device=device)
        sshape = (num_blocks, *rows)
        ks = torch.zeros(sshape, dtype=torch.float32, device=device) if k8 and not kmx else None
        vs = torch.zeros(sshape, dtype=torch.float32, device=device) if v8 else None
        kx = torch.zeros(sshape + (head_dim // 32,), dtype=torch.uint8,
                         device=device) if kmx else None
        bt = torch.as_tensor(block_table, dtype=torch.int32).to(device).contiguous()
        if not table_in_memory:
            # the library then computes block b * max_blocks_per_seq + e itself
            want = torch.arange(bt.numel(), dtype=torch.int32, device=device).view(bt.shape)
            if not torch.equal(bt, want):
                raise ValueError("table_in_memory=False needs the contiguous table")
        return cls(mode, k, v, ks, vs, bt, None, kx, table_in_memory, layout)

    @property
    def head_dim(self) -> int:
        return int(self.k.shape[3])

    @property
    def num_kv_heads(self) -> int:
        return int(self.k.shape[2] if self.layout == "token" else self.k.shape[1])

    @property
    def block_size(self) -> int:
        return int(self.k.shape[1] if self.layout == "token" else self.k.shape[2])

    def desc(self) -> CacheDesc:
        return CacheDesc(MODES[self.mode], int(self.k.shape[0]), self.block_size,
                         self.num_kv_heads, self.head_dim,
                         int(self.block_table.shape[1]), int(self.block_table.shape[0]),
                         _ptr(self.k), _ptr(self.v),
                         _ptr(self.k_scale), _ptr(self.v_scale),
                         _ptr(self.block_table) if self.table_in_memory else None,
                         _ptr(self.k_bias), _ptr(self.k_exp), LAYOUTS[self.layout])


def fp8kv_append(cache: KVCache, k_new, v_new, seq_idx, pos, stream=None) -> None:
    """Quantise and store n_tok new tokens (k_new, v_new: fp32 [n_tok, Hkv, D])."""
    d = cache.desc()
    _check(lib().fp8kv_append(ctypes.byref(d), _ptr(k_new), _ptr(v_new), _ptr(seq_idx),
                              _ptr(pos), int(k_new.shape[0]), _stream(stream)), "fp8kv_append")


def fp8kv_decode_plan(cache: KVCache, batch: int, gqa_group: int, max_seq_len: int):
    """(chunk_tokens, n_splits) of the split-KV decode."""
    d = cache.desc()
    chunk, splits = ctypes.c_int32(), ctypes.c_int32()
    _check(lib().fp8kv_decode_plan(ctypes.byref(d), batch, gqa_group, max_seq_len,
                                   ctypes.byref(chunk), ctypes.byref(splits)),
           "fp8kv_decode_plan")
    return chunk.value, splits.value


def fp8kv_decode_workspace_bytes(cache: KVCache, batch: int, gqa_group: int,
                                 max_seq_len: int) -> int:
    d = cache.desc()
    return int(lib().fp8kv_decode_workspace_bytes(ctypes.byref(d), batch, gqa_group,
                                                  max_seq_len))


def fp8kv_decode_partial(cache: KVCache, q, gqa_group: int, seq_lens, max_seq_len: int,
                         sm_scale: float, chunk_tokens: int, n_splits: int, part_acc,
                         part_ml, stream=None) -> None:
    d = cache.desc()
    _check(lib().fp8kv_decode_partial(ctypes.byref(d), _ptr(q), gqa_group, _ptr(seq_lens),
                                      int(seq_lens.shape[0]), max_seq_len, sm_scale,
                                      chunk_tokens, n_splits, _ptr(part_acc), _ptr(part_ml),
                                      _stream(stream)), "fp8kv_decode_partial")


def fp8kv_decode_merge(batch: int, num_kv_heads: int, gqa_group: int, head_dim: int,
                       n_splits: int, part_acc, part_ml, out, stream=None) -> None:
    _check(lib().fp8kv_decode_merge(batch, num_kv_heads, gqa_group, head_dim, n_splits,
                                    _ptr(part_acc), _ptr(part_ml), _ptr(out),
                                    _stream(stream)), "fp8kv_decode_merge")


def fp8kv_decode(cache: KVCache, q, gqa_group: int, seq_lens, max_seq_len: int,
                 sm_scale: float, out, workspace, stream=None) -> None:
    d = cache.desc()
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().fp8kv_decode(ctypes.byref(d), _ptr(q), gqa_group, _ptr(seq_lens),
                              int(seq_lens.shape[0]), max_seq_len, sm_scale, _ptr(out),
                              _ptr(workspace), ws_bytes, _stream(stream)), "fp8kv_decode")


def fp8kv_decode_noalloc(cache: KVCache, q, gqa_group: int, seq_lens, max_seq_len: int,
                         sm_scale: float, out, stream=None) -> None:
    """fp8kv_decode with the partials in the library's own device scratch
    (no workspace; see include/fp8kv.h for the limit)."""
    d = cache.desc()
    _check(lib().fp8kv_decode_noalloc(ctypes.byref(d), _ptr(q), gqa_group, _ptr(seq_lens),
                                      int(seq_lens.shape[0]), max_seq_len, sm_scale, _ptr(out),
                                      _stream(stream)), "fp8kv_decode_noalloc")


def fp8kv_decode_q8(cache: KVCache, q, gqa_group: int, seq_lens, max_seq_len: int,
                    sm_scale: float, out, workspace, stream=None) -> None:
    """fp8kv_decode with narrow QK (Q quantised to e4m3 in the kernel)."""
    d = cache.desc()
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().fp8kv_decode_q8(ctypes.byref(d), _ptr(q), gqa_group, _ptr(seq_lens),
                                 int(seq_lens.shape[0]), max_seq_len, sm_scale, _ptr(out),
                                 _ptr(workspace), ws_bytes, _stream(stream)), "fp8kv_decode_q8")


def fp8kv_decode_append_q8(cache: KVCache, k_new, v_new, q, gqa_group: int, seq_lens,
                           max_seq_len: int, sm_scale: float, out, workspace,
                           stream=None) -> None:
    """fp8kv_decode_append with narrow QK."""
    d = cache.desc()
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().fp8kv_decode_append_q8(ctypes.byref(d), _ptr(k_new), _ptr(v_new), _ptr(q),
                                        gqa_group, _ptr(seq_lens), int(seq_lens.shape[0]),
                                        max_seq_len, sm_scale, _ptr(out), _ptr(workspace),
                                        ws_bytes, _stream(stream)), "fp8kv_decode_append_q8")


def fp8kv_decode_append(cache: KVCache, k_new, v_new, q, gqa_group: int, seq_lens,
                        max_seq_len: int, sm_scale: float, out, workspace, stream=None) -> None:
    """Store each sequence's new token (k_new, v_new: fp32 [batch, Hkv, D]) at
    position seq_lens[b] - 1, then decode over seq_lens[b] keys."""
    d = cache.desc()
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().fp8kv_decode_append(ctypes.byref(d), _ptr(k_new), _ptr(v_new), _ptr(q),
                                     gqa_group, _ptr(seq_lens), int(seq_lens.shape[0]),
                                     max_seq_len, sm_scale, _ptr(out), _ptr(workspace),
                                     ws_bytes, _stream(stream)), "fp8kv_decode_append")


def fp8kv_decode_append_partial(cache: KVCache, k_new, v_new, q, gqa_group: int, seq_lens,
                                max_seq_len: int, sm_scale: float, chunk_tokens: int,
                                n_splits: int, part_acc, part_ml, stream=None) -> None:
    d = cache.desc()
    _check(lib().fp8kv_decode_append_partial(
        ctypes.byref(d), _ptr(k_new), _ptr(v_new), _ptr(q), gqa_group, _ptr(seq_lens),
        int(seq_lens.shape[0]), max_seq_len, sm_scale, chunk_tokens, n_splits, _ptr(part_acc),
        _ptr(part_ml), _stream(stream)), "fp8kv_decode_append_partial")


def fp8kv_prefill(cache: KVCache, q, gqa_group: int, cu_q, q_pos0, seq_lens,
                  max_q_len: int, sm_scale: float, out, stream=None) -> None:
    d = cache.desc()
    _check(lib().fp8kv_prefill(ctypes.byref(d), _ptr(q), gqa_group, _ptr(cu_q), _ptr(q_pos0),
                               _ptr(seq_lens), int(seq_lens.shape[0]), int(q.shape[0]),
                               max_q_len, sm_scale, _ptr(out), _stream(stream)),
           "fp8kv_prefill")


def fp8kv_dequantize(src: KVCache, dst: KVCache, stream=None) -> None:
    """Convert every row of src into dst (a BF16-mode cache of the same
    geometry): the unfused control."""
    ds, dd = src.desc(), dst.desc()
    _check(lib().fp8kv_dequantize(ctypes.byref(ds), ctypes.byref(dd), _stream(stream)),
           "fp8kv_dequantize")


def fp8kv_strerror(status: int) -> str:
    return strerror(status)
