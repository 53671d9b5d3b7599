"""Helpers shared by the GPU parity tests: build a cache, append sequences
through the C ABI, run decode, read cache rows back in logical order.
Shapes are checked on the host before any launch."""
import numpy as np
import torch

from fp8_kv_cache_append_amd import binding, synth
from fp8_kv_cache_append_amd.binding import KVCache

DEV = "cuda"


def check_layout(table: np.ndarray, bs: int, lens) -> None:
    """Every token a sequence holds must map to a valid block-table entry."""
    for b, n in enumerate(np.asarray(lens)):
        need = -(-int(n) // bs)
        assert need <= table.shape[1], (b, n)
        assert np.all(table[b, :need] >= 0), (b, n)


def make_cache(mode: str, w: synth.Workload, capacity=None, layout="token") -> KVCache:
    bs, table, n_blocks = synth.block_layout(w, capacity)
    check_layout(table, bs, w.lens)
    return KVCache.allocate(mode, n_blocks, bs, w.kv_heads, w.head_dim, table, DEV,
                            layout=layout)


def append_seq(cache: KVCache, b: int, k: np.ndarray, v: np.ndarray, pos0: int = 0) -> None:
    n = k.shape[0]
    if n == 0:
        return
    table = cache.block_table.cpu().numpy()
    check_layout(table, cache.block_size, [0] * b + [pos0 + n])
    kt = torch.from_numpy(np.ascontiguousarray(k, np.float32)).to(DEV)
    vt = torch.from_numpy(np.ascontiguousarray(v, np.float32)).to(DEV)
    seq = torch.full((n,), b, dtype=torch.int32, device=DEV)
    pos = torch.arange(pos0, pos0 + n, dtype=torch.int32, device=DEV)
    binding.fp8kv_append(cache, kt, vt, seq, pos)


def read_rows(cache: KVCache, b: int, n: int) -> dict:
    """Cache contents of tokens 0..n-1 of sequence b, as oracle stores."""
    bs = cache.block_size
    table = cache.block_table.cpu().numpy()
    t = np.arange(n)
    blk = torch.from_numpy(table[b, t // bs].astype(np.int64)).to(DEV)
    slot = torch.from_numpy((t % bs).astype(np.int64)).to(DEV)
    out = {}

    def grab(x):  # rows of a block: [slot][head] or [head][slot]; -> [n, Hkv, ...]
        return (x[blk, slot] if cache.layout == "token" else x[blk, :, slot]).cpu()

    grab_scale = grab

    if cache.mode in binding.K_MX:
        out["k8"] = grab(cache.k).numpy()
        out["kx"] = grab_scale(cache.k_exp).numpy()
    elif cache.mode in binding.K_E4M3:
        out["k8"] = grab(cache.k).numpy()
        out["ks"] = grab_scale(cache.k_scale).numpy()
    else:
        out["k16"] = grab(cache.k).view(torch.int16).numpy().view(np.uint16)
    if cache.mode in binding.V_E4M3:
        out["v8"] = grab(cache.v).numpy()
        out["vs"] = grab_scale(cache.v_scale).numpy()
    else:
        out["v16"] = grab(cache.v).view(torch.int16).numpy().view(np.uint16)
    return out


def q_tensor(q_bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(q_bits).view(np.int16)).to(DEV).view(
        torch.bfloat16)


def decode(cache: KVCache, q_bits: np.ndarray, lens, group: int, sm_scale: float) -> np.ndarray:
    lens = np.asarray(lens, np.int32)
    b, hq, d = q_bits.shape
    assert hq == group * cache.num_kv_heads and d == cache.head_dim
    check_layout(cache.block_table.cpu().numpy(), cache.block_size, lens)
    max_len = int(lens.max()) if b else 0
    ws_bytes = binding.fp8kv_decode_workspace_bytes(cache, b, group, max_len)
    ws = torch.empty(max(ws_bytes // 4, 4), dtype=torch.float32, device=DEV)
    out = torch.full((b, hq, d), float("nan"), dtype=torch.float32, device=DEV)
    binding.fp8kv_decode(cache, q_tensor(q_bits), group, torch.from_numpy(lens).to(DEV),
                         max_len, sm_scale, out, ws)
    return out.cpu().numpy()


def decode_partial(cache: KVCache, q_bits, lens, group, sm_scale, chunk):
    lens = np.asarray(lens, np.int32)
    b, hq, d = q_bits.shape
    check_layout(cache.block_table.cpu().numpy(), cache.block_size, lens)
    max_len = int(lens.max())
    splits = -(-max_len // chunk)
    hkv = cache.num_kv_heads
    pacc = torch.full((b, hkv, splits, group, d), float("nan"), device=DEV)
    pml = torch.full((b, hkv, splits, group, 2), float("nan"), device=DEV)
    binding.fp8kv_decode_partial(cache, q_tensor(q_bits), group,
                                 torch.from_numpy(lens).to(DEV), max_len, sm_scale, chunk,
                                 splits, pacc, pml)
    return pacc.cpu().numpy(), pml.cpu().numpy()
