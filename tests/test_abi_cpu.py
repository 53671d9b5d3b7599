"""The C-ABI library without a GPU: it loads, exports every symbol the header
declares, and its host-side validation rejects bad arguments before any
launch.  Every call here returns on the host before touching a device."""
import ctypes
import os
import re
import subprocess

import pytest

from fp8_kv_cache_append_amd import binding
from fp8_kv_cache_append_amd.binding import CacheDesc

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fp8kv.h")

pytestmark = pytest.mark.skipif(not os.path.exists(binding.LIB_PATH),
                                reason="libfp8kv.so not built")

FAKE = 0x10000  # aligned host-side stand-in; never dereferenced by these calls


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return set(re.findall(r"\b(fp8kv_[a-z0-9_]+)\s*\(", text))


def test_header_declares_binding_exports():
    assert _declared() == set(binding.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = binding.lib()
    for name in _declared():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", binding.LIB_PATH],
                         capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\s[TW]\s+(fp8kv_\w+)$", out, flags=re.M))
    assert _declared() <= exported


def test_strerror():
    assert binding.strerror(0) == "ok"
    assert "invalid" in binding.strerror(-1)
    assert "workspace" in binding.strerror(-2)
    assert "unknown" in binding.strerror(7)


def _desc(**kw):
    base = dict(mode=0, num_blocks=4, block_size=16, num_kv_heads=2, head_dim=128,
                max_blocks_per_seq=4, num_seqs=16, k=FAKE, v=FAKE, k_scale=FAKE, v_scale=FAKE,
                block_table=FAKE, k_bias=None, k_exp=None, layout=0)
    base.update(kw)
    return CacheDesc(**base)


BAD_CACHES = [
    (dict(mode=5), -1),
    (dict(layout=2), -1),               # token-major (0) or head-major (1) only
    (dict(layout=-1), -1),
    (dict(mode=3), -1),                 # K8V16 stores no V scale: v_scale must be NULL
    (dict(mode=3, v_scale=None, k_scale=None), -1),   # ... but a K scale
    (dict(head_dim=96), -4),
    (dict(block_size=8), -1),
    (dict(block_size=0), -1),
    (dict(num_kv_heads=0), -1),
    (dict(num_seqs=0), -1),
    (dict(k=None), -1),
    (dict(k=FAKE + 4), -1),          # codes must be 16-byte aligned
    (dict(k_scale=None), -1),        # K8V8 needs both scales
    (dict(mode=1), -1),              # K16V8 must not carry a K scale
    (dict(mode=2, k_scale=None), -1),  # BF16 must not carry a V scale
    (dict(block_table=FAKE + 2), -1),
    # no table: block ids b * max_blocks_per_seq + e must fit an int32
    (dict(block_table=None, num_seqs=2**20, max_blocks_per_seq=2**12), -1),
    # ... and must all be blocks of the cache (16 sequences x 4 blocks > 63)
    (dict(block_table=None, num_blocks=63), -1),
    (dict(k_bias=FAKE + 4), -1),        # the bias is read 16 bytes at a time
    (dict(mode=4), -1),                 # block-scaled K: no K row scale, but k_exp
    (dict(mode=4, k_scale=None), -1),   # ... k_exp missing
    (dict(k_exp=FAKE), -1),             # k_exp only with block-scaled K
    (dict(mode=4, k_scale=None, k_exp=FAKE + 2), -1),   # misaligned
    (dict(mode=4, k_scale=None, k_exp=FAKE, k_bias=FAKE), -4),  # no bias on block scales
]


def test_contiguous_cache_without_table_is_valid():
    # no table, and exactly num_seqs * max_blocks_per_seq blocks: accepted
    # (append reaches the device check, which has no GPU here)
    d = _desc(block_table=None, num_blocks=64)
    r = binding.lib().fp8kv_append(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, 1, None)
    assert r in (0, -4), r


@pytest.mark.parametrize("kw,status", BAD_CACHES)
def test_append_rejects_bad_cache(kw, status):
    d = _desc(**kw)
    r = binding.lib().fp8kv_append(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, 1, None)
    assert r == status


def test_append_rejects_bad_arguments():
    lib = binding.lib()
    d = _desc()
    assert lib.fp8kv_append(None, FAKE, FAKE, FAKE, FAKE, 1, None) == -1
    assert lib.fp8kv_append(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, -1, None) == -1
    assert lib.fp8kv_append(ctypes.byref(d), None, FAKE, FAKE, FAKE, 1, None) == -1
    assert lib.fp8kv_append(ctypes.byref(d), FAKE + 4, FAKE, FAKE, FAKE, 1, None) == -1
    # zero tokens is a no-op that succeeds without a device
    assert lib.fp8kv_append(ctypes.byref(d), None, None, None, None, 0, None) == 0


def _plan(d, b, g, t):
    c, s = ctypes.c_int32(), ctypes.c_int32()
    r = binding.lib().fp8kv_decode_plan(ctypes.byref(d), b, g, t, ctypes.byref(c),
                                        ctypes.byref(s))
    return r, c.value, s.value


def test_decode_plan():
    # contiguous B16 x 2 KV heads x 2048 tokens
    d = _desc(num_blocks=16, block_size=2048, max_blocks_per_seq=1)
    assert _plan(d, 16, 8, 2048) == (0, 256, 8)
    # the same cache passed with no table (contiguous ids) is valid
    d = _desc(num_blocks=16, block_size=2048, max_blocks_per_seq=1, block_table=None)
    assert _plan(d, 16, 8, 2048) == (0, 256, 8)
    # paged B64 x 8 KV heads up to 32768 tokens: longer splits, bounded grid
    d = _desc(num_blocks=70000, block_size=16, num_kv_heads=8, max_blocks_per_seq=2048,
              num_seqs=64)
    r, c, s = _plan(d, 64, 4, 32768)
    assert r == 0 and c == 1024 and s == 32
    assert _plan(d, 64, 17, 32768)[0] == -4
    assert _plan(d, 64, 0, 32768)[0] == -1
    assert _plan(d, 64, 4, 32768 + 1)[0] == -1   # beyond the block table
    assert _plan(d, 0, 4, 0) == (0, 128, 0)
    # contiguous B16 x 2 KV heads: the chunk doubles while every one of the
    # 256 compute units still gets a work-group
    d = _desc(num_blocks=16, block_size=8192, max_blocks_per_seq=1)
    assert _plan(d, 16, 8, 4096) == (0, 512, 8)      # 256 work-groups
    assert _plan(d, 16, 8, 8192) == (0, 1024, 8)     # 256 work-groups
    assert _plan(d, 16, 8, 512) == (0, 128, 4)       # 64 at 256: half-tile splits, 128
    assert _plan(d, 16, 8, 2048) == (0, 256, 8)      # 256 work-groups at 256 keys
    assert _plan(d, 16, 8, 4097) == (0, 512, 9)
    d16 = _desc(mode=1, num_blocks=16, block_size=8192, max_blocks_per_seq=1, k_scale=None)
    assert _plan(d16, 16, 8, 8192) == (0, 1024, 8)
    big = dict(num_blocks=24, block_size=16384, max_blocks_per_seq=1, num_seqs=24)
    assert _plan(_desc(mode=1, k_scale=None, **big), 16, 8, 16384) == (0, 1024, 16)
    assert _plan(_desc(**big), 16, 8, 16384) == (0, 1024, 16)
    assert _plan(_desc(**big), 1, 8, 16384) == (0, 256, 64)   # 2 pairs: 128 work-groups
    assert _plan(_desc(**big), 24, 8, 8192) == (0, 1024, 8)
    d64 = _desc(mode=2, num_blocks=16, block_size=8192, max_blocks_per_seq=1, head_dim=64,
                k_scale=None, v_scale=None)
    assert _plan(d64, 16, 8, 8192) == (0, 1024, 8)


def test_workspace_bytes():
    d = _desc(num_blocks=16, block_size=2048, max_blocks_per_seq=1)
    n = binding.lib().fp8kv_decode_workspace_bytes(ctypes.byref(d), 16, 8, 2048)
    assert n == 16 * 2 * 8 * 8 * (128 + 2) * 4
    bad = _desc(head_dim=96)
    assert binding.lib().fp8kv_decode_workspace_bytes(ctypes.byref(bad), 16, 8, 2048) == 0


def test_decode_rejects_bad_arguments():
    lib = binding.lib()
    d = _desc(num_blocks=16, block_size=2048, max_blocks_per_seq=1)
    # workspace too small
    assert lib.fp8kv_decode(ctypes.byref(d), FAKE, 8, FAKE, 16, 2048, 0.1, FAKE,
                            FAKE, 16, None) == -2
    assert lib.fp8kv_decode(ctypes.byref(d), FAKE, 8, FAKE, 16, 2048, 0.1, FAKE,
                            None, 10 ** 9, None) == -2
    # chunk not a multiple of 64, too few splits, misaligned partials
    args = (ctypes.byref(d), FAKE, 8, FAKE, 16, 2048, 0.1)
    assert lib.fp8kv_decode_partial(*args, 100, 32, FAKE, FAKE, None) == -1
    assert lib.fp8kv_decode_partial(*args, 256, 7, FAKE, FAKE, None) == -1
    assert lib.fp8kv_decode_partial(*args, 256, 8, FAKE + 4, FAKE, None) == -1
    small = _desc(num_blocks=16, block_size=16, max_blocks_per_seq=128)
    assert lib.fp8kv_decode_partial(ctypes.byref(small), FAKE, 8, FAKE, 16, 2048, 0.1,
                                    2048, 1, FAKE, FAKE, None) == -1   # > 64 blocks a split
    # a chunk <= 64 * block_size whose splits start inside a block can still
    # reach 65 blocks (block_size 112, chunk 7104: split 1 starts at slot 48)
    odd = _desc(num_blocks=16, block_size=112, max_blocks_per_seq=200)
    assert lib.fp8kv_decode_partial(ctypes.byref(odd), FAKE, 8, FAKE, 16, 14208, 0.1,
                                    7104, 2, FAKE, FAKE, None) == -1
    # more splits than the capacity needs: split * chunk would pass 2^31 in
    # the kernel's 32-bit arithmetic (chunk 1024, 2^21 + 1 splits), or merely
    # start past the block table
    big = _desc(num_blocks=1, block_size=1024, max_blocks_per_seq=1, num_seqs=1)
    assert lib.fp8kv_decode_partial(ctypes.byref(big), FAKE, 8, FAKE, 1, 1024, 0.1,
                                    1024, 2 ** 21 + 1, FAKE, FAKE, None) == -1
    assert lib.fp8kv_decode_partial(ctypes.byref(big), FAKE, 8, FAKE, 1, 1024, 0.1,
                                    1024, 2, FAKE, FAKE, None) == -1
    assert lib.fp8kv_decode_append_partial(ctypes.byref(big), FAKE, FAKE, FAKE, 8, FAKE, 1,
                                           1024, 0.1, 1024, 2 ** 21 + 1, FAKE, FAKE,
                                           None) == -1
    assert lib.fp8kv_decode_plan(ctypes.byref(d), 17, 8, 2048, ctypes.byref(ctypes.c_int32()),
                                 ctypes.byref(ctypes.c_int32())) == -1  # batch > table rows
    # merge shape checks
    assert lib.fp8kv_decode_merge(4, 2, 17, 128, 4, FAKE, FAKE, FAKE, None) == -4
    assert lib.fp8kv_decode_merge(4, 2, 8, 96, 4, FAKE, FAKE, FAKE, None) == -4
    assert lib.fp8kv_decode_merge(4, 2, 8, 128, 4, None, FAKE, FAKE, None) == -1
    assert lib.fp8kv_decode_merge(0, 2, 8, 128, 4, None, None, None, None) == 0


def test_decode_append_rejects_bad_arguments():
    lib = binding.lib()
    d = _desc(num_blocks=16, block_size=2048, max_blocks_per_seq=1)
    args = (FAKE, 8, FAKE, 16, 2048, 0.1, FAKE, FAKE, 10 ** 9, None)
    assert lib.fp8kv_decode_append(ctypes.byref(d), None, FAKE, *args) == -1   # no K rows
    assert lib.fp8kv_decode_append(ctypes.byref(d), FAKE, None, *args) == -1   # no V rows
    assert lib.fp8kv_decode_append(ctypes.byref(d), FAKE + 4, FAKE, *args) == -1  # misaligned
    assert lib.fp8kv_decode_append(ctypes.byref(d), FAKE, FAKE, FAKE, 8, FAKE, 16, 2048, 0.1,
                                   FAKE, FAKE, 16, None) == -2                  # workspace
    assert lib.fp8kv_decode_append(ctypes.byref(d), None, None, FAKE, 8, FAKE, 0, 0, 0.1,
                                   FAKE, None, 0, None) == 0                    # empty batch


def test_narrow_qk_entries_validate_like_the_bf16_ones():
    lib = binding.lib()
    d = _desc(num_blocks=16, block_size=2048, max_blocks_per_seq=1)
    # workspace too small, misaligned output, missing rows for the append
    assert lib.fp8kv_decode_q8(ctypes.byref(d), FAKE, 8, FAKE, 16, 2048, 0.1, FAKE,
                               FAKE, 16, None) == -2
    assert lib.fp8kv_decode_q8(ctypes.byref(d), FAKE, 8, FAKE, 16, 2048, 0.1, FAKE + 4,
                               FAKE, 10 ** 9, None) == -1
    assert lib.fp8kv_decode_q8(ctypes.byref(d), FAKE, 17, FAKE, 16, 2048, 0.1, FAKE,
                               FAKE, 10 ** 9, None) == -4   # group > 16
    args = (FAKE, 8, FAKE, 16, 2048, 0.1, FAKE, FAKE, 10 ** 9, None)
    assert lib.fp8kv_decode_append_q8(ctypes.byref(d), None, FAKE, *args) == -1
    assert lib.fp8kv_decode_append_q8(ctypes.byref(d), FAKE + 4, FAKE, *args) == -1
    assert lib.fp8kv_decode_append_q8(ctypes.byref(d), None, None, FAKE, 8, FAKE, 0, 0, 0.1,
                                      FAKE, None, 0, None) == 0   # empty batch


def test_noalloc_refuses_beyond_its_scratch_on_the_host():
    """fp8kv_decode_noalloc refuses partials above its 64 MiB scratch before
    touching a device, and validates like fp8kv_decode otherwise."""
    lib = binding.lib()
    huge = _desc(num_blocks=1, block_size=16, num_kv_heads=8, max_blocks_per_seq=1 << 16,
                 num_seqs=64)
    assert lib.fp8kv_decode_workspace_bytes(ctypes.byref(huge), 64, 4, 1 << 20) > 64 << 20
    assert lib.fp8kv_decode_noalloc(ctypes.byref(huge), FAKE, 4, FAKE, 64, 1 << 20, 0.1,
                                    FAKE, None) == -5
    assert "scratch" in binding.strerror(-5)
    d = _desc(num_blocks=16, block_size=2048, max_blocks_per_seq=1)
    assert lib.fp8kv_decode_noalloc(ctypes.byref(d), FAKE, 17, FAKE, 16, 2048, 0.1, FAKE,
                                    None) == -4
    assert lib.fp8kv_decode_noalloc(ctypes.byref(d), FAKE, 8, FAKE, 17, 2048, 0.1, FAKE,
                                    None) == -1
    assert lib.fp8kv_decode_noalloc(ctypes.byref(d), FAKE, 8, FAKE, 0, 0, 0.1, FAKE,
                                    None) == 0    # empty batch: nothing to do


def test_pre_bias_cache_is_decode_only():
    lib = binding.lib()
    d = _desc(k_bias=FAKE)
    # prefill and narrow QK reject a cache with a K bias before any launch
    assert lib.fp8kv_prefill(ctypes.byref(d), FAKE, 8, FAKE, FAKE, FAKE, 1, 64, 64, 0.1,
                             FAKE, None) == -4
    assert lib.fp8kv_decode_q8(ctypes.byref(d), FAKE, 8, FAKE, 4, 64, 0.1, FAKE, FAKE,
                               10 ** 9, None) == -4
    # decode validates it like any cache (workspace check reached)
    assert lib.fp8kv_decode(ctypes.byref(d), FAKE, 8, FAKE, 4, 64, 0.1, FAKE, None, 0,
                            None) == -2


def test_prefill_rejects_bad_arguments():
    lib = binding.lib()
    d = _desc()
    assert lib.fp8kv_prefill(ctypes.byref(d), FAKE, 17, FAKE, FAKE, FAKE, 1, 64, 64, 0.1,
                             FAKE, None) == -4
    assert lib.fp8kv_prefill(ctypes.byref(d), None, 8, FAKE, FAKE, FAKE, 1, 64, 64, 0.1,
                             FAKE, None) == -1
    assert lib.fp8kv_prefill(ctypes.byref(d), FAKE, 8, FAKE, FAKE, FAKE, 1, -1, 64, 0.1,
                             FAKE, None) == -1
    assert lib.fp8kv_prefill(ctypes.byref(d), FAKE, 8, FAKE, FAKE, FAKE, 17, 64, 64, 0.1,
                             FAKE, None) == -1   # batch > table rows
    assert lib.fp8kv_prefill(ctypes.byref(d), FAKE, 8, FAKE, FAKE, FAKE, 0, 64, 64, 0.1,
                             FAKE, None) == 0


def _max_blocks_spanned(chunk, bs):
    """Brute force: most block-table entries a split touches (its keys
    [s*chunk, (s+1)*chunk) in 16-key sub-blocks); the start offsets into a
    block repeat after bs splits, so those cover every case."""
    return max((s * chunk + chunk - 16) // bs - (s * chunk) // bs + 1 for s in range(bs))


def test_split_window_rule_matches_brute_force():
    """Every (block_size, chunk) whose splits can touch more than 64 blocks is
    rejected, and every plan the library chooses touches at most 64."""
    lib = binding.lib()
    for bs in range(16, 1025, 16):
        for chunk in range(64, 64 * bs + 1, 64):
            if _max_blocks_spanned(chunk, bs) <= 64:
                continue
            d = _desc(num_blocks=16, block_size=bs, max_blocks_per_seq=4096)
            st = lib.fp8kv_decode_partial(ctypes.byref(d), FAKE, 8, FAKE, 16, chunk, 0.1,
                                          chunk, 1, FAKE, FAKE, None)
            assert st == -1, (bs, chunk)
        d = _desc(num_blocks=16, block_size=bs, num_kv_heads=8,
                  max_blocks_per_seq=(1 << 20) // bs, num_seqs=64)
        for L in (1, 300, 5000, (1 << 20) // bs * bs):
            r, c, s = _plan(d, 64, 4, L)
            assert r == 0 and _max_blocks_spanned(c, bs) <= 64, (bs, L, c)


def test_dequantize_rejects_bad_arguments():
    lib = binding.lib()
    src = _desc()                                              # K8V8
    good = _desc(mode=2, k=FAKE + 4096, v=FAKE + 8192, k_scale=None, v_scale=None)
    not_bf16 = _desc(mode=1, k=FAKE + 4096, v=FAKE + 8192, k_scale=None)
    other_shape = _desc(mode=2, k=FAKE + 4096, v=FAKE + 8192, k_scale=None, v_scale=None,
                        num_blocks=5)
    in_place = _desc(mode=2, k_scale=None, v_scale=None)
    other_layout = _desc(mode=2, k=FAKE + 4096, v=FAKE + 8192, k_scale=None, v_scale=None,
                         layout=1)
    for dst in (not_bf16, other_shape, in_place, other_layout):
        assert lib.fp8kv_dequantize(ctypes.byref(src), ctypes.byref(dst), None) == -1
    assert lib.fp8kv_dequantize(None, ctypes.byref(good), None) == -1
    assert lib.fp8kv_dequantize(ctypes.byref(src), None, None) == -1
