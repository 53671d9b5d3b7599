"""GPU parity of fp8kv_append against the oracle: codes and scales bit-exact.

Covers every mode and head dim, paged caches with shuffled block tables,
rows of extreme and subnormal magnitude, zero rows and signed zeros, the
hand-derived fixtures, and an exhaustive sweep of every fp32 in [-448, 448]
through the real append (rows whose amax is 448 have scale exactly 1, so the
stored code is the plain e4m3 encoding of each value).
"""
import ctypes
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import oracle
from fp8_kv_cache_append_amd import binding, synth
from fp8_kv_cache_append_amd.binding import KVCache
from golden_io import e4m3_encode_cases, quantize_cases
from gpu_util import append_seq, make_cache, read_rows

pytestmark = pytest.mark.gpu


def _extreme_rows(seed, n, hkv, d):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((n, hkv, d)).astype(np.float32)
    mag = np.exp(rng.uniform(np.log(1e-38), np.log(1e30), size=(n, hkv, 1)))
    x = (x * mag).astype(np.float32)
    x[0] = 0.0
    x[1, :, ::3] = -0.0
    x[2] *= np.float32(1e-40)
    x[3] = np.float32(2.0 ** -149) * np.arange(d, dtype=np.float32)
    x[4, :, 5] = np.float32(3e38)
    return x


def _expect(mode, k, v):
    return oracle.store_rows(mode, k, v)


def _assert_rows_equal(got, want, ctx):
    assert set(got) == set(want), ctx
    for key in want:
        g, w = got[key], want[key]
        if key in ("ks", "vs"):
            assert np.array_equal(g.view(np.uint32), w.view(np.uint32)), (ctx, key)
        else:
            assert np.array_equal(g, w), (ctx, key, np.argwhere(g != w)[:5])


@pytest.mark.parametrize("layout", ["token", "head"])
@pytest.mark.parametrize("mode", ["K8V8", "K16V8", "BF16", "K8V16"])
@pytest.mark.parametrize("d,hkv,bs", [(128, 2, 16), (64, 4, 32), (128, 8, 0)])
def test_append_bit_exact(mode, d, hkv, bs, layout):
    lens = np.array([37, 160, 1, 64], np.int32)
    w = synth.Workload("t", 4, hkv, hkv, d, lens, block_size=bs, shuffle_blocks=True, seed=3)
    cache = make_cache(mode, w, layout=layout)
    rows = {}
    for b in range(w.batch):
        n = int(lens[b])
        if b == 1:
            k = _extreme_rows(10 + b, n, hkv, d)
            v = _extreme_rows(20 + b, n, hkv, d)
        else:
            k, v = synth.kv_sequence(synth.Workload("t", 4, hkv, hkv, d, lens, "outliers",
                                                    seed=b), b)
        rows[b] = (k, v)
        # append in two calls to exercise positions that do not start at 0
        h = n // 2
        append_seq(cache, b, k[:h], v[:h], 0)
        append_seq(cache, b, k[h:], v[h:], h)
    torch.cuda.synchronize()
    for b, (k, v) in rows.items():
        _assert_rows_equal(read_rows(cache, b, k.shape[0]), _expect(mode, k, v), (mode, b))


def test_append_leaves_other_slots_untouched():
    lens = np.array([20, 40], np.int32)
    w = synth.Workload("t", 2, 2, 2, 128, lens, block_size=16, shuffle_blocks=True, seed=4)
    cache = make_cache("K8V8", w, capacity=64)
    k, v = synth.kv_sequence(w, 1)
    append_seq(cache, 1, k[:10], v[:10], 5)
    torch.cuda.synchronize()
    table = cache.block_table.cpu().numpy()
    written = np.zeros(cache.k.shape[:2], bool)
    for t in range(5, 15):
        written[table[1, t // 16], t % 16] = True
    kk = cache.k.cpu().numpy()
    assert np.all(kk[~written] == 0)
    assert np.all(cache.k_scale.cpu().numpy()[~written] == 0)
    assert np.any(kk[written] != 0)


def test_append_golden_fixtures():
    # quantisation fixture rows, padded with zeros to D = 64 (amax unchanged)
    cases = quantize_cases()
    x = np.zeros((len(cases), 1, 64), np.float32)
    for i, c in enumerate(cases):
        x[i, 0, :4] = c["x"]
    w = synth.Workload("t", 1, 1, 1, 64, np.array([len(cases)], np.int32))
    cache = make_cache("K8V8", w)
    append_seq(cache, 0, x, x)
    got = read_rows(cache, 0, len(cases))
    for i, c in enumerate(cases):
        assert float(got["ks"][i, 0]) == c["scale"], c
        assert list(got["k8"][i, 0, :4]) == c["codes"], c
        assert list(got["v8"][i, 0, :4]) == c["codes"], c
    # encoding fixture: rows [448, value, 0, ...] have scale 1
    enc = e4m3_encode_cases()
    x = np.zeros((len(enc), 1, 64), np.float32)
    x[:, 0, 0] = 448.0
    x[:, 0, 1] = [e[0] for e in enc]
    w = synth.Workload("t", 1, 1, 1, 64, np.array([len(enc)], np.int32))
    cache = make_cache("K8V8", w)
    append_seq(cache, 0, x, x)
    got = read_rows(cache, 0, len(enc))
    for i, (val, code, why) in enumerate(enc):
        if abs(val) > 448:   # would become the row's amax: not a scale-1 row
            continue
        assert int(got["k8"][i, 0, 1]) == code, (val, why)


@pytest.mark.timeout(600)
def test_append_exhaustive_e4m3_encoding():
    """Every fp32 with |x| <= 448, both signs, through fp8kv_append."""
    d, per_row = 128, 127
    chunk = per_row * (1 << 17)
    top = int(np.array([448.0], np.float32).view(np.uint32)[0]) + 1
    n_rows = -(-chunk // per_row)
    w = synth.Workload("t", 1, 1, 1, d, np.array([n_rows], np.int32))
    cache = make_cache("K8V8", w)
    x = torch.zeros((n_rows, 1, d), dtype=torch.float32, device="cuda")
    x[:, 0, 0] = 448.0
    seq = torch.zeros(n_rows, dtype=torch.int32, device="cuda")
    pos = torch.arange(n_rows, dtype=torch.int32, device="cuda")
    from fp8_kv_cache_append_amd import binding

    def check(bits, codes):
        want = oracle.e4m3_encode(bits.view(np.float32))
        return int(np.count_nonzero(want != codes))

    bad, jobs = 0, []
    with ThreadPoolExecutor(max_workers=12) as pool:
        for sign in (0, 0x80000000):
            for lo in range(0, top, chunk):
                bits = np.arange(lo, min(lo + chunk, top), dtype=np.uint32) | np.uint32(sign)
                n = bits.size
                buf = np.zeros(n_rows * per_row, np.uint32)
                buf[:n] = bits
                xt = torch.from_numpy(buf.view(np.float32).reshape(n_rows, per_row)).to("cuda")
                x[:, 0, 1:] = xt
                binding.fp8kv_append(cache, x, x, seq, pos)
                codes = cache.k[0, :n_rows, 0, 1:].cpu().numpy().reshape(-1)[:n]
                assert np.all(cache.k_scale[0, :n_rows, 0].cpu().numpy() == 1.0)
                jobs.append(pool.submit(check, bits, codes))
                if len(jobs) > 24:
                    bad += sum(j.result() for j in jobs)
                    jobs = []
        bad += sum(j.result() for j in jobs)
    assert bad == 0


def test_append_bf16_rounding_sweep():
    """K16V8 K rows and BF16 rows: bf16 RNE of random and tie-heavy fp32."""
    rng = np.random.default_rng(8)
    n = 1 << 14
    bits = rng.integers(0, 2 ** 32, size=(n, 1, 128), dtype=np.uint64).astype(np.uint32)
    bits[: n // 2, :, ::2] = (bits[: n // 2, :, ::2] & np.uint32(0xFFFF0000)) | np.uint32(0x8000)
    x = bits.view(np.float32)
    x[~np.isfinite(x) | (np.abs(x) > 3.3e38)] = 1.0
    w = synth.Workload("t", 1, 1, 1, 128, np.array([n], np.int32))
    for mode in ("K16V8", "BF16", "K8V16"):
        cache = make_cache(mode, w)
        append_seq(cache, 0, x, x)
        got = read_rows(cache, 0, n)
        if mode != "K8V16":
            assert np.array_equal(got["k16"], oracle.bf16_round_f32(x))
        if mode != "K16V8":
            assert np.array_equal(got["v16"], oracle.bf16_round_f32(x))


def test_append_is_deterministic():
    lens = np.array([300, 77], np.int32)
    w = synth.Workload("t", 2, 8, 2, 128, lens, "outliers", block_size=16,
                       shuffle_blocks=True, seed=9)
    cache = make_cache("K8V8", w)
    k, v = synth.kv_sequence(w, 0)
    append_seq(cache, 0, k, v)
    ref = cache.k.clone(), cache.k_scale.clone()
    for _ in range(20):
        append_seq(cache, 0, k, v)
    assert torch.equal(cache.k, ref[0]) and torch.equal(cache.k_scale, ref[1])


@pytest.mark.parametrize("mode", ["K8V8", "K16V8", "MXK8V8"])
@pytest.mark.parametrize("d,hkv", [(128, 4), (64, 1)])
def test_append_bulk_bit_exact(mode, d, hkv):
    """A bulk append (more rows than the compute units hold threads at once:
    the kernel's several-rows-per-thread path) into a paged cache behind a
    shuffled table, with some tokens carrying out-of-range sequence or
    position indices: every valid row bit-exact with the oracle, the
    skipped rows' slots left untouched."""
    n_seq, per = 4, 5008 if hkv == 4 else 10000
    lens = np.full(n_seq, per, np.int32)
    w = synth.Workload("t", n_seq, hkv, hkv, d, lens, block_size=16, shuffle_blocks=True,
                       seed=9)
    cache = make_cache(mode, w)
    n_tok = n_seq * per
    assert 2 * n_tok * hkv * (d // 4) >= 256 * 2048   # the bulk path
    rng = np.random.default_rng(9)
    k = rng.standard_normal((n_tok, hkv, d)).astype(np.float32) * 3
    v = rng.standard_normal((n_tok, hkv, d)).astype(np.float32)
    seq = np.repeat(np.arange(n_seq, dtype=np.int32), per)
    pos = np.tile(np.arange(per, dtype=np.int32), n_seq)
    order = rng.permutation(n_tok)                       # tokens in any order
    seq, pos, k, v = seq[order], pos[order], k[order], v[order]
    bad = rng.choice(n_tok, 64, replace=False)           # skipped: out-of-range indices
    seq_dev, pos_dev = seq.copy(), pos.copy()
    seq_dev[bad[:32]] = n_seq + 7
    pos_dev[bad[32:]] = -3
    binding.fp8kv_append(cache, torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda(),
                         torch.from_numpy(seq_dev).cuda(), torch.from_numpy(pos_dev).cuda())
    torch.cuda.synchronize()
    skipped = np.zeros(n_tok, bool)
    skipped[bad] = True
    for b in range(n_seq):
        mine = np.flatnonzero((seq == b) & ~skipped)
        want = _expect(mode, k[mine][np.argsort(pos[mine])], v[mine][np.argsort(pos[mine])])
        got = read_rows(cache, b, per)
        kept = np.sort(pos[mine])
        for key in want:
            g = got[key][kept]
            wv = want[key]
            if key in ("ks", "vs"):
                assert np.array_equal(g.view(np.uint32), wv.view(np.uint32)), (mode, b, key)
            else:
                assert np.array_equal(g, wv), (mode, b, key)
        lost = np.setdiff1d(np.arange(per), kept)        # slots of skipped tokens: untouched
        for key, a in got.items():
            assert not np.any(a[lost]), (mode, b, key, "skipped slot written")


def _near_midpoint_rows(seed, d):
    """Rows [amax, values...] whose values divided by the row's scale
    (fp32(amax / 448)) land within a few fp32 ulp of an e4m3 rounding
    midpoint -- every midpoint of the normal binades 2^-6 .. 2^8 and of the
    subnormal range -- for many non-power-of-two scales."""
    rng = np.random.default_rng(seed)
    mids = [(1 + (2 * j + 1) / 16) * 2.0 ** e for e in range(-6, 9) for j in range(8)]
    mids += [(2 * j + 1) * 2.0 ** -10 for j in range(8)]
    mids = np.array([m for m in mids if m < 448], np.float64)
    rows = []
    for amax in rng.uniform(0.5, 1000, 40).astype(np.float32):
        scale = np.float32(amax / np.float32(448))
        base = (mids * np.float64(scale)).astype(np.float32)
        vals = np.concatenate([(base.view(np.int32) + k).view(np.float32) for k in range(-6, 7)])
        vals *= np.where(rng.random(vals.size) < 0.5, -1, 1).astype(np.float32)
        n_row = -(-vals.size // (d - 1))
        vals = np.concatenate([vals, np.zeros(n_row * (d - 1) - vals.size, np.float32)])
        block = np.concatenate([np.full((n_row, 1), amax, np.float32),
                                vals.reshape(n_row, d - 1)], axis=1)
        rows.append(block)
    return np.concatenate(rows)


@pytest.mark.parametrize("mode", ["K8V8", "K16V8"])
@pytest.mark.parametrize("n_tok", [64, 1200])   # one row per thread / the bulk path
def test_append_near_midpoint_quotients(mode, n_tok):
    """The append kernel divides by a reciprocal where that cannot change a
    code and exactly where it can: quotients next to e4m3 midpoints must
    still give the correctly rounded codes (bit-exact with the oracle)."""
    d, hkv = 128, 8
    base = _near_midpoint_rows(31, d)
    rng = np.random.default_rng(32)
    k = base[rng.integers(0, base.shape[0], n_tok * hkv)].reshape(n_tok, hkv, d)
    v = base[rng.integers(0, base.shape[0], n_tok * hkv)].reshape(n_tok, hkv, d)
    if n_tok * hkv >= base.shape[0]:   # every constructed row at least once
        k.reshape(-1, d)[:base.shape[0]] = base
    lens = np.array([n_tok], np.int32)
    w = synth.Workload("t", 1, hkv, hkv, d, lens, block_size=16, shuffle_blocks=True, seed=5)
    cache = make_cache(mode, w)
    append_seq(cache, 0, k, v)
    torch.cuda.synchronize()
    _assert_rows_equal(read_rows(cache, 0, n_tok), _expect(mode, k, v), (mode, n_tok))


def _cache_tensors(cache):
    return [t.clone() for t in (cache.k, cache.v, cache.k_scale, cache.v_scale, cache.k_exp)
            if t is not None]


@pytest.mark.parametrize("layout", ["token", "head"])
@pytest.mark.parametrize("mode", ["K8V8", "K16V8", "MXK8V8"])
@pytest.mark.parametrize("n_tok", [40, 1100])   # one row per thread / the bulk path
def test_append_64bit_row_indices(mode, layout, n_tok):
    """A cache of 2^31 rows or more takes the kernel's 64-bit row arithmetic
    (smaller ones a 32-bit row index).  The same rows are appended twice into
    two copies of a small cache: once through its own descriptor, once through
    a descriptor that declares 2^28 blocks (2^35 rows) while its block table
    still names only blocks the copy holds, so every access stays inside the
    allocation.  Both copies must hold the same bytes."""
    hkv, d, bs = 8, 128, 16
    lens = np.array([n_tok], np.int32)
    w = synth.Workload("t", 1, hkv, hkv, d, lens, block_size=bs, shuffle_blocks=True, seed=21)
    small, large = make_cache(mode, w, layout=layout), make_cache(mode, w, layout=layout)
    assert torch.equal(small.block_table, large.block_table)
    rng = np.random.default_rng(21)
    k = torch.from_numpy(rng.standard_normal((n_tok, hkv, d)).astype(np.float32) * 3).cuda()
    v = torch.from_numpy(rng.standard_normal((n_tok, hkv, d)).astype(np.float32)).cuda()
    seq = torch.zeros(n_tok, dtype=torch.int32, device="cuda")
    pos = torch.from_numpy(rng.permutation(n_tok).astype(np.int32)).cuda()
    binding.fp8kv_append(small, k, v, seq, pos)
    desc = large.desc()
    assert desc.num_blocks * bs * hkv < 2 ** 31
    desc.num_blocks = 2 ** 28
    st = binding.lib().fp8kv_append(ctypes.byref(desc), binding._ptr(k), binding._ptr(v),
                                    binding._ptr(seq), binding._ptr(pos), n_tok, None)
    assert st == 0, binding.lib().fp8kv_strerror(st)
    torch.cuda.synchronize()
    for a, b in zip(_cache_tensors(small), _cache_tensors(large)):
        assert torch.equal(a, b), (mode, layout, n_tok)
    assert torch.count_nonzero(small.k) > 0
