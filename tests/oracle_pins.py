"""Checks that pin the fp64 oracle to something other than itself.

Each ``pin_*`` function raises AssertionError when the oracle disagrees with a
brute-force computation, a closed form, an invariant or a figure printed on the
pages.  ``test_oracle.py`` runs them as tests, and also runs them against
deliberately broken copies of the oracle (on the CPU) to show that each planted
mistake is caught by at least one pin.
"""
from __future__ import annotations

import math
import struct

import numpy as np

import oracle
import synth
from tests.golden.read import load as load_golden


# ---------------------------------------------------------------------------- helpers

def _bf16_to_float(bits: int) -> float:
    """Independent bf16 decode: the 16 bits are the top half of a big-endian binary32."""
    return struct.unpack(">f", struct.pack(">I", (int(bits) & 0xFFFF) << 16))[0]


def _f16_to_float(bits: int) -> float:
    """Independent binary16 decode through the struct module's half-precision format."""
    return struct.unpack("<e", struct.pack("<H", int(bits) & 0xFFFF))[0]


def _e4m3_to_float(bits: int) -> float:
    """Independent OCP E4M3 decode, one code at a time (sign, 4-bit exponent with bias
    7, 3-bit mantissa; exponent 0 is subnormal; S.1111.111 is NaN)."""
    b = int(bits) & 0xFF
    if b & 0x7F == 0x7F:
        return math.nan
    sign = -1.0 if b >> 7 else 1.0
    e, m = (b >> 3) & 15, b & 7
    if e == 0:
        return sign * math.ldexp(m, -9)
    return sign * math.ldexp(8 + m, e - 10)


def _f32_to_float(bits: int) -> float:
    return struct.unpack("<f", struct.pack("<I", int(bits) & 0xFFFFFFFF))[0]


_ELEMENT = {"bf16": _bf16_to_float, "f16": _f16_to_float, "fp8_e4m3": _e4m3_to_float,
            "f32": _f32_to_float}


def brute_force_rows(wl) -> np.ndarray:
    """Multi-row window by brute force: row i is single-row decode of length L - n + 1 + i,
    evaluated by brute_force_decode on a copy whose lengths are cut to that value."""
    import copy
    n = wl.num_rows
    out = np.zeros((wl.batch, n, wl.num_q_heads, wl.head_dim))
    for i in range(n):
        one = copy.copy(wl)
        one.num_rows = 1
        one.q = np.ascontiguousarray(wl.q[:, i])
        one.seq_lens = (wl.seq_lens - n + 1 + i).astype(np.int32)
        out[:, i] = brute_force_decode(one)
    return out


def brute_force_decode(wl) -> np.ndarray:
    """Pure-Python decode attention: explicit flat indexing, exp without max shift, fsum.

    Element (page p, KV head g, slot s, column c) sits at flat index
    p*page_stride + g*head_stride + s*row_stride + c.  Scores are kept small by the
    callers, so exp(s) / sum exp(s) is evaluated literally.
    """
    D, G = wl.head_dim, wl.num_q_heads // wl.num_kv_heads
    out = np.zeros((wl.batch, wl.num_q_heads, D))
    pool = wl.pool
    elem = _ELEMENT[wl.kv_dtype]
    ks, vs = wl.k_scale, wl.v_scale
    for r in range(wl.batch):
        L = int(wl.seq_lens[r])
        lo = L - wl.window if (wl.window and L > wl.window) else 0
        for g in range(wl.num_kv_heads):
            keys, vals = [], []
            for j in range(lo, L):
                p = int(wl.table[r][j // wl.page_size])
                base = p * wl.page_stride + g * wl.head_stride + (j % wl.page_size) * wl.row_stride
                row = [elem(pool[base + c]) for c in range(wl.row_cols)]
                v = [x * vs for x in row[wl.v_offset:wl.v_offset + D]]
                if wl.fmt == "split":
                    k = [x * ks for x in row[wl.k_offset:wl.k_offset + D]]
                else:
                    k = [x * ks for x in row[wl.k_offset:wl.k_offset + wl.rot_cols]] + v[wl.rot_cols:]
                keys.append(k)
                vals.append(v)
            for h in range(g * G, (g + 1) * G):
                qh = [float(x) for x in wl.q[r, h]]
                w = [math.exp(wl.scale * math.fsum(qh[d] * k[d] for d in range(D))) for k in keys]
                Z = math.fsum(w)
                out[r, h] = [math.fsum(w[j] * vals[j][d] for j in range(len(w))) / Z for d in range(D)]
    return out


def _assert_close(a, b, tol, what):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    err = float(np.max(np.abs(a - b))) if a.size else 0.0
    scale = max(1.0, float(np.max(np.abs(b)))) if b.size else 1.0
    assert err <= tol * scale, f"{what}: max|diff| = {err:.3e} > {tol:.1e} x {scale:.3g}"


def _rng(seed):
    return np.random.default_rng(seed)


# ---------------------------------------------------------------------------- pins

BRUTE_CASES = [
    # (seq_lens, Hq, Hkv, D, page_size, window, fmt, layout)
    ([1, 5, 16], 4, 2, 17, 4, 0, "split", synth.HEAD_MAJOR),
    ([3, 16], 6, 3, 1, 8, 0, "split", synth.TOKEN_MAJOR),
    ([16, 7], 16, 2, 512, 4, 0, "split", synth.HEAD_MAJOR),
    ([14, 9, 1], 8, 1, 512, 4, 0, "folded", synth.TOKEN_MAJOR),
    ([16, 11, 4, 2], 4, 4, 17, 4, 5, "split", synth.HEAD_MAJOR),
]

# Other stored element types: (kv_dtype, seq_lens, Hq, Hkv, D, page_size, window, fmt, layout)
DTYPE_CASES = [
    ("fp8_e4m3", [16, 7], 16, 2, 512, 4, 0, "split", synth.HEAD_MAJOR),
    ("fp8_e4m3", [14, 9], 8, 1, 512, 4, 0, "folded", synth.TOKEN_MAJOR),
    ("fp8_e4m3", [16, 11, 4], 4, 4, 17, 4, 5, "split", synth.TOKEN_MAJOR),
    ("f16", [12, 5], 8, 2, 64, 4, 0, "split", synth.HEAD_MAJOR),
    ("f16", [9], 8, 1, 512, 4, 0, "folded", synth.HEAD_MAJOR),
    ("f32", [13, 3], 4, 2, 33, 4, 6, "split", synth.TOKEN_MAJOR),
]


def pin_brute_force():
    """Dense fp64 oracle == literal pure-Python softmax on tiny paged inputs."""
    for i, (lens, hq, hkv, D, ps, W, fmt, layout) in enumerate(BRUTE_CASES):
        wl = synth.make_workload(lens, num_q_heads=hq, num_kv_heads=hkv, head_dim=D, page_size=ps,
                                 window=W, fmt=fmt, rot_cols=128, seed=10 + i, layout=layout,
                                 spare_pages=3, pad="big")
        _assert_close(oracle.decode_attention(wl), brute_force_decode(wl), 1e-13, f"brute case {i}")


def pin_dtype_brute_force():
    """f16, FP8 E4M3 (with K and V dequantisation factors) and f32 pools: the fp64
    oracle == literal pure-Python decode with its own per-element decoders."""
    for i, (dt, lens, hq, hkv, D, ps, W, fmt, layout) in enumerate(DTYPE_CASES):
        wl = synth.make_workload(lens, num_q_heads=hq, num_kv_heads=hkv, head_dim=D, page_size=ps,
                                 window=W, fmt=fmt, rot_cols=128, seed=40 + i, layout=layout,
                                 spare_pages=2, pad="nan", kv_dtype=dt)
        assert wl.pool.dtype.itemsize == synth.KV_BYTES[dt]
        _assert_close(oracle.decode_attention(wl), brute_force_decode(wl), 1e-13,
                      f"dtype case {i} ({dt} {fmt})")


def pin_e4m3_codes():
    """All 256 E4M3 codes: the oracle's decode == torch's float8_e4m3fn widening, the
    per-code decoder above, and the closed forms of the encoding (largest finite 448,
    smallest subnormal 2^-9, smallest normal 2^-6, 1.0 = 0x38, two NaN codes, -0)."""
    import torch
    codes = np.arange(256, dtype=np.uint8)
    got = oracle.e4m3_bits_to_f64(codes)
    ref = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    fin = ~np.isnan(ref)
    assert np.array_equal(got[fin], ref[fin])
    assert np.array_equal(np.signbit(got[fin]), np.signbit(ref[fin]))
    mine = np.array([_e4m3_to_float(c) for c in range(256)])
    assert np.array_equal(got[fin], mine[fin]) and np.isnan(mine[~fin]).all()
    assert got[0x7E] == 448.0 and got[0xFE] == -448.0
    assert got[0x01] == 2.0 ** -9 and got[0x08] == 2.0 ** -6 and got[0x07] == 7 * 2.0 ** -9
    assert got[0x38] == 1.0 and got[0xB8] == -1.0 and got[0x39] == 1.125
    assert np.flatnonzero(np.isnan(got)).tolist() == [0x7F, 0xFF]
    assert got[0x80] == 0.0 and np.signbit(got[0x80])
    pos = got[:0x7F]
    assert np.all(np.diff(pos) > 0), "positive codes must increase strictly"


def pin_f16_f32_codes():
    """Every binary16 pattern widens as torch's float16 does (and closed forms); binary32
    closed forms."""
    import torch
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = oracle.f16_bits_to_f64(bits)
    ref = torch.from_numpy(bits.view(np.int16).copy()).view(torch.float16).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan) and np.array_equal(got[~nan], ref[~nan])
    assert got[0x3C00] == 1.0 and got[0x0001] == 2.0 ** -24 and got[0x7BFF] == 65504.0
    assert got[0x7C00] == math.inf and got[0xFC00] == -math.inf and got[0x0400] == 2.0 ** -14
    f = oracle.f32_bits_to_f64(np.array([0x3F800000, 0x00000001, 0x7F7FFFFF, 0xC0490FDB],
                                        dtype=np.uint32))
    assert f[0] == 1.0 and f[1] == 2.0 ** -149 and f[2] == (2 - 2.0 ** -23) * 2.0 ** 127
    assert f[3] == -3.1415927410125732


def pin_dequant_factors():
    """K's factor acts as a factor on the softmax scale, V's as a factor on the output:
    decode(k_scale = a, v_scale = b) == b * decode(k_scale = 1, v_scale = 1, scale * a)."""
    import copy
    for fmt in ("split", "folded"):
        D = 512 if fmt == "folded" else 64
        wl = synth.make_workload([37, 20], num_q_heads=8, num_kv_heads=2, head_dim=D, page_size=8,
                                 fmt=fmt, seed=44, kv_dtype="fp8_e4m3", pad="big")
        got = oracle.decode_attention(wl)
        one = copy.copy(wl)
        one.v_scale = 1.0
        if fmt == "split":
            one.k_scale = 1.0
            one.scale = wl.scale * wl.k_scale
        else:
            # folded: the query's rotated part meets K columns, the rest meets V columns
            one.k_scale = 1.0
            q = wl.q.astype(np.float64).copy()
            q[..., :128] *= wl.k_scale
            q[..., 128:] *= wl.v_scale
            one.q = q
        ref = wl.v_scale * oracle.decode_attention(one)
        _assert_close(got, ref, 1e-13, f"dequantisation factors ({fmt})")
        assert not np.allclose(got, oracle.decode_attention(copy.copy(one)), atol=1e-3)


def pin_single_key():
    """L = 1: softmax of one score is exactly 1, so o = v_0 bit for bit."""
    for fmt in ("split", "folded"):
        wl = synth.make_workload([1], num_q_heads=8, num_kv_heads=1, head_dim=512, page_size=256,
                                 fmt=fmt, seed=3)
        v0 = oracle.bf16_bits_to_f64(oracle.gather_rows(wl, 0, 0, np.array([0])))[0]
        v0 = v0[wl.v_offset:wl.v_offset + 512]
        o = oracle.decode_attention(wl)
        for h in range(8):
            assert np.array_equal(o[0, h], v0), "L=1 output is not v_0"


def pin_uniform_scores():
    """q = 0 (all scores equal) or identical keys: o is the plain mean of V."""
    wl = synth.make_workload([37], num_q_heads=4, num_kv_heads=2, head_dim=64, page_size=16, seed=4)
    wl.q[:] = 0.0
    pos = np.arange(37)
    o = oracle.decode_attention(wl)
    for g in range(2):
        V = oracle.bf16_bits_to_f64(oracle.gather_rows(wl, 0, g, pos))[:, 64:128]
        for h in (2 * g, 2 * g + 1):
            _assert_close(o[0, h], V.mean(axis=0), 1e-14, "q=0 mean")
    # identical keys, arbitrary q
    D = 32
    K = np.tile(_rng(5).standard_normal(D), (9, 1))
    V = _rng(6).standard_normal((9, D))
    q = _rng(7).standard_normal((3, D))
    _assert_close(oracle.dense_attention(q, K, V, 0.3), np.tile(V.mean(axis=0), (3, 1)), 1e-14,
                  "identical keys mean")


def pin_two_keys():
    """Two keys: o = sigma(s1 - s2) v1 + sigma(s2 - s1) v2."""
    rng = _rng(8)
    for _ in range(20):
        D = int(rng.integers(1, 40))
        K = rng.standard_normal((2, D)) * 3
        V = rng.standard_normal((2, D))
        q = rng.standard_normal((1, D))
        scale = float(rng.uniform(0.1, 2))
        s1, s2 = scale * float(q[0] @ K[0]), scale * float(q[0] @ K[1])
        w1 = 1.0 / (1.0 + math.exp(s2 - s1))
        expect = w1 * V[0] + (1.0 - w1) * V[1]
        _assert_close(oracle.dense_attention(q, K, V, scale)[0], expect, 1e-14, "two keys")


def pin_needle():
    """One key scoring 40 above every other: o = v_needle to within L e^-40."""
    rng = _rng(9)
    n, D = 300, 48
    q = rng.standard_normal(D)
    K = rng.standard_normal((n, D)) * 0.01
    K[123] = q / np.dot(q, q) * 45.0          # score 45 against at most ~1 for the rest
    V = rng.standard_normal((n, D))
    o = oracle.dense_attention(q[None], K, V, 1.0)[0]
    _assert_close(o, V[123], n * math.exp(-40.0), "needle")


def pin_gqa_grouping():
    """Eight query heads per KV head, consecutive: head h reads KV head h // G.

    Every V row of KV head g is the constant g + 1, so o[h] = h // G + 1 (to rounding).
    """
    wl = synth.make_workload([40], num_q_heads=32, num_kv_heads=4, head_dim=16, page_size=8,
                             seed=11)
    rows = wl.pool.reshape(wl.num_pages, 4, 8, 32)
    for g in range(4):
        rows[:, g, :, 16:] = synth.f32_to_bf16_bits(np.float32(g + 1))
    o = oracle.decode_attention(wl)
    for h in range(32):
        assert np.max(np.abs(o[0, h] - (h // 8 + 1))) < 1e-13, f"head {h} did not read KV head {h // 8}"


def pin_linearity_and_order():
    """o is linear in V, invariant to reordering the keys, and to (q, scale) -> (cq, scale/c)."""
    rng = _rng(12)
    n, D = 50, 24
    q = rng.standard_normal((3, D))
    K = rng.standard_normal((n, D))
    V1 = rng.standard_normal((n, D))
    V2 = rng.standard_normal((n, D))
    f = oracle.dense_attention
    _assert_close(f(q, K, V1 + 2 * V2, 0.4), f(q, K, V1, 0.4) + 2 * f(q, K, V2, 0.4), 1e-13, "linear")
    p = rng.permutation(n)
    _assert_close(f(q, K[p], V1[p], 0.4), f(q, K, V1, 0.4), 1e-13, "key order")
    _assert_close(f(4 * q, K, V1, 0.1), f(q, K, V1, 0.4), 1e-13, "scale")


def _split_cuts(n, ways):
    """Equal-as-possible cut points; more ways than tokens gives empty partitions."""
    return [(i * n) // ways for i in range(ways + 1)]


def pin_partition_invariance():
    """Split-KV partials merged in two levels == dense, for 1/2/3/4/7/16-way splits of the
    13 x 17 fixture (16-way has empty partitions), random cuts at D=512, L=1024."""
    fx = load_golden("partition_fixture.txt")
    n, D = fx["tokens"], fx["dims"]
    rng = _rng(13)
    q = rng.standard_normal(D)
    K = rng.standard_normal((n, D))
    V = rng.standard_normal((n, D))
    dense = oracle.dense_attention(q[None], K, V, 0.5)[0]
    for ways in fx["ways"]:
        cuts = _split_cuts(n, ways)
        if ways > n:
            assert any(a == b for a, b in zip(cuts[:-1], cuts[1:])), "no empty partition"
        for group in (1, 2, 3, ways):
            got = oracle.split_kv_attention(q, K, V, 0.5, cuts, group)
            _assert_close(got, dense, 1e-13, f"{ways}-way, group {group}")
    n, D = 1024, 512
    q = rng.standard_normal(D)
    K = rng.standard_normal((n, D))
    V = rng.standard_normal((n, D))
    dense = oracle.dense_attention(q[None], K, V, 1 / math.sqrt(D))[0]
    for _ in range(5):
        inner = np.sort(rng.integers(0, n + 1, size=int(rng.integers(1, 40))))
        cuts = [0] + inner.tolist() + [n]
        got = oracle.split_kv_attention(q, K, V, 1 / math.sqrt(D), cuts, int(rng.integers(1, 9)))
        _assert_close(got, dense, 1e-13, "random cuts")


def pin_empty_merge_identity():
    """merge(a, empty) and merge(empty, a) are a bit for bit (alpha = e^0 = 1, beta = 0)."""
    rng = _rng(14)
    D = 33
    a = oracle.partial_state(rng.standard_normal(D), rng.standard_normal((7, D)),
                             rng.standard_normal((7, D)), 0.7)
    e = oracle.empty_state(D)
    for m in (oracle.merge(a, e), oracle.merge(e, a)):
        assert m.m == a.m and m.l == a.l and np.array_equal(m.acc, a.acc), "empty merge changed a"
    ee = oracle.merge(e, e)
    assert ee.m == -math.inf and ee.l == 0.0 and not np.any(ee.acc)


def pin_merge_identity_values():
    """merge(partial(A), partial(B)) == partial(A u B) for the state itself, not just O/S."""
    rng = _rng(15)
    D = 20
    q = rng.standard_normal(D)
    K = rng.standard_normal((30, D)) * 2
    V = rng.standard_normal((30, D))
    whole = oracle.partial_state(q, K, V, 0.9)
    m = oracle.merge(oracle.partial_state(q, K[:11], V[:11], 0.9),
                     oracle.partial_state(q, K[11:], V[11:], 0.9))
    assert m.m == whole.m
    _assert_close(m.l, whole.l, 1e-14, "merged S")
    _assert_close(m.acc, whole.acc, 1e-14, "merged O")


def pin_gem_audit_bounds(lengths=None):
    """At gem's audit lengths with P = 32, DV = 512, the split path stays inside the bounds
    the page prints against direct softmax (upper bounds: fp64 should be far below)."""
    gold = load_golden("gem_online_merge_audit.txt")
    P, D = gold["partitions"], gold["value_dim"]
    rng = _rng(16)
    for n in (lengths or gold["lengths"]):
        K = rng.standard_normal((n, D)).astype(np.float32).astype(np.float64)
        V = rng.standard_normal((n, D)).astype(np.float32).astype(np.float64)
        q = rng.standard_normal(D).astype(np.float32).astype(np.float64)
        dense = oracle.dense_attention(q[None], K, V, 1 / math.sqrt(D))[0]
        got = oracle.split_kv_attention(q, K, V, 1 / math.sqrt(D), _split_cuts(n, P), 8)
        err = got - dense
        nmse = float(np.sum(err ** 2) / np.sum(dense ** 2))
        corr = float(np.corrcoef(got, dense)[0, 1])
        assert np.all(np.isfinite(got))
        assert float(np.max(np.abs(err))) < gold["max_abs_max"], f"max|diff| at {n}"
        assert nmse <= gold["nmse_max"], f"NMSE at {n}"
        assert corr >= gold["corr_min"], f"corr at {n}"
        # repeat determinism
        again = oracle.split_kv_attention(q, K, V, 1 / math.sqrt(D), _split_cuts(n, P), 8)
        assert np.array_equal(got, again)


def pin_window():
    """Windowed decode == dense attention over the sliced in-window keys, for L around W;
    the pad in masked slots (older keys of resident pages) does not change a bit."""
    W = 64
    for L in (1, W - 1, W, W + 1, W + 16, W + 64, 3 * W + 5):
        outs = {}
        for pad in ("nan", "big", "zero"):
            wl = synth.make_workload([L], num_q_heads=4, num_kv_heads=2, head_dim=32, page_size=16,
                                     window=W, seed=17, pad=pad)
            outs[pad] = oracle.decode_attention(wl)
        assert np.array_equal(outs["nan"], outs["big"]) and np.array_equal(outs["nan"], outs["zero"])
        lo = max(0, L - W)
        for g in range(2):
            rows = oracle.bf16_bits_to_f64(oracle.gather_rows(wl, 0, g, np.arange(lo, L)))
            K, V = rows[:, :32], rows[:, 32:]
            assert K.shape[0] == min(L, W)
            ref = oracle.dense_attention(wl.q[0, 2 * g:2 * g + 2], K, V, wl.scale)
            _assert_close(outs["zero"][0, 2 * g:2 * g + 2], ref, 1e-15, f"window L={L}")


def pin_permutation_invariance():
    """Any page-table permutation (data moved with it) and either pool layout: same bits."""
    base = synth.make_workload([300, 77], num_q_heads=8, num_kv_heads=2, head_dim=64, page_size=32,
                               seed=18, table_seed=1)
    ref = oracle.decode_attention(base)
    for ts, layout in ((2, synth.HEAD_MAJOR), (3, synth.TOKEN_MAJOR), (1, synth.TOKEN_MAJOR)):
        wl = synth.make_workload([300, 77], num_q_heads=8, num_kv_heads=2, head_dim=64, page_size=32,
                                 seed=18, table_seed=ts, layout=layout)
        if ts != 1:
            assert not np.array_equal(wl.table, base.table)
        assert np.array_equal(oracle.decode_attention(wl), ref), f"table seed {ts} {layout}"


def pin_folded_equals_split():
    """Folded row + folded query == split row with K[rot:] = w * V[rot:] (fp64, unrounded)."""
    wl = synth.make_workload([700], num_q_heads=8, num_kv_heads=1, head_dim=512, page_size=256,
                             fmt="folded", seed=19)
    # fold w into q in fp64 here, so the identity is exact (the fp32 fold rounds by 2^-24)
    q64 = wl.q_unfolded.astype(np.float64)
    q64[:, :, 128:] *= wl.fold_w.astype(np.float64)
    wl.q = q64
    o_fold = oracle.decode_attention(wl)
    rows = oracle.bf16_bits_to_f64(oracle.gather_rows(wl, 0, 0, np.arange(700)))
    krot, V = rows[:, :128], rows[:, 128:640]
    K = np.concatenate([krot, V[:, 128:] * wl.fold_w.astype(np.float64)], axis=1)
    o_split = oracle.dense_attention(wl.q_unfolded[0], K, V, wl.scale)
    _assert_close(o_fold[0], o_split, 1e-12, "folded vs split")


def pin_fail_closed():
    """States no finite key set can produce are refused, as is finalize of no keys."""
    D = 4
    good = oracle.State(0.5, 2.0, np.ones(D))
    bad = [
        oracle.State(math.nan, 1.0, np.zeros(D)),
        oracle.State(math.inf, 1.0, np.zeros(D)),
        oracle.State(-math.inf, 1.0, np.zeros(D)),
        oracle.State(-math.inf, 0.0, np.ones(D)),
        oracle.State(0.0, 0.5, np.zeros(D)),
        oracle.State(0.0, 2.0, np.array([1.0, math.nan, 0.0, 0.0])),
        oracle.State(0.0, math.inf, np.zeros(D)),
    ]
    for st in bad:
        for args in ((st, good), (good, st)):
            try:
                oracle.merge(*args)
            except oracle.InvalidState:
                continue
            raise AssertionError(f"merge accepted invalid state {st}")
        try:
            oracle.finalize(st)
        except oracle.InvalidState:
            pass
        else:
            raise AssertionError(f"finalize accepted invalid state {st}")
    try:
        oracle.finalize(oracle.empty_state(D))
    except oracle.InvalidState:
        pass
    else:
        raise AssertionError("finalize of the empty state returned")


def pin_query_rows():
    """A window of n query rows: row i is ordinary decode at length L - n + 1 + i (brute
    force per row), the last row is the single-row decode of the whole context, and the
    first row of an n-row window over L keys equals the last row of a window over
    L - n + 1 keys.  Whole context and sliding window."""
    for W, fmt in ((0, "split"), (6, "split"), (0, "folded")):
        D = 17 if fmt == "split" else 512
        wl = synth.make_workload([9, 4, 16], num_q_heads=4, num_kv_heads=2, head_dim=D, page_size=4,
                                 window=W, fmt=fmt, seed=30, num_rows=4, pad="big", spare_pages=2)
        got = oracle.decode_attention(wl)
        assert got.shape == (3, 4, 4, D)
        _assert_close(got, brute_force_rows(wl), 1e-13, f"rows W={W} {fmt}")
    wl = synth.make_workload([40, 33], num_q_heads=8, num_kv_heads=1, head_dim=64, page_size=8,
                             seed=31, num_rows=5)
    rows = oracle.decode_attention(wl)
    import copy
    last = copy.copy(wl)
    last.num_rows = 1
    last.q = np.ascontiguousarray(wl.q[:, -1])
    assert np.array_equal(rows[:, -1], oracle.decode_attention(last))
    first = copy.copy(wl)
    first.num_rows = 1
    first.q = np.ascontiguousarray(wl.q[:, 0])
    first.seq_lens = (wl.seq_lens - 4).astype(np.int32)
    assert np.array_equal(rows[:, 0], oracle.decode_attention(first))


def brute_force_prefill(wl) -> np.ndarray:
    """Prefill by brute force: the packed row of request r at position p is single-row
    decode of length p + 1 over request r alone, evaluated by brute_force_decode."""
    import dataclasses
    out = np.zeros((wl.q.shape[0], wl.num_q_heads, wl.head_dim))
    t = 0
    for r in range(wl.batch):
        L, n = int(wl.seq_lens[r]), int(wl.q_lens[r])
        for i in range(n):
            one = dataclasses.replace(wl, batch=1, table=wl.table[r:r + 1],
                                      seq_lens=np.array([L - n + i + 1], dtype=np.int32),
                                      q=np.ascontiguousarray(wl.q[t][None]), q_lens=None,
                                      num_rows=1)
            out[t] = brute_force_decode(one)[0]
            t += 1
    return out


PREFILL_CASES = [
    # (seq_lens, q_lens, Hq, Hkv, D, page_size, window, fmt, layout, kv_dtype)
    # window crossing, ragged, continuation, a request with no new rows
    ([9, 4, 16, 5], [9, 2, 7, 0], 4, 2, 17, 4, 6, "split", synth.HEAD_MAJOR, "bf16"),
    # fresh prompt and a one-row continuation over the folded row
    ([12, 3], [12, 1], 8, 1, 512, 4, 0, "folded", synth.TOKEN_MAJOR, "bf16"),
    # tiny: one key, one row
    ([1], [1], 2, 1, 8, 4, 0, "split", synth.HEAD_MAJOR, "bf16"),
    # other element types with their dequantisation factors
    ([10, 6], [4, 6], 4, 2, 33, 4, 5, "split", synth.TOKEN_MAJOR, "fp8_e4m3"),
    ([7], [7], 4, 1, 512, 4, 0, "folded", synth.HEAD_MAJOR, "f16"),
]


def pin_prefill_brute_force():
    """Every prompt row against the pure-Python definition (causal, windowed, ragged,
    continuation, zero and one-row requests, split and folded rows, FP8 and f16)."""
    for k, (lens, ql, hq, hkv, D, ps, W, fmt, layout, dt) in enumerate(PREFILL_CASES):
        wl = synth.make_workload(lens, num_q_heads=hq, num_kv_heads=hkv, head_dim=D, page_size=ps,
                                 window=W, fmt=fmt, layout=layout, seed=90 + k, q_lens=ql,
                                 kv_dtype=dt, pad="nan", spare_pages=2)
        got = oracle.prefill_attention(wl)
        assert got.shape == (sum(ql), hq, D)
        _assert_close(got, brute_force_prefill(wl), 1e-13, f"prefill case {k}")


def pin_prefill_rows_are_decode():
    """A prompt row is decode at its own length: each packed row equals the (separately
    pinned) decode oracle on request r alone with length position + 1, bit for bit; the
    last row of a request equals decode over its whole context."""
    import dataclasses
    for W in (0, 12):
        wl = synth.make_workload([40, 33, 20], num_q_heads=8, num_kv_heads=2, head_dim=64,
                                 page_size=8, window=W, seed=95 + W, q_lens=[40, 5, 1])
        got = oracle.prefill_attention(wl)
        for t, (r, p) in enumerate(oracle.prefill_row_index(wl)):
            one = dataclasses.replace(wl, batch=1, table=wl.table[r:r + 1],
                                      seq_lens=np.array([p + 1], dtype=np.int32),
                                      q=np.ascontiguousarray(wl.q[t][None]), q_lens=None,
                                      num_rows=1)
            assert np.array_equal(got[t], oracle.decode_attention(one)[0]), (W, t)
        sel = oracle.prefill_attention(wl, rows=[39, 44, 45])
        assert np.array_equal(sel, got[[39, 44, 45]])


def pin_prefill_causality():
    """Rewriting the keys and values after a row's position leaves that row's output
    unchanged bit for bit and changes the later rows; the first row of a fresh prompt is
    v0 exactly."""
    wl = synth.make_workload([24], num_q_heads=4, num_kv_heads=1, head_dim=32, page_size=8,
                             seed=97, q_lens=[24])
    base = oracle.prefill_attention(wl)
    v0 = oracle.keys_values(wl, oracle.stored_to_f64(oracle.gather_rows(wl, 0, 0, [0])))[1][0]
    assert all(np.array_equal(base[0, h], v0) for h in range(4))
    p = 10
    other = synth.make_workload([24], num_q_heads=4, num_kv_heads=1, head_dim=32, page_size=8,
                                seed=98, q_lens=[24])
    pool = wl.pool.copy()
    for j in range(p + 1, 24):
        page, slot = int(wl.table[0][j // 8]), j % 8
        opage = int(other.table[0][j // 8])
        dst = page * wl.page_stride + slot * wl.row_stride
        src = opage * other.page_stride + slot * other.row_stride
        pool[dst:dst + wl.row_cols] = other.pool[src:src + other.row_cols]
    import dataclasses
    moved = oracle.prefill_attention(dataclasses.replace(wl, pool=pool))
    assert np.array_equal(moved[:p + 1], base[:p + 1])
    assert not np.array_equal(moved[p + 1:], base[p + 1:])


def brute_force_tree(wl) -> np.ndarray:
    """Tree attention by brute force: window row i sees the keys before the window that
    a causal row i sees, and the window rows on its path to the root, found by walking
    the parent indices (never the masks); pure-Python scores and sums."""
    D, G, n = wl.head_dim, wl.num_q_heads // wl.num_kv_heads, wl.num_rows
    out = np.zeros((wl.batch, n, wl.num_q_heads, D))
    elem = _ELEMENT[wl.kv_dtype]
    for r in range(wl.batch):
        L = int(wl.seq_lens[r])
        for i in range(n):
            path, j = set(), i
            while j >= 0:
                path.add(j)
                j = int(wl.tree_parents[r][j])
            here = L - n + i + 1                   # a causal row i's length
            lo = here - wl.window if (wl.window and here > wl.window) else 0
            positions = [t for t in range(lo, L) if t < L - n or (t - (L - n)) in path]
            for g in range(wl.num_kv_heads):
                keys, vals = [], []
                for t in positions:
                    pg = int(wl.table[r][t // wl.page_size])
                    base = pg * wl.page_stride + g * wl.head_stride + (t % wl.page_size) * wl.row_stride
                    row = [elem(wl.pool[base + c]) for c in range(wl.row_cols)]
                    v = row[wl.v_offset:wl.v_offset + D]
                    k = (row[wl.k_offset:wl.k_offset + D] if wl.fmt == "split" else
                         row[wl.k_offset:wl.k_offset + wl.rot_cols] + v[wl.rot_cols:])
                    keys.append(k)
                    vals.append(v)
                for h in range(g * G, (g + 1) * G):
                    qh = [float(x) for x in wl.q[r, i, h]]
                    w = [math.exp(wl.scale * math.fsum(qh[d] * k[d] for d in range(D))) for k in keys]
                    z = math.fsum(w)
                    out[r, i, h] = [math.fsum(w[t] * vals[t][d] for t in range(len(keys))) / z
                                    for d in range(D)]
    return out


def pin_tree_brute_force():
    """Tree attention on random forests (whole context and a window, split and folded)
    against the parent-walking brute force; a chain of rows is the causal window bit for
    bit; a row whose mask shows no key (no keys before the window) is NaN, the others
    unaffected."""
    for W, fmt, seed in ((0, "split", 40), (5, "split", 41), (0, "folded", 42)):
        D = 17 if fmt == "split" else 512
        wl = synth.make_workload([11, 7, 9], num_q_heads=4, num_kv_heads=2, head_dim=D,
                                 page_size=4, window=W, fmt=fmt, seed=seed, num_rows=6,
                                 pad="big", spare_pages=2)
        synth.set_tree(wl, synth.random_parents(3, 6, seed))
        _assert_close(oracle.decode_attention(wl), brute_force_tree(wl), 1e-13,
                      f"tree W={W} {fmt}")
    wl = synth.make_workload([40, 33], num_q_heads=8, num_kv_heads=1, head_dim=64, page_size=8,
                             seed=43, num_rows=5)
    causal = oracle.decode_attention(wl)
    synth.set_tree(wl, np.tile(np.arange(-1, 4), (2, 1)))
    assert np.array_equal(oracle.decode_attention(wl), causal)
    wl = synth.make_workload([4], num_q_heads=2, num_kv_heads=1, head_dim=8, page_size=4,
                             seed=44, num_rows=4)
    synth.set_tree(wl, np.array([[-1, 0, 0, 1]]))
    masks = wl.row_masks.copy()
    wl.row_masks[0, 2] = np.uint64(0)
    got = oracle.decode_attention(wl)
    assert np.all(np.isnan(got[0, 2]))
    wl.row_masks = masks
    ref = oracle.decode_attention(wl)
    assert np.array_equal(np.delete(got, 2, axis=1), np.delete(ref, 2, axis=1))


def brute_force_chunk_state(wl, r: int, g: int, h: int, row: int, a: int, b: int):
    """(m, l, acc) of query head h (query row ``row`` of request r) over the keys of
    positions [a, b) that the row sees, by pure Python; None when it sees none there.

    Row i of an n-row window over L keys is the token at position p = L - n + i; it sees
    every position j <= p, and with a window W only those with j > p - W.  Scores by
    fsum of explicit products over flat pool indices; m is their maximum, l the fsum of
    e^(s - m), acc the fsum of e^(s - m) v per dimension.
    """
    D = wl.head_dim
    n = getattr(wl, "num_rows", 1)
    elem = _ELEMENT[wl.kv_dtype]
    ks, vs = wl.k_scale, wl.v_scale
    p = int(wl.seq_lens[r]) - n + row
    qh = [float(x) for x in (wl.q[r, row, h] if n > 1 else wl.q[r, h])]
    scores, vals = [], []
    for j in range(a, b):
        if j < 0 or j > p or (wl.window and j <= p - wl.window):
            continue
        pg = int(wl.table[r][j // wl.page_size])
        base = pg * wl.page_stride + g * wl.head_stride + (j % wl.page_size) * wl.row_stride
        rowv = [elem(wl.pool[base + c]) for c in range(wl.row_cols)]
        v = [x * vs for x in rowv[wl.v_offset:wl.v_offset + D]]
        if wl.fmt == "split":
            k = [x * ks for x in rowv[wl.k_offset:wl.k_offset + D]]
        else:
            k = [x * ks for x in rowv[wl.k_offset:wl.k_offset + wl.rot_cols]] + v[wl.rot_cols:]
        scores.append(wl.scale * math.fsum(qh[d] * k[d] for d in range(D)))
        vals.append(v)
    if not scores:
        return None
    m = max(scores)
    e = [math.exp(s - m) for s in scores]
    return m, math.fsum(e), [math.fsum(e[t] * vals[t][d] for t in range(len(e))) for d in range(D)]


# (seq_lens, Hq, Hkv, D, page_size, window, fmt, rows, kv_dtype)
PARTIAL_CASES = [
    ([37, 20, 5], 8, 2, 17, 4, 0, "split", 1, "bf16"),     # whole context, ragged
    ([37, 9, 23], 4, 2, 17, 4, 6, "split", 1, "bf16"),      # window crossing chunks
    ([30, 12], 4, 1, 17, 4, 0, "split", 4, "bf16"),         # each row of a 4-row window
    ([30, 14], 4, 2, 17, 4, 5, "split", 3, "bf16"),         # rows and a window
    ([21], 8, 1, 512, 4, 0, "folded", 2, "bf16"),           # folded row, two rows
    ([26, 11], 4, 2, 33, 4, 7, "split", 2, "fp8_e4m3"),     # FP8 with its factors
]


def pin_paged_partials():
    """Per-chunk states of the paged pool (the states every per-chunk GPU check compares
    against) == a pure-Python state of the keys each chunk and row sees: random cut
    points, chunks wholly before the window or past the length (empty), zero-width
    chunks, every query row of a multi-row window, a window, folded rows, FP8 factors.
    The states of a chunking that covers every key, folded in order, give the pinned
    decode output (gem design note, opening status section: partitions with empty
    members merge to the direct softmax)."""
    rng = _rng(50)
    for k, (lens, hq, hkv, D, ps, W, fmt, n, dt) in enumerate(PARTIAL_CASES):
        wl = synth.make_workload(lens, num_q_heads=hq, num_kv_heads=hkv, head_dim=D, page_size=ps,
                                 window=W, fmt=fmt, seed=60 + k, num_rows=n, kv_dtype=dt,
                                 pad="nan", spare_pages=2)
        G = hq // hkv
        dense = oracle.decode_attention(wl)
        for r, L in enumerate(lens):
            inner = sorted(int(x) for x in rng.integers(0, L + 1, size=4))
            cuts = [-ps, 0] + inner + [L, L + 2 * ps]
            ranges = list(zip(cuts[:-1], cuts[1:])) + [(L // 2, L // 2)]
            for row in range(n):
                for g in range(hkv):
                    states = oracle.paged_partials(wl, r, g, ranges, row=row)
                    assert len(states) == G and all(len(s) == len(ranges) for s in states)
                    for i in range(G):
                        h = g * G + i
                        for c, (a, b) in enumerate(ranges):
                            st = states[i][c]
                            ref = brute_force_chunk_state(wl, r, g, h, row, a, b)
                            what = f"partials case {k} r={r} row={row} h={h} chunk [{a},{b})"
                            if ref is None:
                                assert st.m == -math.inf and st.l == 0.0 and not np.any(st.acc), what
                                continue
                            m, l, acc = ref
                            assert abs(st.m - m) <= 1e-13 * max(1.0, abs(m)), what
                            assert abs(st.l - l) <= 1e-13 * l, what
                            _assert_close(np.asarray(st.acc) / st.l, np.asarray(acc) / l, 1e-13, what)
                        # a chunking that covers every key: folded in order == decode output
                        got = oracle.finalize(oracle.fold(states[i][:-1]))
                        want = dense[r, row, h] if n > 1 else dense[r, h]
                        _assert_close(got, want, 1e-13, what + " (folded)")


ALL_PINS = [pin_brute_force, pin_single_key, pin_uniform_scores, pin_two_keys, pin_needle,
            pin_gqa_grouping, pin_linearity_and_order, pin_partition_invariance,
            pin_empty_merge_identity, pin_merge_identity_values, pin_window,
            pin_permutation_invariance, pin_folded_equals_split, pin_fail_closed,
            pin_query_rows, pin_dtype_brute_force, pin_e4m3_codes, pin_f16_f32_codes,
            pin_dequant_factors, pin_prefill_brute_force, pin_prefill_rows_are_decode,
            pin_prefill_causality, pin_tree_brute_force, pin_paged_partials]
