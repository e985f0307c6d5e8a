"""Pins for the row-write / query-fold reference (CPU only)."""
import math
import struct

import numpy as np
import pytest
import torch

import oracle
import synth


def test_rne_keeps_representable_values():
    rng = np.random.default_rng(0)
    bits = rng.integers(0, 1 << 16, size=5000, dtype=np.uint32).astype(np.uint16)
    bits = bits[(bits & 0x7F80) != 0x7F80]  # finite only
    x = (bits.astype(np.uint32) << 16).view(np.float32)
    assert np.array_equal(oracle.f32_to_bf16_rne(x), bits)


def test_rne_ties_go_to_even_and_halfway_rules():
    def f(b):  # float32 from bit pattern
        return struct.unpack("<f", struct.pack("<I", b))[0]
    cases = [
        (0x3F808000, 0x3F80),  # 1 + 2^-8: exact half, kept part even -> down
        (0x3F818000, 0x3F82),  # kept part odd, exact half -> up to even
        (0x3F808001, 0x3F81),  # just above half -> up
        (0x3F807FFF, 0x3F80),  # just below half -> down
        (0xBF818000, 0xBF82),  # negative, same rule on the magnitude
        (0x7F7FFFFF, 0x7F80),  # largest float rounds to +inf
        (0x7F800000, 0x7F80),  # +inf stays
        (0x00000001, 0x0000),  # tiny denormal rounds to +0
    ]
    x = np.array([f(b) for b, _ in cases], dtype=np.float32)
    got = oracle.f32_to_bf16_rne(x)
    assert [int(v) for v in got] == [e for _, e in cases]
    nan = oracle.f32_to_bf16_rne(np.array([f(0x7F800001), f(0xFFC00000)], dtype=np.float32))
    assert int(nan[0]) == 0x7FC0 and int(nan[1]) == 0xFFC0


def test_rne_matches_torch_bfloat16_conversion():
    """An independent implementation (torch's CPU conversion) agrees on random data."""
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.standard_normal(200000), rng.uniform(-1e30, 1e30, 1000),
                        rng.uniform(-1e-30, 1e-30, 1000)]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.f32_to_bf16_rne(x), ref)


def test_rne_error_bound():
    rng = np.random.default_rng(2)
    x = rng.standard_normal(100000).astype(np.float32)
    back = (oracle.f32_to_bf16_rne(x).astype(np.uint32) << 16).view(np.float32)
    rel = np.abs(back.astype(np.float64) - x) / np.abs(x)
    assert rel.max() <= 2.0 ** -8 * (1 + 1e-12)  # half an ulp of 7 stored mantissa bits


@pytest.mark.parametrize("fmt,layout", [("split", synth.HEAD_MAJOR), ("folded", synth.TOKEN_MAJOR)])
def test_write_rows_lands_where_decode_reads(fmt, layout):
    """Rows written at positions [s, s+n) are exactly what the decode gather returns there,
    and nothing else in the pool changes."""
    wl = synth.make_workload([300, 40], num_q_heads=8, num_kv_heads=2, head_dim=512, page_size=64,
                             fmt=fmt, seed=3, layout=layout, spare_pages=2)
    rng = np.random.default_rng(4)
    n = 37
    start = np.array([250, 1], dtype=np.int32)
    kc = 512 if fmt == "split" else 128
    k = rng.standard_normal((2, n, 2, kc)).astype(np.float32)
    v = rng.standard_normal((2, n, 2, 512)).astype(np.float32)
    # enlarge the logical range so positions up to 286 / 37 are mapped
    new = oracle.write_rows(wl, k, v, start)
    changed = np.flatnonzero(new != wl.pool)
    import copy
    wl2 = copy.copy(wl)
    wl2.pool = new
    touched = set()
    for r in range(2):
        pos = np.arange(start[r], start[r] + n)
        for g in range(2):
            rows = oracle.gather_rows(wl2, r, g, pos)
            assert np.array_equal(rows[:, wl.v_offset:wl.v_offset + 512],
                                  oracle.f32_to_bf16_rne(v[r, :, g]))
            assert np.array_equal(rows[:, wl.k_offset:wl.k_offset + kc],
                                  oracle.f32_to_bf16_rne(k[r, :, g]))
            for j in pos:
                page = wl.table[r][j // 64]
                base = page * wl.page_stride + g * wl.head_stride + (j % 64) * wl.row_stride
                touched.update(range(base + wl.k_offset, base + wl.k_offset + kc))
                touched.update(range(base + wl.v_offset, base + wl.v_offset + 512))
    assert set(changed.tolist()) <= touched


def test_fold_query_is_the_elementwise_product():
    rng = np.random.default_rng(5)
    q = rng.standard_normal((3, 8, 512)).astype(np.float32)
    w = rng.uniform(0.5, 1.5, 384).astype(np.float32)
    qf = oracle.fold_query(q, w, 128)
    assert np.array_equal(qf[..., :128], q[..., :128])
    assert np.array_equal(qf[..., 128:], np.float32(q[..., 128:]) * w)
    # the folded score against V equals the split score against w * V (exact in fp64 up to
    # the single fp32 rounding of q * w, bounded by 2^-24 relative per term)
    vv = rng.standard_normal(384)
    s_fold = float(qf[0, 0, 128:].astype(np.float64) @ vv)
    s_split = float(q[0, 0, 128:].astype(np.float64) @ (w.astype(np.float64) * vv))
    bound = 2.0 ** -24 * float(np.abs(q[0, 0, 128:].astype(np.float64) * w * vv).sum())
    assert abs(s_fold - s_split) <= bound


# ---------------------------------------------------------------- other element types

def _e4m3_values():
    return oracle.e4m3_bits_to_f64(np.arange(256, dtype=np.uint8))


def test_e4m3_every_finite_code_round_trips():
    """Decoding a code and encoding the value gives the code back (254 finite codes, both
    zeros included); the decoded NaN codes encode to a NaN code."""
    vals = _e4m3_values()
    codes = np.arange(256, dtype=np.uint8)
    fin = ~np.isnan(vals)
    got = oracle.f32_to_e4m3(vals.astype(np.float32))
    assert np.array_equal(got[fin], codes[fin])
    assert got[0x7F] & 0x7F == 0x7F and got[0xFF] & 0x7F == 0x7F


def test_e4m3_ties_go_to_the_even_code():
    """Every midpoint between neighbouring non-negative values (0 .. 448) encodes to the
    neighbour with the even mantissa; one float32 step either side goes to the nearer."""
    g = _e4m3_values()[:0x7F]  # codes 0 .. 126 in increasing order
    mid = ((g[:-1] + g[1:]) / 2).astype(np.float32)
    assert np.array_equal(mid.astype(np.float64), (g[:-1] + g[1:]) / 2)  # midpoints are exact
    lo_code = np.arange(0x7E)
    even = np.where(lo_code % 2 == 0, lo_code, lo_code + 1)
    assert np.array_equal(oracle.f32_to_e4m3(mid), even.astype(np.uint8))
    assert np.array_equal(oracle.f32_to_e4m3(-mid), (even | 0x80).astype(np.uint8))
    below = np.nextafter(mid, np.float32(0))
    above = np.nextafter(mid, np.float32(np.inf))
    assert np.array_equal(oracle.f32_to_e4m3(below), lo_code.astype(np.uint8))
    assert np.array_equal(oracle.f32_to_e4m3(above), (lo_code + 1).astype(np.uint8))


def test_e4m3_saturation_nan_and_signed_zero():
    big = np.array([448.0, 449.0, 464.0, 479.9, 480.0, 1e30, np.inf], dtype=np.float32)
    assert np.all(oracle.f32_to_e4m3(big) == 0x7E)
    assert np.all(oracle.f32_to_e4m3(-big) == 0xFE)
    nan = np.array([np.nan, -np.nan], dtype=np.float32)
    nan[1] = -np.abs(nan[1])
    assert oracle.f32_to_e4m3(nan).tolist() == [0x7F, 0xFF]
    tiny = np.array([2.0 ** -10, 1e-30, 0.0], dtype=np.float32)  # round to zero
    assert oracle.f32_to_e4m3(tiny).tolist() == [0, 0, 0]
    assert oracle.f32_to_e4m3(-tiny).tolist() == [0x80, 0x80, 0x80]


def test_e4m3_matches_torch_in_range():
    """An independent implementation (torch's float8_e4m3fn conversion) agrees wherever
    no saturation is involved."""
    rng = np.random.default_rng(7)
    x = np.concatenate([rng.standard_normal(100000) * s for s in (1e-3, 0.1, 1, 30, 200)])
    x = x[np.abs(x) <= 448].astype(np.float32)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(oracle.f32_to_e4m3(x), ref)


def test_e4m3_error_bound():
    """Inside the normal range the error is at most half a step (2^-4 relative)."""
    rng = np.random.default_rng(8)
    x = rng.uniform(2.0 ** -6, 448, 100000).astype(np.float32)
    back = oracle.e4m3_bits_to_f64(oracle.f32_to_e4m3(x))
    assert np.max(np.abs(back - x) / x) <= 2.0 ** -4


def test_f16_rounding_closed_forms_and_torch():
    def f16(b):
        return np.array([b], dtype=np.uint16)
    cases = np.array([65504.0, 65519.99, 65520.0, 2.0 ** -24, 2.0 ** -25, 3 * 2.0 ** -25,
                      1 + 2.0 ** -11, 1 + 3 * 2.0 ** -11], dtype=np.float32)
    got = oracle.f32_to_f16_rne(cases).tolist()
    assert got == [0x7BFF, 0x7BFF, 0x7C00, 0x0001, 0x0000, 0x0002, 0x3C00, 0x3C02]
    rng = np.random.default_rng(9)
    x = np.concatenate([rng.standard_normal(100000), rng.uniform(-1e5, 1e5, 1000),
                        rng.uniform(-1e-6, 1e-6, 1000)]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.float16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.f32_to_f16_rne(x), ref)


def test_encode_stored_divides_by_the_factor_first():
    x = np.array([1.0, -3.3, 100.0, 0.07], dtype=np.float32)
    f = 0.0175
    q = x / np.float32(f)
    assert np.array_equal(oracle.encode_stored(x, "fp8_e4m3", f), oracle.f32_to_e4m3(q))
    assert np.array_equal(oracle.encode_stored(x, "f32", 1.0), x.view(np.uint32))
    assert np.array_equal(oracle.encode_stored(x, "bf16"), oracle.f32_to_bf16_rne(x))
    assert np.array_equal(oracle.encode_stored(x, "f16", 2.0), oracle.f32_to_f16_rne(x / np.float32(2)))
    # a written FP8 value inside the range dequantises to within half a step of the
    # original; 100 / 0.0175 is past 448 and saturates
    y = np.array([1.0, -3.3, 5.0, 0.07], dtype=np.float32)
    back = oracle.e4m3_bits_to_f64(oracle.encode_stored(y, "fp8_e4m3", f)) * f
    assert np.all(np.abs(back - y) <= 2.0 ** -4 * np.abs(y) + 1e-12)
    assert oracle.encode_stored(x, "fp8_e4m3", f)[2] == 0x7E


@pytest.mark.parametrize("dt", ["f16", "fp8_e4m3", "f32"])
def test_write_rows_other_types_land_where_decode_reads(dt):
    """Rows written into an f16, FP8 or f32 pool are the encoded values where the decode
    gather reads them, and nothing else in the pool changes."""
    wl = synth.make_workload([200, 40], num_q_heads=8, num_kv_heads=2, head_dim=512, page_size=64,
                             fmt="split", seed=13, spare_pages=2, kv_dtype=dt)
    rng = np.random.default_rng(14)
    n = 23
    start = np.array([170, 3], dtype=np.int32)
    k = (rng.standard_normal((2, n, 2, 512)) * 3).astype(np.float32)
    v = (rng.standard_normal((2, n, 2, 512)) * 3).astype(np.float32)
    new = oracle.write_rows(wl, k, v, start)
    assert new.dtype == wl.pool.dtype
    import copy
    wl2 = copy.copy(wl)
    wl2.pool = new
    touched = set()
    for r in range(2):
        pos = np.arange(start[r], start[r] + n)
        for g in range(2):
            rows = oracle.gather_rows(wl2, r, g, pos)
            assert np.array_equal(rows[:, 512:1024], oracle.encode_stored(v[r, :, g], dt, wl.v_scale))
            assert np.array_equal(rows[:, 0:512], oracle.encode_stored(k[r, :, g], dt, wl.k_scale))
            for j in pos:
                page = wl.table[r][j // 64]
                base = page * wl.page_stride + g * wl.head_stride + (j % 64) * wl.row_stride
                touched.update(range(base, base + 1024))
    assert set(np.flatnonzero(new != wl.pool).tolist()) <= touched
