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
