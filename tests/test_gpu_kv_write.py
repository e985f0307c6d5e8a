"""GPU parity of the row write and the query fold (bit-exact: byte work) and of a decode
step that appends its token through them."""
import copy

import numpy as np
import pytest
import torch

import oracle
import paged_split_kv_02_amd as K
import synth
from tests.gpu_harness import Device, note
from tests.test_gpu_parity import check

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _t(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to(DEV)


_SIGNED = {np.dtype(np.uint16): np.int16, np.dtype(np.uint8): np.uint8, np.dtype(np.uint32): np.int32}


def _write_on_gpu(wl, k, v, start, expect_bad=False):
    plan = K.attn_decode_plan(K.make_desc(**wl.desc_fields()), wl.seq_lens)
    pool = _t(wl.pool.view(_SIGNED[wl.pool.dtype]))
    bad = torch.zeros(1, dtype=torch.int32, device=DEV)
    K.attn_kv_write(plan, _t(k), _t(v), k.shape[1], _t(np.asarray(start, dtype=np.int32)), pool,
                    _t(wl.table), bad)
    torch.cuda.synchronize()
    assert int(bad.item()) == int(expect_bad)
    return pool.cpu().numpy().view(wl.pool.dtype)


@pytest.mark.parametrize("fmt,layout,n", [("split", synth.HEAD_MAJOR, 37), ("folded", synth.TOKEN_MAJOR, 37),
                                          ("split", synth.TOKEN_MAJOR, 1), ("folded", synth.HEAD_MAJOR, 300)])
def test_write_rows_bit_exact(fmt, layout, n):
    note(f"[gpu] kv write {fmt} {layout} n={n}")
    wl = synth.make_workload([700, 520], **synth.GLOBAL, fmt=fmt, seed=20, layout=layout, spare_pages=2)
    rng = np.random.default_rng(21)
    kc = 512 if fmt == "split" else 128
    k = rng.standard_normal((2, n, 4, kc)).astype(np.float32) * 3
    v = rng.standard_normal((2, n, 4, 512)).astype(np.float32) * 3
    start = [700 - n, 200]
    got = _write_on_gpu(wl, k, v, start)
    assert np.array_equal(got, oracle.write_rows(wl, k, v, np.array(start)))


def test_prefill_sized_write_bit_exact():
    note("[gpu] kv write prefill 10602 tokens")
    wl = synth.global_decode(10602, seed=22)
    rng = np.random.default_rng(23)
    k = rng.standard_normal((1, 10602, 4, 512)).astype(np.float32)
    v = rng.standard_normal((1, 10602, 4, 512)).astype(np.float32)
    got = _write_on_gpu(wl, k, v, [0])
    assert np.array_equal(got, oracle.write_rows(wl, k, v, np.array([0])))


def test_bad_rows_are_skipped_and_flagged():
    note("[gpu] kv write past the table")
    wl = synth.make_workload([300], **synth.GLOBAL, seed=24)
    rng = np.random.default_rng(25)
    k = rng.standard_normal((1, 4, 4, 512)).astype(np.float32)
    v = rng.standard_normal((1, 4, 4, 512)).astype(np.float32)
    cap = wl.max_pages * 256
    got = _write_on_gpu(wl, k, v, [cap - 2], expect_bad=True)   # last two rows fall past the row
    ref = oracle.write_rows(wl, k[:, :2], v[:, :2], np.array([cap - 2]))
    assert np.array_equal(got, ref)


def test_query_fold_bit_exact():
    note("[gpu] query fold")
    wl = synth.make_workload([64, 64], **synth.GLOBAL, fmt="folded", seed=26)
    plan = K.attn_decode_plan(K.make_desc(**wl.desc_fields()), wl.seq_lens)
    q = _t(wl.q_unfolded)
    out = torch.empty_like(q)
    K.attn_query_fold(plan, q, _t(wl.fold_w), out)
    torch.cuda.synchronize()
    ref = oracle.fold_query(wl.q_unfolded, wl.fold_w, 128)
    assert np.array_equal(out.cpu().numpy().view(np.uint32), ref.view(np.uint32))


@pytest.mark.parametrize("fmt", ["split", "folded"])
def test_append_then_decode(fmt):
    """One decode step end to end: fold q (folded pool), write the new token's row at L-1,
    then split + merge; compare with the oracle on the oracle-written pool."""
    note(f"[gpu] append + decode {fmt}")
    lens = [5000, 777]
    wl = synth.make_workload(lens, **synth.GLOBAL, fmt=fmt, seed=27)
    rng = np.random.default_rng(28)
    kc = 512 if fmt == "split" else 128
    k = rng.standard_normal((2, 1, 4, kc)).astype(np.float32)
    v = rng.standard_normal((2, 1, 4, 512)).astype(np.float32)
    start = np.array(lens, dtype=np.int32) - 1
    dev = Device(wl)
    K.attn_kv_write(dev.plan, _t(k), _t(v), 1, _t(start), dev.pool, dev.table)
    if fmt == "folded":
        K.attn_query_fold(dev.plan, _t(wl.q_unfolded), _t(wl.fold_w), dev.q)
    got = dev.run()
    assert dev.guards_intact()
    ref_wl = copy.copy(wl)
    ref_wl.pool = oracle.write_rows(wl, k, v, start)
    if fmt == "folded":
        ref_wl.q = oracle.fold_query(wl.q_unfolded, wl.fold_w, 128)
    check(got, oracle.decode_attention(ref_wl), f"append+decode {fmt}")


def _hard_values(rng, shape, dt, factor):
    """Random values with the encodings' hard cases planted: exact E4M3 midpoints (ties),
    saturating and tiny magnitudes, f16 overflow and subnormals, signed zeros, and (FP8)
    NaN, all scaled by the tensor's factor so that the quotient hits them."""
    x = rng.standard_normal(shape).astype(np.float32) * np.float32(2.0)
    flat = x.reshape(-1)
    if dt == "fp8_e4m3":
        g = oracle.e4m3_bits_to_f64(np.arange(0x7F, dtype=np.uint8))
        special = np.concatenate([(g[:-1] + g[1:]) / 2, g, [449.0, 480.0, 1e6, np.inf, 2.0 ** -11,
                                                            0.0, -0.0, np.nan]])
    elif dt == "f16":
        special = np.array([65504.0, 65520.0, 1e6, np.inf, 2.0 ** -24, 2.0 ** -25, 3 * 2.0 ** -25,
                            1 + 2.0 ** -11, 1 + 3 * 2.0 ** -11, 0.0, -0.0])
    else:
        special = np.array([np.inf, 1e-40, 3.4e38, 0.0, -0.0])
    special = np.concatenate([special, -special]).astype(np.float32) * np.float32(factor)
    idx = rng.choice(flat.size, size=special.size, replace=False)
    flat[idx] = special
    return x


@pytest.mark.parametrize("dt,fmt,factors", [("f16", "split", (1.0, 1.0)),
                                            ("fp8_e4m3", "split", (1.0, 1.0)),
                                            ("fp8_e4m3", "folded", (None, None)),
                                            ("fp8_e4m3", "split", (None, None)),
                                            ("f32", "split", (1.0, 1.0)),
                                            ("f16", "folded", (0.5, 2.0))])
def test_write_rows_other_types_bit_exact(dt, fmt, factors):
    """f16, FP8 E4M3 and f32 pools: every written element equals the oracle's encoding of
    value / factor (nearest with ties to even; FP8 saturating at 448, NaN kept), over the
    whole pool; the pool's own factors (FP8: 0.0175 / 0.0225) or unit ones."""
    note(f"[gpu] kv write {dt} {fmt} factors={factors}")
    kw = {} if factors[0] is None else dict(k_scale=factors[0], v_scale=factors[1])
    wl = synth.make_workload([700, 520], **synth.GLOBAL, fmt=fmt, seed=30, spare_pages=2,
                             kv_dtype=dt, **kw)
    rng = np.random.default_rng(31)
    n = 64
    kc = 512 if fmt == "split" else 128
    k = _hard_values(rng, (2, n, 4, kc), dt, wl.k_scale)
    v = _hard_values(rng, (2, n, 4, 512), dt, wl.v_scale)
    start = [700 - n, 100]
    got = _write_on_gpu(wl, k, v, start)
    ref = oracle.write_rows(wl, k, v, np.array(start))
    assert got.dtype == ref.dtype
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("dt", ["f16", "fp8_e4m3", "f32"])
def test_append_then_decode_other_types(dt):
    """A decode step over an f16, FP8 or f32 pool after the library writes the new token's
    row (FP8 with its factors): the step equals the oracle on the oracle-written pool."""
    note(f"[gpu] append + decode {dt}")
    lens = [3000, 640]
    wl = synth.make_workload(lens, **synth.GLOBAL, seed=32, kv_dtype=dt)
    rng = np.random.default_rng(33)
    k = (rng.standard_normal((2, 1, 4, 512)) * 2).astype(np.float32)
    v = (rng.standard_normal((2, 1, 4, 512)) * 2).astype(np.float32)
    if dt == "fp8_e4m3":  # values the factors bring inside the FP8 range
        k *= np.float32(wl.k_scale * 100)
        v *= np.float32(wl.v_scale * 100)
    start = np.array(lens, dtype=np.int32) - 1
    dev = Device(wl)
    K.attn_kv_write(dev.plan, _t(k), _t(v), 1, _t(start), dev.pool, dev.table)
    got = dev.run()
    assert dev.guards_intact()
    ref_wl = copy.copy(wl)
    ref_wl.pool = oracle.write_rows(wl, k, v, start)
    check(got, oracle.decode_attention(ref_wl), f"append+decode {dt}")
