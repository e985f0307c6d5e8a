"""GPU parity for the pool element types other than bf16: f16 rows (multiplied on
f16 MFMA), FP8 E4M3 rows with K and V dequantisation factors (widened to bf16
on their way into LDS), and f32 rows (split or folded; multiplied in full fp32 on the fp32
MFMA, R = 16 / G query rows in its 16 columns), against the fp64 oracle at the same bar as
bf16."""
import numpy as np
import pytest
import torch

import oracle
import paged_split_kv_02_amd as K
import synth
from tests.gpu_harness import Device, note
from tests.test_gpu_parity import check, check_partials, run_case

pytestmark = pytest.mark.gpu

DTYPES = [synth.F16, synth.FP8]
ALL_DTYPES = DTYPES + [synth.F32]


@pytest.mark.parametrize("fmt", ["split", "folded"])
@pytest.mark.parametrize("dt", ALL_DTYPES)
def test_global_ragged(dt, fmt):
    wl = synth.make_workload([1000, 333, 17], **synth.GLOBAL, fmt=fmt, seed=70, kv_dtype=dt,
                             spare_pages=3, pad="nan")
    for n in (0, 9):
        _, got = run_case(wl, f"{dt} {fmt} L=1000,333,17 n={n}", num_chunks=n)
        check(got, oracle.decode_attention(wl), f"{dt} {fmt} n={n}")


@pytest.mark.parametrize("dt", ALL_DTYPES)
def test_partials_per_chunk(dt):
    wl = synth.make_workload([1000, 333], **synth.GLOBAL, seed=71, kv_dtype=dt, spare_pages=2)
    dev, got = run_case(wl, f"{dt} partials n=9", num_chunks=9, merge_group=4)
    check_partials(dev, wl)
    check(got, oracle.decode_attention(wl), f"{dt} partials")


@pytest.mark.parametrize("dt", ALL_DTYPES)
def test_hostile_padding_bit_identical(dt):
    """NaN, the largest finite value or zero in every slot no query sees: same bits."""
    outs = []
    for pad in ("nan", "big", "zero"):
        wl = synth.make_workload([1000, 257, 16], **synth.GLOBAL, seed=72, kv_dtype=dt, pad=pad,
                                 spare_pages=3)
        _, got = run_case(wl, f"{dt} pad {pad}")
        outs.append(got)
    check(outs[0], oracle.decode_attention(wl), f"{dt} padding")
    assert np.array_equal(outs[0].view(np.uint32), outs[1].view(np.uint32))
    assert np.array_equal(outs[0].view(np.uint32), outs[2].view(np.uint32))


@pytest.mark.parametrize("dt", ALL_DTYPES)
def test_sliding_batch(dt):
    wl = synth.sliding_batch(seed=73, kv_dtype=dt, pad="nan")
    _, got = run_case(wl, f"{dt} sliding batch")
    check(got, oracle.decode_attention(wl), f"{dt} sliding")


@pytest.mark.parametrize("dt", ALL_DTYPES)
@pytest.mark.parametrize("rows", [3, 4])
def test_rows(dt, rows):
    wl = synth.make_workload([2000, rows + 6], **synth.GLOBAL, seed=74 + rows, kv_dtype=dt,
                             num_rows=rows, pad="nan")
    _, got = run_case(wl, f"{dt} rows={rows}")
    check(got, oracle.decode_attention(wl), f"{dt} rows={rows}")
    ws = synth.make_workload([1030, 40], **synth.SLIDING, seed=76 + rows, kv_dtype=dt,
                             num_rows=rows, pad="nan", max_pages=64)
    _, got = run_case(ws, f"{dt} sliding rows={rows}")
    check(got, oracle.decode_attention(ws), f"{dt} sliding rows={rows}")


@pytest.mark.parametrize("rows", [1, 4])
def test_fp8_widening_is_exact(rows):
    """FP8 codes with unit factors and the bf16 pool of the same values (E4M3 is a subset
    of bf16) give identical bits: the kernel multiplies the same bf16 operands.  One row
    runs the split kernel, four rows the 32-key tile kernel."""
    wl8 = synth.make_workload([3000, 700], **synth.GLOBAL, seed=78, kv_dtype=synth.FP8,
                              k_scale=1.0, v_scale=1.0, pad="nan", num_rows=rows)
    # make sure every class of code is present in live rows: subnormals, +-448, +-0
    live = np.flatnonzero(oracle.e4m3_bits_to_f64(wl8.pool) == oracle.e4m3_bits_to_f64(wl8.pool))
    rng = np.random.default_rng(78)
    pick = rng.choice(live, size=4000, replace=False)
    wl8.pool[pick] = rng.choice(np.array([0x01, 0x81, 0x07, 0x87, 0x08, 0x7E, 0xFE, 0x00, 0x80],
                                         dtype=np.uint8), size=pick.size)
    bf = torch.from_numpy(wl8.pool.copy()).view(torch.float8_e4m3fn).to(torch.bfloat16)
    wl16 = synth.make_workload([3000, 700], **synth.GLOBAL, seed=78, pad="nan", num_rows=rows)
    wl16.pool = bf.view(torch.int16).numpy().view(np.uint16)
    wl16.table = wl8.table
    dev8, got8 = run_case(wl8, f"fp8 with extreme codes rows={rows}")
    _, got16 = run_case(wl16, f"bf16 of the same values rows={rows}")
    assert dev8.plan.tile == (32 if rows > 1 else 16)
    assert np.array_equal(got8.view(np.uint32), got16.view(np.uint32))
    # the absolute bar is stated for N(0, 1) values; here V reaches 448, so it scales by that
    check(got8, oracle.decode_attention(wl8), "fp8 extreme codes", tol=2e-3 * 448)


@pytest.mark.parametrize("dt,fmt", [(synth.FP8, "split"), (synth.FP8, "folded"),
                                    (synth.F16, "split"), (synth.F32, "split"),
                                    (synth.F32, "folded")])
def test_full_length_163k(dt, fmt):
    note(f"[gpu] {dt} {fmt} L=163336: generating")
    wl = synth.global_decode(163336, seed=79, fmt=fmt, kv_dtype=dt)
    dev = Device(wl)
    got = dev.run()
    assert dev.guards_intact()
    note(f"[gpu] {dt} {fmt} L=163336: oracle (n={dev.plan.num_chunks})")
    check(got, oracle.decode_attention(wl), f"{dt} {fmt} 163K")


@pytest.mark.parametrize("shape,rows", [("global", 2), ("global", 7), ("sliding", 8),
                                        ("sliding", 13), ("folded", 3), ("sliding-late", 5)])
def test_f32_rows_groups_and_chunks(shape, rows):
    """f32 windows of several rows: R = 16 / G rows share the 16 MFMA columns (2 at head dim
    512, 8 at 256), more rows take further row groups; automatic and explicit chunk counts,
    a window crossing pages, NaN padding."""
    if shape in ("global", "folded"):
        wl = synth.make_workload([2500, rows + 20, 700], **synth.GLOBAL, seed=81 + rows,
                                 kv_dtype=synth.F32, num_rows=rows, pad="nan", spare_pages=2,
                                 fmt="split" if shape == "global" else "folded")
    elif shape == "sliding":
        wl = synth.make_workload([1500, rows + 3, 1030], **synth.SLIDING, seed=81 + rows,
                                 kv_dtype=synth.F32, num_rows=rows, pad="nan", max_pages=40)
    else:
        # the first tile holds keys only the first rows of the window see (their windows
        # start 14 .. 18 keys into it): the later rows' columns have no visible key yet while
        # the first rows' columns move their maximum, and must keep their empty sums
        wl = synth.make_workload([2674, 2944, 1818], **synth.SLIDING, seed=81 + rows,
                                 kv_dtype=synth.F32, num_rows=rows, pad="big")
    ref = oracle.decode_attention(wl)
    for n in (0, 5):
        dev, got = run_case(wl, f"f32 {shape} rows={rows} n={n}", num_chunks=n)
        check(got, ref, f"f32 {shape} rows={rows} n={n}")


def test_f32_rows_partials_per_chunk():
    """Each chunk state of a 3-row f32 window against the oracle's state of the keys that
    row sees in that chunk."""
    import math
    wl = synth.make_workload([900], **synth.GLOBAL, seed=85, kv_dtype=synth.F32, num_rows=3)
    dev, got = run_case(wl, "f32 rows=3 partials n=5", num_chunks=5)
    m, l, o = dev.partials()
    ranges = dev.chunk_ranges(0)
    for row in range(3):
        for g in range(4):
            states = oracle.paged_partials(wl, 0, g, ranges, row=row)
            for i in range(8):
                h = g * 8 + i
                for c, st in enumerate(states[i]):
                    if st.m == -math.inf:
                        assert m[row, h, c] == -np.inf and l[row, h, c] == 0
                        continue
                    mg = float(m[row, h, c])
                    assert st.m - 8 * math.log(2) - 1e-5 <= mg <= st.m + 1e-5 * max(1, abs(st.m))
                    k = math.exp(mg - st.m)
                    assert abs(l[row, h, c] * k - st.l) <= 1e-5 * st.l
                    assert np.max(np.abs(o[row, h, c] * k / st.l - st.acc / st.l)) <= 1e-4
    check(got, oracle.decode_attention(wl), "f32 rows partial case")


@pytest.mark.parametrize("shape", ["split", "folded", "sliding"])
def test_fp8_one_row_quarter_lengths(shape):
    """The one-row FP8 kernel's piece pipeline at quarters of 1, 2, 4, 8 and 16 tiles (and
    empty ones): explicit chunk counts over ragged lengths, outputs and every chunk state."""
    if shape == "sliding":
        wl = synth.make_workload([1100, 333, 17], **synth.SLIDING, seed=90, kv_dtype=synth.FP8,
                                 pad="nan", max_pages=64)
        counts = (1, 2, 4, 5)
    else:
        wl = synth.make_workload([1000, 333, 17], **synth.GLOBAL, fmt=shape, seed=91,
                                 kv_dtype=synth.FP8, spare_pages=2, pad="nan")
        counts = (1, 2, 4, 8, 16)
    ref = oracle.decode_attention(wl)
    for n in counts:
        dev, got = run_case(wl, f"fp8 {shape} one row n={n}", num_chunks=n)
        check(got, ref, f"fp8 {shape} n={n}")
        check_partials(dev, wl)


@pytest.mark.parametrize("shape", ["split", "folded", "sliding"])
def test_fp8_one_row_poisoning(shape):
    """Forced from the host (every kernel exits normally): a table entry outside the pool, or
    a device length past the plan, turns only that request's output into NaN."""
    kw = dict(**synth.SLIDING, max_pages=64) if shape == "sliding" else \
        dict(**synth.GLOBAL, fmt=shape, spare_pages=2)
    wl = synth.make_workload([600, 600], seed=92, kv_dtype=synth.FP8, **kw)
    good = wl.table[1][1]
    wl.table[1][1] = wl.num_pages + 100
    _, got = run_case(wl, f"fp8 {shape} bad page id")
    assert np.all(np.isnan(got[1]))
    wl.table[1][1] = good
    check(got[:1], oracle.decode_attention(wl)[:1], f"fp8 {shape} healthy request")
    note(f"[gpu] fp8 {shape} device length past the plan")
    dev = Device(wl, seq_lens_dev=[600, 5000])
    got = dev.run()
    assert dev.guards_intact()
    assert np.all(np.isnan(got[1]))
    check(got[:1], oracle.decode_attention(wl)[:1], f"fp8 {shape} request 0")


@pytest.mark.parametrize("shape", ["split", "folded", "sliding"])
def test_fp8_one_row_token_major(shape):
    """Token-major pages (the KV heads of a slot side by side: a row stride of several rows)
    through the one-row FP8 kernel."""
    kw = dict(**synth.SLIDING, max_pages=64) if shape == "sliding" else \
        dict(**synth.GLOBAL, fmt=shape, spare_pages=2)
    wl = synth.make_workload([1500, 260, 33], seed=93, kv_dtype=synth.FP8, pad="nan",
                             layout=synth.TOKEN_MAJOR, **kw)
    _, got = run_case(wl, f"fp8 {shape} token-major")
    check(got, oracle.decode_attention(wl), f"fp8 {shape} token-major")
