"""GPU parity of multi-row decode (a window of query rows per request, causal inside
the window) against the fp64 oracle."""
import math

import numpy as np
import pytest

import oracle
import synth
from tests.gpu_harness import Device, note
from tests.test_gpu_parity import check, run_case

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("rows", [2, 3, 4, 5, 8])
@pytest.mark.parametrize("fmt", ["split", "folded"])
def test_rows_global(rows, fmt):
    wl = synth.make_workload([3000, 777, rows + 5], **synth.GLOBAL, fmt=fmt, seed=40 + rows,
                             num_rows=rows, pad="nan")
    dev, got = run_case(wl, f"rows={rows} {fmt}")
    assert dev.plan.num_rows == rows
    check(got, oracle.decode_attention(wl), f"rows={rows} {fmt}")


@pytest.mark.parametrize("rows", [2, 4, 7])
def test_rows_sliding_window(rows):
    wl = synth.make_workload([1030, 1024 + rows - 1, 40, 3000], **synth.SLIDING, seed=50 + rows,
                             num_rows=rows, pad="nan", max_pages=64)
    _, got = run_case(wl, f"sliding rows={rows}")
    check(got, oracle.decode_attention(wl), f"sliding rows={rows}")


@pytest.mark.parametrize("fmt", ["split", "folded"])
def test_rows_global_with_window(fmt):
    """Head dim 512 with a window (the 32-key tile kernel): every row's window starts at a
    different key, chunks start at the first row's window start rounded to a tile, and
    windows cross chunk and tile boundaries; plus a request shorter than the window."""
    wl = synth.make_workload([3000, 1400, 300], **dict(synth.GLOBAL, window=700), fmt=fmt,
                             seed=63, num_rows=6, pad="nan")
    dev, got = run_case(wl, f"rows=6 window=700 {fmt}", num_chunks=7)
    assert dev.plan.tile == 32
    check(got, oracle.decode_attention(wl), f"rows=6 window {fmt}")


@pytest.mark.parametrize("head", [0, 5])
@pytest.mark.parametrize("fmt", ["split", "folded"])
def test_rows_dominant_key(fmt, head):
    """A key at position 100 scores ~160 log2 units above the rest for every row of one
    query head: beyond the headroom of the tile kernel's no-rescale loop, so the workgroups
    of that chunk recompute with rescaling.  With query head 5 no overflowing column sits on
    a wave's first lane; the workgroup's vote must still see it."""
    wl = synth.make_workload([900, 300], **synth.GLOBAL, fmt=fmt, seed=65, num_rows=4, pad="nan")
    u = np.ascontiguousarray(wl.q[0, 2, head], dtype=np.float32)
    wl.q[0, :, head, :] = u
    j = 100
    pid = int(wl.table[0][j // wl.page_size])
    base = pid * wl.page_stride + (j % wl.page_size) * wl.row_stride + wl.k_offset  # KV head 0
    wl.pool[base:base + wl.rot_cols if fmt == "folded" else base + wl.head_dim] = \
        synth.f32_to_bf16_bits((5.0 * (u[:wl.rot_cols] if fmt == "folded" else u)).astype(np.float32))
    if fmt == "folded":   # the unrotated dims score against the V columns: scale those too
        vb = base - wl.k_offset + wl.v_offset + wl.rot_cols
        vals = 5.0 * u[wl.rot_cols:] / wl.fold_w
        wl.pool[vb:vb + wl.head_dim - wl.rot_cols] = synth.f32_to_bf16_bits(vals.astype(np.float32))
    dev, got = run_case(wl, f"rows=4 {fmt} dominant key head {head}", num_chunks=3)
    assert dev.plan.tile == 32
    ref = oracle.decode_attention(wl)
    check(got, ref, f"rows=4 {fmt} dominant key head {head}")
    vj = oracle.keys_values(wl, oracle.stored_to_f64(oracle.gather_rows(wl, 0, 0, [j])))[1][0]
    assert np.max(np.abs(got[0, :, head] - vj)) <= 1e-5


@pytest.mark.parametrize("shape", ["split", "folded", "sliding"])
def test_rows_bad_page_and_device_lengths(shape):
    """Forced from the host (every kernel exits normally): a table entry outside the pool,
    a device length below the row count, and one at the table's capacity (past the plan's
    chunks, or onto empty table entries) each turn only that request's rows into NaN; the
    other request matches the oracle.  Head dim 512 runs the 32-key tile kernel, 256 the
    16-key rows kernel."""
    if shape == "sliding":
        wl = synth.make_workload([1300, 900], **synth.SLIDING, seed=64, num_rows=4, max_pages=40)
    else:
        wl = synth.make_workload([1300, 900], **synth.GLOBAL, fmt=shape, seed=64, num_rows=4)
    ref0 = oracle.decode_attention(wl)[:1]
    good = int(wl.table[1][1])
    wl.table[1][1] = wl.num_pages + 100
    _, got = run_case(wl, f"{shape} rows=4 bad page id")
    assert np.all(np.isnan(got[1]))
    check(got[:1], ref0, f"{shape} healthy request beside a bad page")
    wl.table[1][1] = good
    for lens in ([1300, 3], [1300, wl.max_pages * wl.page_size]):
        note(f"[gpu] {shape} rows=4 device lengths {lens}")
        dev = Device(wl, seq_lens_dev=lens)
        got = dev.run()
        assert dev.guards_intact()
        assert np.all(np.isnan(got[1])), lens
        check(got[:1], ref0, f"{shape} request 0 beside device lengths {lens}")


def test_rows_minimal_lengths_and_explicit_chunks():
    """L == rows (the first row sees one key: exactly v_0), and more chunks than tiles."""
    wl = synth.make_workload([4, 4], **synth.GLOBAL, seed=60, num_rows=4, pad="big")
    dev, got = run_case(wl, "rows=4 L=4 n=9", num_chunks=9)
    check(got, oracle.decode_attention(wl), "rows L=4")
    v0 = oracle.gather_rows(wl, 0, 0, np.array([0]))[0][512:1024]
    v0 = (v0.astype(np.uint32) << 16).view(np.float32)
    for h in range(8):
        assert np.array_equal(got[0, 0, h].view(np.uint32), v0.view(np.uint32))


def test_rows_partials_per_chunk():
    wl = synth.make_workload([900], **synth.GLOBAL, seed=61, num_rows=3)
    dev, got = run_case(wl, "rows=3 partials n=5", num_chunks=5)
    m, l, o = dev.partials()
    ranges = dev.chunk_ranges(0)
    for row in range(3):
        for g in range(4):
            states = oracle.paged_partials(wl, 0, g, ranges, row=row)
            for i in range(8):
                h = g * 8 + i
                for c, st in enumerate(states[i]):
                    b = row  # partial rows are (request * rows + row)
                    if st.m == -math.inf:
                        assert m[b, h, c] == -np.inf and l[b, h, c] == 0
                        continue
                    mg = float(m[b, h, c])
                    assert st.m - 8 * math.log(2) - 1e-5 <= mg <= st.m + 1e-5 * max(1, abs(st.m))
                    k = math.exp(mg - st.m)
                    assert abs(l[b, h, c] * k - st.l) <= 1e-5 * st.l
                    assert np.max(np.abs(o[b, h, c] * k / st.l - st.acc / st.l)) <= 1e-4
    check(got, oracle.decode_attention(wl), "rows partial case")


def test_rows_full_size_163k():
    note("[gpu] rows=4 at 163,336: generating")
    wl = synth.make_workload([163336], **synth.GLOBAL, seed=62, num_rows=4, spare_pages=1)
    dev, got = run_case(wl, "rows=4 L=163336")
    check(got, oracle.decode_attention(wl), "rows=4 163K")
