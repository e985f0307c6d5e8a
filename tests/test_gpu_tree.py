"""GPU parity of tree attention over a window of query rows (attn_decode_split_tree +
attn_decode_merge through the C ABI) against the fp64 oracle: seeded random forests on
both multi-row kernels (head dim 512 over bf16 or FP8 pages: the 32-key tile kernel; head
dim 256 and f16 pools: the 16-key rows kernel), a chain of rows equal to the
causal window bit for bit, a row that sees no key, per-chunk partials and the full
163,336-token length.  Bar as for decode: max |GPU - oracle| <= 2e-3, NMSE <= 1e-4."""
import math

import numpy as np
import pytest
import torch

import oracle
import paged_split_kv_02_amd as K
import synth
from tests.gpu_harness import Device, note
from tests.test_gpu_parity import check

pytestmark = pytest.mark.gpu


class TreeDevice(Device):
    """A multi-row workload with tree masks, stepped through attn_decode_split_tree."""

    def __init__(self, wl, **kw):
        super().__init__(wl, **kw)
        self.masks = torch.from_numpy(np.ascontiguousarray(wl.row_masks).view(np.int64)).to("cuda:0")

    def step(self, stream=None):
        K.attn_decode_split_tree(self.plan, self.q, self.pool, self.table, self.lens,
                                 self.masks, self.ws, stream=stream)
        K.attn_decode_merge(self.plan, self.ws, self.out, stream=stream)


def run_tree(wl, what, **kw):
    note(f"[gpu] tree {what}")
    dev = TreeDevice(wl, **kw)
    got = dev.run()
    assert dev.guards_intact(), f"{what}: wrote outside out / workspace"
    return dev, got


@pytest.mark.parametrize("rows", [2, 5, 8])
@pytest.mark.parametrize("fmt", ["split", "folded"])
def test_tree_global(rows, fmt):
    wl = synth.make_workload([3000, 777, rows + 5], **synth.GLOBAL, fmt=fmt, seed=120 + rows,
                             num_rows=rows, pad="nan")
    synth.set_tree(wl, synth.random_parents(3, rows, 120 + rows))
    dev, got = run_tree(wl, f"rows={rows} {fmt}")
    assert dev.plan.tile == 32
    check(got, oracle.decode_attention(wl), f"tree rows={rows} {fmt}")


@pytest.mark.parametrize("fmt", ["split", "folded"])
def test_tree_global_with_window(fmt):
    """The tile kernel with tree masks and a window lower bound (700 keys): the bound
    applies to the window's own keys too, rows' bounds differ, chunks are explicit."""
    wl = synth.make_workload([3000, 1400, 300], **dict(synth.GLOBAL, window=700), fmt=fmt,
                             seed=125, num_rows=8, pad="nan")
    synth.set_tree(wl, synth.random_parents(3, 8, 125))
    dev, got = run_tree(wl, f"rows=8 window=700 {fmt}", num_chunks=7)
    assert dev.plan.tile == 32
    check(got, oracle.decode_attention(wl), f"tree window {fmt}")


@pytest.mark.parametrize("shape", ["sliding", "global-f16", "global-fp8"])
def test_tree_on_other_shapes(shape):
    """Head dim 256 and f16 pools on the 16-key rows kernel; FP8 pools at head dim 512 on
    the 32-key tile kernel (codes widened to bf16 on their way into LDS)."""
    if shape == "sliding":
        wl = synth.make_workload([1030, 1500, 40, 3000], **synth.SLIDING, seed=130, num_rows=7,
                                 pad="nan", max_pages=64)
    else:
        dt = synth.F16 if shape.endswith("f16") else synth.FP8
        wl = synth.make_workload([2000, 600], **synth.GLOBAL, seed=131, kv_dtype=dt, num_rows=6,
                                 pad="nan")
    synth.set_tree(wl, synth.random_parents(wl.batch, wl.num_rows, 132))
    dev, got = run_tree(wl, shape)
    assert dev.plan.tile == (32 if shape == "global-fp8" else 16)
    check(got, oracle.decode_attention(wl), f"tree {shape}")


@pytest.mark.parametrize("shape", ["global", "sliding"])
def test_chain_equals_causal_bit_for_bit(shape):
    """Masks 2^(i+1) - 1 through the tree entry point give attn_decode_split's bits."""
    if shape == "global":
        wl = synth.make_workload([2500, 900], **synth.GLOBAL, seed=133, num_rows=4)
    else:
        wl = synth.make_workload([1300, 700], **synth.SLIDING, seed=133, num_rows=4, max_pages=32)
    causal = Device(wl).run()
    synth.set_tree(wl, np.tile(np.arange(-1, 3, dtype=np.int32), (wl.batch, 1)))
    _, got = run_tree(wl, f"chain {shape}")
    assert np.array_equal(got.view(np.uint32), causal.view(np.uint32))


@pytest.mark.parametrize("shape", ["global", "sliding"])
def test_row_that_sees_no_key(shape):
    """A request with no keys before its window and a row whose mask is empty: that row
    is NaN (0 / 0), the request's other rows and the other request match the oracle."""
    if shape == "global":
        wl = synth.make_workload([4, 300], **synth.GLOBAL, seed=134, num_rows=4)
    else:
        wl = synth.make_workload([4, 300], **synth.SLIDING, seed=134, num_rows=4, max_pages=8)
    synth.set_tree(wl, np.array([[-1, 0, -1, 2], [-1, 0, 1, 0]], dtype=np.int32))
    wl.row_masks[0, 2] = np.uint64(0)
    _, got = run_tree(wl, f"empty row {shape}")
    ref = oracle.decode_attention(wl)
    assert np.all(np.isnan(got[0, 2])) and np.all(np.isnan(ref[0, 2]))
    keep = [(0, 0), (0, 1), (0, 3)]
    check(np.stack([got[r, i] for r, i in keep]), np.stack([ref[r, i] for r, i in keep]),
          f"rows beside the empty one ({shape})")
    check(got[1], ref[1], f"other request ({shape})")


def test_tree_partials_per_chunk():
    """Chunk states of a tree window against the oracle's per-chunk states over the keys
    each row sees (m within 8 ln 2 below the chunk's largest score, l and O relative)."""
    wl = synth.make_workload([900], **synth.GLOBAL, seed=135, num_rows=5)
    synth.set_tree(wl, np.array([[-1, 0, 0, 1, -1]], dtype=np.int32))
    dev, got = run_tree(wl, "partials n=5", num_chunks=5)
    m, l, o = dev.partials()
    ranges = dev.chunk_ranges(0)
    L = 900
    for row in range(5):
        pos = oracle.window_row_positions(L, 5, row, 0, int(wl.row_masks[0, row]))
        for g in range(4):
            for c, (a, b) in enumerate(ranges):
                sel = pos[(pos >= a) & (pos < b)]
                for i in range(8):
                    h = g * 8 + i
                    if sel.size == 0:
                        assert m[row, h, c] == -np.inf and l[row, h, c] == 0
                        continue
                    Kk, V = oracle.keys_values(wl, oracle.stored_to_f64(oracle.gather_rows(wl, 0, g, sel)))
                    s = wl.scale * (Kk @ wl.q[0, row, h].astype(np.float64))
                    mt = float(s.max())
                    mg = float(m[row, h, c])
                    assert mt - 8 * math.log(2) - 1e-5 <= mg <= mt + 1e-5 * max(1, abs(mt))
                    e = np.exp(s - mg)
                    assert abs(l[row, h, c] - e.sum()) <= 1e-5 * e.sum()
                    assert np.max(np.abs(o[row, h, c] - e @ V)) <= 1e-4 * e.sum()
    check(got, oracle.decode_attention(wl), "tree partial case")


def test_tree_full_size_163k():
    note("[gpu] tree rows=4 at 163,336: generating")
    wl = synth.make_workload([163336], **synth.GLOBAL, seed=136, num_rows=4, spare_pages=1)
    synth.set_tree(wl, np.array([[-1, 0, 0, 1]], dtype=np.int32))
    _, got = run_tree(wl, "rows=4 L=163336")
    check(got, oracle.decode_attention(wl), "tree rows=4 163K")
