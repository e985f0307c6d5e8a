"""GPU parity of paged prefill (attn_prefill through the C ABI) against the fp64 oracle.

Bar: max |GPU - oracle| <= 2e-3 (the global prefill gate of pegainfer PR #1055,
Verification, taken against fp64), max |GPU - oracle| <= 1e-3 x max|o| (the decode
tests' relative bar, which still bites where long rows make |o| small), NMSE <= 1e-4
and correlation >= 0.9999.  Cases follow
the windowed prefill gates of pegainfer PR #1057 (Verification): crossing the window,
ragged prompts, a continuation and a tiny prompt; plus hostile padding, page-permutation
and layout invariance, determinism, full-size sampled rows, the slow rescale path and
device-side mismatches.
"""
import numpy as np
import pytest
import torch

import oracle
import paged_split_kv_02_amd as K
import synth
from tests.gpu_harness import SENTINEL, compare, fnv1a, note

pytestmark = pytest.mark.gpu

TOL = 2e-3
REL = 1e-3
GUARD_ROWS = 2


class PrefillDevice:
    """A prefill workload's buffers on the GPU, its plan, and a guarded output."""

    def __init__(self, wl, q_starts_dev=None, seq_lens_dev=None, table=None):
        dev = torch.device("cuda:0")
        self.wl = wl
        self.desc = K.make_desc(**wl.desc_fields())
        self.plan = K.attn_prefill_plan(self.desc, wl.seq_lens, wl.q_starts)
        self.q = torch.from_numpy(np.ascontiguousarray(wl.q, dtype=np.float32)).to(dev)
        self.pool = torch.from_numpy(wl.pool.view(np.uint8)).to(dev)
        self.table = torch.from_numpy(wl.table if table is None else table).to(dev)
        lens = wl.seq_lens if seq_lens_dev is None else np.asarray(seq_lens_dev, dtype=np.int32)
        starts = wl.q_starts if q_starts_dev is None else np.asarray(q_starts_dev, dtype=np.int32)
        self.lens = torch.from_numpy(np.ascontiguousarray(lens)).to(dev)
        self.starts = torch.from_numpy(np.ascontiguousarray(starts)).to(dev)
        self.row = wl.num_q_heads * wl.head_dim
        T = int(wl.q_starts[-1])
        self.out_buf = torch.full(((T + 2 * GUARD_ROWS) * self.row,), SENTINEL, dtype=torch.int32,
                                  device=dev)
        self.out = self.out_buf.view(torch.float32)[GUARD_ROWS * self.row:(GUARD_ROWS + T) * self.row]

    def launch(self):
        K.attn_prefill(self.plan, self.q, self.pool, self.table, self.lens, self.starts, self.out)

    def run(self) -> np.ndarray:
        self.launch()
        torch.cuda.synchronize()
        wl = self.wl
        return self.out.cpu().numpy().reshape(-1, wl.num_q_heads, wl.head_dim).copy()

    def guards_intact(self) -> bool:
        ob = self.out_buf.cpu().numpy()
        g = GUARD_ROWS * self.row
        return bool(np.all(ob[:g] == SENTINEL) and np.all(ob[-g:] == SENTINEL))


def check(got, ref, what, tol=TOL):
    st = compare(got, ref)
    note(f"  {what}: max|d|={st['max_abs']:.3e} max|o|={st['max_ref']:.3e} "
         f"nmse={st['nmse']:.3e} corr={st['corr']:.9f}")
    assert st["finite"], what
    assert st["max_abs"] <= tol, (what, st)
    assert st["max_abs"] <= REL * st["max_ref"], (what, st)
    assert st["nmse"] <= 1e-4 and st["corr"] >= 0.9999, (what, st)
    return st


def run_case(wl, what, **kw):
    note(f"[gpu] prefill {what}")
    dev = PrefillDevice(wl, **kw)
    got = dev.run()
    assert dev.guards_intact(), f"{what}: wrote outside out"
    return dev, got


@pytest.mark.parametrize("fmt", ["split", "folded"])
def test_global_ragged(fmt):
    """Fresh prompts, a continuation after earlier keys, a one-row request, a request with
    no new rows, rows crossing pages of 256 and row tiles cut by the prompt's end."""
    wl = synth.make_workload([300, 610, 1, 45, 257], **synth.GLOBAL, fmt=fmt, seed=200,
                             q_lens=[300, 37, 1, 0, 257], spare_pages=3, pad="nan")
    _, got = run_case(wl, f"global {fmt} ragged")
    check(got, oracle.prefill_attention(wl), f"global {fmt} ragged")


def test_sliding_window_cases():
    """Window 1024 over pages of 64: a prompt crossing the window (1300 rows), a
    continuation whose first rows already reach past the window, a short prompt and a
    tiny one."""
    wl = synth.make_workload([1300, 1500, 70, 1], **synth.SLIDING, seed=201,
                             q_lens=[1300, 150, 70, 1], max_pages=40, pad="nan")
    _, got = run_case(wl, "sliding window cases")
    rows = list(range(0, 1300, 7)) + list(range(1300, 1521))
    ref = oracle.prefill_attention(wl, rows=rows)
    check(got[rows], ref, "sliding window cases")


def test_hostile_padding_bit_identical():
    """NaN, a huge value or zero in every slot no prompt row sees: same output bits."""
    outs = []
    for pad in ("nan", "big", "zero"):
        wl = synth.make_workload([200, 1100], **synth.SLIDING, seed=202, q_lens=[200, 90],
                                 pad=pad, max_pages=20)
        _, got = run_case(wl, f"padding {pad}")
        outs.append(got)
    assert np.array_equal(outs[0].view(np.uint32), outs[1].view(np.uint32))
    assert np.array_equal(outs[0].view(np.uint32), outs[2].view(np.uint32))
    check(outs[0], oracle.prefill_attention(wl), "padding")


def test_page_permutation_and_layout_invariance():
    """The same logical rows at other physical pages, or with the slots of all KV heads
    interleaved (token-major pages), give the same bits; so do repeated runs."""
    base = synth.make_workload([700, 300], **synth.GLOBAL, seed=203, q_lens=[700, 64])
    other = synth.make_workload([700, 300], **synth.GLOBAL, seed=203, q_lens=[700, 64],
                                table_seed=999)
    tm = synth.make_workload([700, 300], **synth.GLOBAL, seed=203, q_lens=[700, 64],
                             layout=synth.TOKEN_MAJOR)
    assert not np.array_equal(base.table, other.table)
    dev, a = run_case(base, "permutation base")
    hashes = {fnv1a(a)}
    for _ in range(4):
        hashes.add(fnv1a(dev.run()))
    assert len(hashes) == 1, "repeated runs differ"
    _, b = run_case(other, "permutation other table")
    _, c = run_case(tm, "token-major pages")
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    assert np.array_equal(a.view(np.uint32), c.view(np.uint32))
    check(a[::5], oracle.prefill_attention(base, rows=range(0, 764, 5)), "permutation")


@pytest.mark.parametrize("head", [0, 5])
@pytest.mark.parametrize("shape", ["global", "sliding"])
def test_slow_path_on_a_dominant_key(shape, head):
    """A key planted at position 100 scores ~113 nat (global) / ~80 nat (sliding) above every
    other key for the rows after it: beyond the headroom of the no-rescale loop (the
    probabilities would overflow), so the workgroups recompute with rescaling.  Rows before
    it are ordinary.  With query head 5 no column that overflows sits on a wave's first
    lane: the workgroup's vote must still see it."""
    if shape == "global":
        wl = synth.make_workload([400], **synth.GLOBAL, seed=204, q_lens=[400], pad="nan")
    else:
        wl = synth.make_workload([400], **synth.SLIDING, seed=204, q_lens=[400], pad="nan",
                                 max_pages=8)
    u = np.ascontiguousarray(wl.q[150, head], dtype=np.float32)  # the head's query at row 150
    wl.q[:, head, :] = u                                         # every row of it asks for u
    key = synth.f32_to_bf16_bits((5.0 * u).astype(np.float32))
    j = 100
    g = head // (wl.num_q_heads // wl.num_kv_heads)               # the head's KV head
    pid = int(wl.table[0][j // wl.page_size])
    base = (pid * wl.page_stride + g * wl.head_stride + (j % wl.page_size) * wl.row_stride
            + wl.k_offset)
    wl.pool[base:base + wl.head_dim] = key
    _, got = run_case(wl, f"dominant key {shape} head {head}")
    ref = oracle.prefill_attention(wl)
    check(got, ref, f"dominant key {shape} head {head}")
    v100 = oracle.keys_values(wl, oracle.stored_to_f64(oracle.gather_rows(wl, 0, g, [j])))[1][0]
    assert np.max(np.abs(got[j:, head] - v100)) <= 1e-5


def test_slow_path_with_rows_past_the_window():
    """A dominant key at position 1100 of a 1400-row sliding prompt (window 1024): the
    workgroups of rows 1088 and later recompute with rescaling, and their rows' windows
    start at different tiles, so some columns of a wave have no visible key yet while
    others move their maximum.  Those columns must come out unharmed."""
    wl = synth.make_workload([1400], **synth.SLIDING, seed=207, q_lens=[1400], pad="nan",
                             max_pages=24)
    u = np.ascontiguousarray(wl.q[700, 0], dtype=np.float32)
    wl.q[:, 0, :] = u
    j = 1100
    pid = int(wl.table[0][j // wl.page_size])
    base = pid * wl.page_stride + (j % wl.page_size) * wl.row_stride + wl.k_offset
    wl.pool[base:base + wl.head_dim] = synth.f32_to_bf16_bits((5.0 * u).astype(np.float32))
    _, got = run_case(wl, "dominant key past the window")
    rows = sorted(set(range(0, 1400, 9)) | set(range(1080, 1230)) | set(range(1380, 1400)))
    check(got[rows], oracle.prefill_attention(wl, rows=rows), "dominant key past the window")
    vj = oracle.keys_values(wl, oracle.stored_to_f64(oracle.gather_rows(wl, 0, 0, [j])))[1][0]
    assert np.max(np.abs(got[j:, 0] - vj)) <= 1e-5


def test_full_size_global_sampled():
    """The 10,602-token prompt of one request (pages of 256, shuffled), split and folded,
    at the launch configuration the bench times; sampled rows against the oracle: the first
    rows, row-tile and page boundaries, the last rows and a seeded random sample."""
    rng = np.random.default_rng(7)
    n = 10602
    rows = sorted(set([0, 1, 7, 8, 9, 255, 256, 257, 4095, 4096, n - 9, n - 8, n - 2, n - 1]
                      + list(range(131, n, 128)) + rng.integers(0, n, 40).tolist()))
    for fmt in ("split", "folded"):
        note(f"[gpu] prefill {fmt} n=10602: generating")
        wl = synth.global_prefill(n, seed=205, fmt=fmt)
        dev, got = run_case(wl, f"{fmt} 10602 rows")
        check(got[rows], oracle.prefill_attention(wl, rows=rows), f"{fmt} 10602 sampled")
        assert fnv1a(dev.run()) == fnv1a(got)


def test_full_size_sliding_sampled():
    """Sixteen ragged prompts (lengths 1..4096, seeded), window 1024, pages of 64: the
    sliding-layer varlen prefill at the size the bench times; sampled rows per request."""
    wl = synth.sliding_prefill(seed=12)
    _, got = run_case(wl, "sliding 16 ragged prompts")
    rng = np.random.default_rng(8)
    starts = wl.q_starts
    rows = []
    for r in range(wl.batch):
        a, b = int(starts[r]), int(starts[r + 1])
        rows += sorted(set([a, a + 1, b - 1] + list(range(a + 63, b, 64)) +
                           rng.integers(a, b, 8).tolist()))
    check(got[rows], oracle.prefill_attention(wl, rows=rows), "sliding 16 sampled")


@pytest.mark.parametrize("fmt", ["split", "folded"])
def test_fp8_global_ragged(fmt):
    """FP8 E4M3 pools (factors 0.0175 / 0.0225): the codes are widened to bf16 on their
    way into LDS; ragged prompts, a continuation, a one-row and a zero-row request."""
    wl = synth.make_workload([300, 610, 1, 45, 257], **synth.GLOBAL, fmt=fmt, seed=210,
                             q_lens=[300, 37, 1, 0, 257], spare_pages=3, pad="nan",
                             kv_dtype=synth.FP8)
    _, got = run_case(wl, f"fp8 global {fmt} ragged")
    check(got, oracle.prefill_attention(wl), f"fp8 global {fmt} ragged")


def test_fp8_sliding_window_cases():
    wl = synth.make_workload([1300, 1500, 70, 1], **synth.SLIDING, seed=211, kv_dtype=synth.FP8,
                             q_lens=[1300, 150, 70, 1], max_pages=40, pad="nan")
    _, got = run_case(wl, "fp8 sliding window cases")
    rows = list(range(0, 1300, 7)) + list(range(1300, 1521))
    check(got[rows], oracle.prefill_attention(wl, rows=rows), "fp8 sliding window cases")


@pytest.mark.parametrize("shape", ["global-split", "global-folded", "sliding"])
def test_fp8_prefill_equals_bf16_of_the_same_values(shape):
    """With unit factors an FP8 pool and the bf16 pool of the same values (every E4M3
    value is a bf16 value) give identical output bits: the widening is exact and the
    kernel multiplies the same operands.  Extreme codes (+-448, subnormals, +-0) are
    planted among the live keys."""
    if shape == "sliding":
        kw = dict(synth.SLIDING)
        mk = dict(max_pages=20, q_lens=[200, 90])
        lens = [200, 1100]
    else:
        kw = dict(synth.GLOBAL)
        mk = dict(fmt=shape.split("-")[1], q_lens=[300, 64])
        lens = [300, 700]
    wl8 = synth.make_workload(lens, **kw, seed=212, kv_dtype=synth.FP8, k_scale=1.0, v_scale=1.0,
                              pad="nan", **mk)
    live = np.flatnonzero(oracle.e4m3_bits_to_f64(wl8.pool) == oracle.e4m3_bits_to_f64(wl8.pool))
    rng = np.random.default_rng(212)
    pick = rng.choice(live, size=3000, replace=False)
    wl8.pool[pick] = rng.choice(np.array([0x01, 0x81, 0x07, 0x87, 0x08, 0x7E, 0xFE, 0x00, 0x80],
                                         dtype=np.uint8), size=pick.size)
    wl16 = synth.make_workload(lens, **kw, seed=212, pad="nan", **mk)
    bf = torch.from_numpy(wl8.pool.copy()).view(torch.float8_e4m3fn).to(torch.bfloat16)
    wl16.pool = bf.view(torch.int16).numpy().view(np.uint16)
    wl16.table = wl8.table
    _, got8 = run_case(wl8, f"fp8 {shape} extreme codes")
    _, got16 = run_case(wl16, f"bf16 {shape} of the same values")
    assert np.array_equal(got8.view(np.uint32), got16.view(np.uint32))
    check(got8, oracle.prefill_attention(wl8), f"fp8 {shape} extreme codes", tol=2e-3 * 448)


def test_device_mismatches_fail_closed():
    """Device inputs the plan cannot serve: a request whose device offsets claim more rows
    than the plan allows is skipped (its rows keep the sentinel); a device length below the
    row count, or a page id outside the pool, turns that request's rows into NaN; the other
    requests are unaffected."""
    wl = synth.make_workload([300, 200, 100], **synth.GLOBAL, seed=206, q_lens=[300, 50, 100],
                             spare_pages=2)
    good = run_case(wl, "mismatch baseline")[1]
    starts = wl.q_starts.copy()            # [0, 300, 350, 450]
    bad_starts = starts.copy()
    bad_starts[1] = 0                      # request 0 claims 0 rows, request 1 claims 350 > 300
    dev = PrefillDevice(wl, q_starts_dev=bad_starts)
    got = dev.run()
    assert np.all(got[0:300].view(np.uint32) == SENTINEL)     # request 1 skipped: rows 0..299 untouched
    assert np.array_equal(got[350:].view(np.uint32), good[350:].view(np.uint32))
    assert dev.guards_intact()
    lens = wl.seq_lens.copy()
    lens[1] = 10                           # fewer keys than its 50 rows
    got = PrefillDevice(wl, seq_lens_dev=lens).run()
    assert np.all(np.isnan(got[300:350]))
    assert np.array_equal(got[:300].view(np.uint32), good[:300].view(np.uint32))
    table = wl.table.copy()
    table[2, 0] = wl.num_pages + 5         # a page id outside the pool for request 2
    got = PrefillDevice(wl, table=table).run()
    assert np.all(np.isnan(got[350:450]))
    assert np.array_equal(got[:350].view(np.uint32), good[:350].view(np.uint32))


@pytest.mark.parametrize("fmt", ["split", "folded"])
def test_f16_global_ragged(fmt):
    """f16 pools: rows multiplied on the f16 MFMA (query and probabilities as high and low
    f16 parts); ragged prompts, a continuation, a one-row and a zero-row request."""
    wl = synth.make_workload([300, 610, 1, 45, 257], **synth.GLOBAL, fmt=fmt, seed=220,
                             q_lens=[300, 37, 1, 0, 257], spare_pages=3, pad="nan",
                             kv_dtype=synth.F16)
    _, got = run_case(wl, f"f16 global {fmt} ragged")
    check(got, oracle.prefill_attention(wl), f"f16 global {fmt} ragged")


def test_f16_sliding_window_cases():
    wl = synth.make_workload([1300, 1500, 70, 1], **synth.SLIDING, seed=221, kv_dtype=synth.F16,
                             q_lens=[1300, 150, 70, 1], max_pages=40, pad="nan")
    _, got = run_case(wl, "f16 sliding window cases")
    rows = list(range(0, 1300, 7)) + list(range(1300, 1521))
    check(got[rows], oracle.prefill_attention(wl, rows=rows), "f16 sliding window cases")


@pytest.mark.parametrize("shape", ["global", "sliding"])
def test_f16_slow_path_on_a_dominant_key(shape):
    """f16 operands hold probabilities only up to 65504, so the no-rescale loop allows 2^15
    above a column's reference: a key planted at position 100 that scores ~23 nat (global) /
    ~16 nat (sliding) above the rest sends the workgroups of later rows through the
    rescaling loop (the fast loop would overflow to infinity)."""
    if shape == "global":
        wl = synth.make_workload([400], **synth.GLOBAL, seed=222, q_lens=[400], pad="nan",
                                 kv_dtype=synth.F16)
    else:
        wl = synth.make_workload([400], **synth.SLIDING, seed=222, q_lens=[400], pad="nan",
                                 max_pages=8, kv_dtype=synth.F16)
    head = 3
    u = np.ascontiguousarray(wl.q[150, head], dtype=np.float32)
    wl.q[:, head, :] = u
    j = 100
    g = head // (wl.num_q_heads // wl.num_kv_heads)
    pid = int(wl.table[0][j // wl.page_size])
    base = (pid * wl.page_stride + g * wl.head_stride + (j % wl.page_size) * wl.row_stride
            + wl.k_offset)
    wl.pool[base:base + wl.head_dim] = u.astype(np.float16).view(np.uint16)
    _, got = run_case(wl, f"f16 dominant key {shape}")
    check(got, oracle.prefill_attention(wl), f"f16 dominant key {shape}")


@pytest.mark.parametrize("fmt", ["split", "folded"])
def test_f32_global_ragged(fmt):
    """f32 pools: prompt rows on the f32 kernel's prefill mode, two rows of the eight heads
    per workgroup, each wave a quarter of the keys; ragged prompts, a continuation, a
    one-row and a zero-row request, rows crossing pages of 256."""
    wl = synth.make_workload([300, 610, 1, 45, 257], **synth.GLOBAL, fmt=fmt, seed=230,
                             q_lens=[300, 37, 1, 0, 257], spare_pages=3, pad="nan",
                             kv_dtype=synth.F32)
    dev, got = run_case(wl, f"f32 global {fmt} ragged")
    assert dev.plan.row_tile == 2 and dev.plan.key_tile == 16
    check(got, oracle.prefill_attention(wl), f"f32 global {fmt} ragged")


def test_f32_sliding_window_cases():
    """f32, window 1024 over pages of 64: eight rows of the two heads per workgroup; a
    prompt crossing the window, a continuation, a short and a tiny prompt."""
    wl = synth.make_workload([1300, 1500, 70, 1], **synth.SLIDING, seed=231, kv_dtype=synth.F32,
                             q_lens=[1300, 150, 70, 1], max_pages=40, pad="nan")
    dev, got = run_case(wl, "f32 sliding window cases")
    assert dev.plan.row_tile == 8
    rows = list(range(0, 1300, 7)) + list(range(1300, 1521))
    check(got[rows], oracle.prefill_attention(wl, rows=rows), "f32 sliding window cases")


def test_f32_hostile_padding_and_repeat():
    """NaN or huge values in every slot no row sees leave the f32 prefill's bits unchanged;
    a second launch gives the same bits."""
    outs = []
    for pad in ("nan", "big"):
        wl = synth.make_workload([200, 700], **synth.GLOBAL, seed=232, q_lens=[200, 90], pad=pad,
                                 kv_dtype=synth.F32, spare_pages=2)
        dev, got = run_case(wl, f"f32 padding {pad}")
        outs.append(got)
    assert np.array_equal(outs[0].view(np.uint32), outs[1].view(np.uint32))
    assert fnv1a(dev.run()) == fnv1a(outs[1])
    check(outs[0], oracle.prefill_attention(wl), "f32 padding")
