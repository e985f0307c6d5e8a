"""Seeded random cases through the decode and prefill entry points against the fp64 oracle.

Each case draws its own shape from a seed: the global family (split or folded rows, with
or without a window) or the sliding family, any element type, one request or a ragged
batch, one query row or a window of rows (causal or a random tree), automatic or explicit
chunk counts, head- or token-major pages and NaN / huge / zero padding.  The bars are
those of the fixed-case suites: max |GPU - oracle| <= 2e-3, <= 1e-3 of max|o|, NMSE <= 1e-4.
Every drawn case is one the plans accept.
"""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_harness import note
from tests.test_gpu_parity import check, run_case
from tests.test_gpu_prefill import check as check_prefill, run_case as run_prefill
from tests.test_gpu_tree import run_tree

pytestmark = pytest.mark.gpu


def decode_case(seed: int):
    rng = np.random.default_rng(5000 + seed)
    family = "global" if rng.random() < 0.65 else "sliding"
    shape = dict(synth.GLOBAL if family == "global" else synth.SLIDING)
    dtype = [synth.BF16, synth.BF16, synth.F16, synth.FP8, synth.F32][int(rng.integers(5))]
    fmt = "folded" if family == "global" and rng.random() < 0.35 else "split"
    rows = 1 if rng.random() < 0.5 else int(rng.integers(2, 9))
    if family == "global" and dtype == synth.BF16 and rng.random() < 0.25:
        shape["window"] = int(rng.integers(64, 2000))
    batch = int(rng.integers(1, 5))
    lens = [int(rng.integers(rows, 3500)) for _ in range(batch)]
    layout = synth.TOKEN_MAJOR if rng.random() < 0.25 else synth.HEAD_MAJOR
    pad = ["nan", "big", "zero"][int(rng.integers(3))]
    wl = synth.make_workload(lens, **shape, fmt=fmt, seed=6000 + seed, kv_dtype=dtype,
                             num_rows=rows, layout=layout, pad=pad,
                             spare_pages=int(rng.integers(0, 4)))
    tree = rows > 1 and rng.random() < 0.5
    if tree:
        synth.set_tree(wl, synth.random_parents(batch, rows, 7000 + seed))
    chunks = 0 if rng.random() < 0.5 else int(rng.integers(1, 65))
    what = (f"seed {seed}: {family} {fmt} {dtype} rows={rows}{' tree' if tree else ''} "
            f"window={shape.get('window', 0)} lens={lens} chunks={chunks} {layout} pad={pad}")
    return wl, tree, chunks, what


@pytest.mark.parametrize("seed", range(128))
def test_random_decode(seed):
    wl, tree, chunks, what = decode_case(seed)
    note(f"[gpu] random decode {what}")
    if tree:
        _, got = run_tree(wl, what, num_chunks=chunks)
    else:
        _, got = run_case(wl, what, num_chunks=chunks)
    check(got, oracle.decode_attention(wl), what)


@pytest.mark.parametrize("seed", range(48))
def test_random_prefill(seed):
    rng = np.random.default_rng(8000 + seed)
    family = "global" if rng.random() < 0.6 else "sliding"
    shape = dict(synth.GLOBAL if family == "global" else synth.SLIDING)
    u = rng.random()
    dtype = synth.FP8 if u < 0.25 else synth.F16 if u < 0.4 else synth.F32 if u < 0.5 else synth.BF16
    fmt = "folded" if family == "global" and rng.random() < 0.35 else "split"
    batch = int(rng.integers(1, 4))
    lens = [int(rng.integers(1, 1800)) for _ in range(batch)]
    q_lens = [int(rng.integers(0, min(L, 300) + 1)) for L in lens]
    q_lens[int(rng.integers(batch))] = max(1, q_lens[0])  # at least one new row
    q_lens = [min(n, L) for n, L in zip(q_lens, lens)]
    layout = synth.TOKEN_MAJOR if rng.random() < 0.25 else synth.HEAD_MAJOR
    pad = ["nan", "big", "zero"][int(rng.integers(3))]
    wl = synth.make_workload(lens, **shape, fmt=fmt, seed=9000 + seed, kv_dtype=dtype,
                             q_lens=q_lens, layout=layout, pad=pad, spare_pages=2)
    what = f"seed {seed}: {family} {fmt} {dtype} lens={lens} new rows={q_lens} {layout} pad={pad}"
    note(f"[gpu] random prefill {what}")
    _, got = run_prefill(wl, what)
    # every request's first and last new rows, plus a seeded sample
    starts = np.concatenate([[0], np.cumsum(q_lens)])
    rows = {int(starts[r]) for r in range(batch) if q_lens[r]}
    rows |= {int(starts[r + 1]) - 1 for r in range(batch) if q_lens[r]}
    total = int(starts[-1])
    rows |= set(rng.integers(0, total, size=min(total, 24)).tolist())
    rows = sorted(rows)
    check_prefill(got[rows], oracle.prefill_attention(wl, rows=rows), what)
