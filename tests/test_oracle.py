"""The fp64 oracle against brute force, closed forms, invariants and the pages' figures,
plus planted mistakes (in copies of the oracle, on the CPU) that the pins must catch."""
import math

import numpy as np
import pytest

import oracle
import oracle.attention as OA
from tests import oracle_pins as P


@pytest.mark.parametrize("pin", P.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin()


def test_gem_audit_bounds_short():
    P.pin_gem_audit_bounds(lengths=[8191, 8192, 8193])


def test_gem_audit_bounds_long():
    P.pin_gem_audit_bounds(lengths=[65536, 131072])


# ---------------------------------------------------------------------- planted mistakes

def _kv_swapped(wl, rows):
    K, V = _orig_keys_values(wl, rows)
    return V, K


def _gqa_modulo(wl):
    G = wl.num_q_heads // wl.num_kv_heads
    out = np.empty((wl.batch, wl.num_q_heads, wl.head_dim))
    for r in range(wl.batch):
        lo, L = OA.visible_range(int(wl.seq_lens[r]), wl.window)
        for h in range(wl.num_q_heads):
            g = h % wl.num_kv_heads
            K, V = OA.keys_values(wl, OA.bf16_bits_to_f64(OA.gather_rows(wl, r, g, np.arange(lo, L))))
            out[r, h] = OA.dense_attention(wl.q[r, h][None], K, V, wl.scale)[0]
    return out


def _no_scale(q, K, V, scale):
    return _orig_dense(q, K, V, 1.0)


def _window_off_by_one(L, window):
    lo, hi = _orig_visible(L, window)
    return (lo + 1 if window > 0 and lo > 0 else lo), hi


def _folded_wrong_cols(wl, rows):
    K, V = _orig_keys_values(wl, rows)
    if wl.fmt == "folded":
        K = rows[:, :wl.head_dim]
    return K, V


def _merge_no_rescale(a, b):
    OA.validate(a)
    OA.validate(b)
    M = max(a.m, b.m)
    if M == -math.inf:
        return OA.empty_state(a.acc.shape[0])
    alpha = 0.0 if a.m == -math.inf else math.exp(a.m - M)
    beta = 0.0 if b.m == -math.inf else math.exp(b.m - M)
    return OA.State(M, alpha * a.l + beta * b.l, a.acc + b.acc)


def _merge_swapped_weights(a, b):
    OA.validate(a)
    OA.validate(b)
    M = max(a.m, b.m)
    if M == -math.inf:
        return OA.empty_state(a.acc.shape[0])
    alpha = 0.0 if a.m == -math.inf else math.exp(a.m - M)
    beta = 0.0 if b.m == -math.inf else math.exp(b.m - M)
    return OA.State(M, beta * a.l + alpha * b.l, beta * a.acc + alpha * b.acc)


def _gather_slot_page_swapped(wl, r, g, positions):
    positions = np.asarray(positions, dtype=np.int64)
    pages = wl.table[r][(positions % wl.page_size) % wl.table.shape[1]].astype(np.int64)
    pages = np.clip(pages, 0, wl.num_pages - 1)
    return OA.row_view(wl)[pages, g, positions // wl.page_size % wl.page_size]


def _dense_max_wrong_axis(q, K, V, scale):
    q = np.asarray(q, dtype=np.float64)
    s = scale * (q @ K.T)
    m = s.max(axis=0, keepdims=True)
    e = np.exp(s - m)
    return (e @ V) / e.sum(axis=1, keepdims=True).max()


def _validate_lenient(st):
    return None


_orig_keys_values = OA.keys_values
_orig_dense = OA.dense_attention
_orig_visible = OA.visible_range

def _rows_off_by_one(wl):
    n = getattr(wl, "num_rows", 1)
    if n == 1:
        return _orig_decode(wl)
    import copy
    one = copy.copy(wl)
    one.num_rows = 1
    outs = []
    for i in range(n):
        one.q = np.ascontiguousarray(wl.q[:, i])
        one.seq_lens = np.minimum(wl.seq_lens - n + 2 + i, wl.seq_lens).astype(np.int32)
        outs.append(_orig_decode(one))
    return np.stack(outs, axis=1)


_orig_decode = OA.decode_attention


def _k_factor_dropped(wl, rows):
    import copy
    one = copy.copy(wl)
    one.k_scale = 1.0
    return _orig_keys_values(one, rows)


def _folded_key_takes_k_factor(wl, rows):
    K, V = _orig_keys_values(wl, rows)
    if wl.fmt == "folded":
        K = K.copy()
        K[:, wl.rot_cols:] *= wl.k_scale / wl.v_scale
    return K, V


def _e4m3_bias_8(bits):
    return _orig_e4m3(bits) / 2.0


def _e4m3_subnormal_as_normal(bits):
    b = np.asarray(bits, dtype=np.uint8).astype(np.int64)
    out = _orig_e4m3(bits)
    e, m = (b >> 3) & 15, (b & 7).astype(np.float64)
    sub = (e == 0) & (m > 0)
    sign = np.where(b & 0x80, -1.0, 1.0)
    return np.where(sub, sign * (1 + m / 8) * 2.0 ** -7, out)


_orig_e4m3 = OA.e4m3_bits_to_f64


def _prefill_rows_from_zero(wl):
    return [(r, i) for r in range(wl.batch) for i in range(int(wl.q_lens[r]))]


def _prefill_excludes_own_key(wl, rows=None):
    import dataclasses
    G = wl.num_q_heads // wl.num_kv_heads
    index = OA.prefill_row_index(wl)
    sel = range(len(index)) if rows is None else list(rows)
    out = np.empty((len(sel), wl.num_q_heads, wl.head_dim))
    for k, t in enumerate(sel):
        r, p = index[t]
        lo, hi = OA.visible_range(max(p, 1), wl.window)
        for g in range(wl.num_kv_heads):
            K, V = OA.keys_values(wl, OA.stored_to_f64(OA.gather_rows(wl, r, g, np.arange(lo, hi)),
                                                       wl.kv_dtype))
            hs = slice(g * G, (g + 1) * G)
            out[k, hs] = OA.dense_attention(wl.q[t, hs], K, V, wl.scale)
    return out

def _tree_masks_read_by_index(L, n, i, window, mask):
    # reads the mask as "the first popcount(mask) rows" instead of the rows it names
    if mask is not None:
        mask = (1 << bin(mask).count("1")) - 1
    return _window_row_positions(L, n, i, window, mask)


_window_row_positions = OA.window_row_positions


def _partials_variant(row_offset=True, window=True, clip=True):
    """paged_partials with one of its visible-range steps left out."""
    def f(wl, r, g, ranges, row=0):
        G = wl.num_q_heads // wl.num_kv_heads
        n = getattr(wl, "num_rows", 1)
        q = wl.q if n > 1 else wl.q[:, None]
        hi = int(wl.seq_lens[r]) - n + 1 + row if row_offset else int(wl.seq_lens[r])
        lo, L = OA.visible_range(hi, wl.window if window else 0)
        out = [[] for _ in range(G)]
        for a, b in ranges:
            pos = np.arange(max(a, lo), min(b, L)) if clip else np.arange(max(a, 0), b)
            pos = pos[pos < int(wl.seq_lens[r])] if not clip else pos
            K, V = OA.keys_values(wl, OA._stored_rows(wl, r, g, pos))
            for i in range(G):
                out[i].append(OA.partial_state(q[r, row, g * G + i], K, V, wl.scale))
        return out
    return f



MUTANTS = {
    "rows_see_one_key_too_many": ("decode_attention", _rows_off_by_one),
    "k_v_swapped": ("keys_values", _kv_swapped),
    "gqa_modulo": ("decode_attention", _gqa_modulo),
    "scale_dropped": ("dense_attention", _no_scale),
    "window_off_by_one": ("visible_range", _window_off_by_one),
    "folded_wrong_columns": ("keys_values", _folded_wrong_cols),
    "merge_without_rescale": ("merge", _merge_no_rescale),
    "merge_weights_swapped": ("merge", _merge_swapped_weights),
    "gather_slot_page_swapped": ("gather_rows", _gather_slot_page_swapped),
    "softmax_max_wrong_axis": ("dense_attention", _dense_max_wrong_axis),
    "no_fail_closed": ("validate", _validate_lenient),
    "k_factor_dropped": ("keys_values", _k_factor_dropped),
    "folded_key_takes_k_factor": ("keys_values", _folded_key_takes_k_factor),
    "e4m3_bias_8": ("e4m3_bits_to_f64", _e4m3_bias_8),
    "e4m3_subnormal_as_normal": ("e4m3_bits_to_f64", _e4m3_subnormal_as_normal),
    "prefill_rows_from_zero": ("prefill_row_index", _prefill_rows_from_zero),
    "prefill_excludes_own_key": ("prefill_attention", _prefill_excludes_own_key),
    "tree_masks_read_by_index": ("window_row_positions", _tree_masks_read_by_index),
    "partials_row_offset_dropped": ("paged_partials", _partials_variant(row_offset=False)),
    "partials_window_dropped": ("paged_partials", _partials_variant(window=False)),
    "partials_not_clipped_to_row": ("paged_partials", _partials_variant(clip=False)),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(OA, attr, fn)
    monkeypatch.setattr(oracle, attr, fn, raising=False)
    caught = []
    for pin in P.ALL_PINS:
        try:
            pin()
        except (AssertionError, IndexError, ValueError, FloatingPointError):
            caught.append(pin.__name__)
    assert caught, f"no pin caught the planted mistake {name}"
