"""Plain, slow, fp64 reference for paged decode attention and its split-KV algebra.

TEST INFRASTRUCTURE ONLY (see the package docstring): the product path never
reaches this module.

What it computes, and where the pages fix it
--------------------------------------------
* Decode attention for one new token per request: every query head h attends,
  with a dense softmax, over the keys of its KV group at the visible positions.
  The paged layout only changes *where* a row lives: logical position j of
  request r is slot j % page_size of physical page table[r][j // page_size]
  (TensorFold PR #1619, body: "page p is rows [256p, 256(p+1))"; the table maps a
  stream's logical pages to leased pool pages).
* GQA: eight query heads share one KV head (gem design note, "Fixed production
  shape").  Reading taken: head h uses KV head h // (Hq / Hkv), the consecutive
  grouping.
* Rows: the split row is K | V; the folded row keeps only the rotated K columns
  and all of V, and the unrotated part of the score is taken against V with the
  norm weight folded into the query (pegainfer PR #1055, Description).
* Windowed decode (sliding layers): the resident pages may hold one page more
  than the window and those older keys are masked (pegainfer PR #1057,
  Description).  Reading taken: position j is visible iff L - W <= j < L.
* Several query rows per request (TensorFold PR #1619, review thread: drafted verify
  windows go through the paged decode kernels): row i of an n-row window is the token at
  position L - n + i and sees the keys before L - n + i + 1, i.e. each row is ordinary
  decode at its own length.
* Prefill (prompt rows): the generated global prefill reads the split or folded pool
  beside the decode kernels (pegainfer PR #1055, Description), the sliding family's
  prompt rows attend through a varlen kernel with a window lower bound over pages of
  64 (pegainfer PR #1057, Description; its gates cover crossing the window, ragged
  prompts, a continuation and a tiny prompt, Verification), and prompt rows read keys
  through the slot's page-table row (TensorFold PR #1619, body).  Reading taken: a
  request with n new rows and L keys in all holds its new rows at positions L - n ..
  L - 1, and each row attends causally, i.e. exactly as a decode token at length
  position + 1 (n = 0: nothing to compute; n < L: a continuation after L - n earlier
  keys).
* Split-KV: each key chunk yields an online-softmax partial (running max M, sum
  S, unnormalised numerator O); partials merge with the exact rescaling identity
  M = max(Ma, Mb), S = Sa e^(Ma-M) + Sb e^(Mb-M), O likewise, then O / S; empty
  partitions are valid states, and invalid finite states fail closed (gem design
  note, opening status paragraph and "Candidate ownership and storage").  The
  merge runs in two levels: groups of consecutive chunk partials first, then the
  group states (pegainfer PR #1055, Description).

* Stored element types (the KV precisions other than bf16: F32 KV in the gem design
  note, "Fixed production shape"; F16 and quantised KV named there as separate axes).
  Reading taken for "quantised": FP8 E4M3 as defined by the OCP 8-bit floating point
  specification (OFP8, the E4M3 encoding: bias 7, three mantissa bits, subnormals,
  no infinities, only S.1111.111 is NaN), with one dequantisation factor for all of K
  and one for all of V: the key used is stored value * k_scale, the value
  stored value * v_scale.  Other element types take factors too (1 by default).

All arithmetic is float64.  Every stored element type widens exactly (bf16, f16,
FP8 and f32 values are all float64 values); fp32 queries widen exactly.  Library
primitives used as steps: numpy's matmul, exp, max and sum, and numpy's IEEE binary16
and binary32 types for widening f16 and f32 bit patterns.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Sequence

import numpy as np

__all__ = [
    "InvalidState", "State", "bf16_bits_to_f64", "f16_bits_to_f64", "e4m3_bits_to_f64",
    "f32_bits_to_f64", "stored_to_f64", "visible_range", "row_view", "gather_rows",
    "keys_values", "dense_attention", "decode_attention", "window_row_positions",
    "partial_state", "empty_state",
    "merge", "finalize", "fold", "split_kv_attention", "paged_partials", "validate",
    "prefill_attention", "prefill_row_index",
]


class InvalidState(ValueError):
    """A split-KV state that cannot arise from any set of finite keys."""


# --------------------------------------------------------------------------------------
# data access

def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 is the upper half of an IEEE binary32, so widening is exact."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def f16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """IEEE binary16 bit patterns to float64 (numpy's half type as the widening step)."""
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def e4m3_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """OCP FP8 E4M3 codes to float64, from the encoding's fields.

    sign s = bit 7, exponent e = bits 6..3 (bias 7), mantissa m = bits 2..0:
      e == 0      : (-1)^s * m/8 * 2^(1-7)       (subnormal; m = 0 gives +-0)
      otherwise   : (-1)^s * (1 + m/8) * 2^(e-7)
      e = 15, m = 7 : NaN (the only non-finite codes; there is no infinity)
    """
    b = np.asarray(bits, dtype=np.uint8).astype(np.int64)
    sign = np.where(b & 0x80, -1.0, 1.0)
    e = (b >> 3) & 0xF
    m = (b & 0x7).astype(np.float64)
    mag = np.where(e == 0, (m / 8.0) * 2.0 ** (1 - 7), (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((b & 0x7F) == 0x7F, np.nan, mag)
    return sign * mag


def f32_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """IEEE binary32 bit patterns to float64."""
    return np.asarray(bits, dtype=np.uint32).view(np.float32).astype(np.float64)


def stored_to_f64(bits: np.ndarray, kv_dtype: str = "bf16") -> np.ndarray:
    """Stored element bit patterns of the given type, widened to float64 (no scaling)."""
    if kv_dtype == "bf16":
        return bf16_bits_to_f64(bits)
    if kv_dtype == "f16":
        return f16_bits_to_f64(bits)
    if kv_dtype == "fp8_e4m3":
        return e4m3_bits_to_f64(bits)
    if kv_dtype == "f32":
        return f32_bits_to_f64(bits)
    raise ValueError(f"unknown element type {kv_dtype}")


def _stored_rows(wl, r: int, g: int, positions: np.ndarray) -> np.ndarray:
    return stored_to_f64(gather_rows(wl, r, g, positions), getattr(wl, "kv_dtype", "bf16"))


def visible_range(L: int, window: int) -> tuple[int, int]:
    """Positions [lo, L) that a decode token at context length L attends to."""
    if L < 1:
        raise ValueError("a decode step needs at least one key")
    lo = max(0, L - window) if window > 0 else 0
    return lo, L


def row_view(wl) -> np.ndarray:
    """The pool seen as rows[page][kv_head][slot][col] through the layout strides."""
    itemsize = wl.pool.dtype.itemsize
    return np.lib.stride_tricks.as_strided(
        wl.pool,
        shape=(wl.num_pages, wl.num_kv_heads, wl.page_size, wl.row_cols),
        strides=(wl.page_stride * itemsize, wl.head_stride * itemsize,
                 wl.row_stride * itemsize, itemsize),
        writeable=False)


def gather_rows(wl, r: int, g: int, positions: np.ndarray) -> np.ndarray:
    """Bit patterns of the stored rows of KV head g at logical positions of request r."""
    positions = np.asarray(positions, dtype=np.int64)
    pages = wl.table[r][positions // wl.page_size].astype(np.int64)
    if positions.size and (pages.min() < 0 or pages.max() >= wl.num_pages):
        raise IndexError("page table points outside the pool")
    slots = positions % wl.page_size
    return row_view(wl)[pages, g, slots]


def keys_values(wl, rows_f64: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Split a stored row into the vectors the score and the output use.

    split : k = row[k_off : k_off+D],  v = row[v_off : v_off+D]
    folded: the score is q'[0:rot].row[k_off : k_off+rot] + q'[rot:D].v[rot:D],
            so the effective key is (row[k_off : k_off+rot], v[rot:D]).
    Stored values are dequantised: K columns times k_scale, V columns times v_scale
    (the folded key's V columns are V columns, so they take v_scale).
    """
    D = wl.head_dim
    ks = float(getattr(wl, "k_scale", 1.0))
    vs = float(getattr(wl, "v_scale", 1.0))
    V = rows_f64[:, wl.v_offset:wl.v_offset + D] * vs
    if wl.fmt == "split":
        K = rows_f64[:, wl.k_offset:wl.k_offset + D] * ks
    else:
        rot = wl.rot_cols
        K = np.concatenate([rows_f64[:, wl.k_offset:wl.k_offset + rot] * ks, V[:, rot:]], axis=1)
    return K, V


# --------------------------------------------------------------------------------------
# dense definition

def dense_attention(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float) -> np.ndarray:
    """softmax(scale * q K^T) V for query rows q[H][D] over keys K[n][D], values V[n][Dv].

    Materialise every score, subtract the row maximum, exponentiate, normalise.
    """
    q = np.asarray(q, dtype=np.float64)
    s = scale * (q @ K.T)                      # [H][n]
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    z = e.sum(axis=1, keepdims=True)
    return (e @ V) / z


def window_row_positions(L: int, n: int, i: int, window: int, mask: int | None) -> np.ndarray:
    """Key positions row i of an n-row window over L keys attends to, ascending.

    Causal (mask None): the positions before L - n + i + 1, and with a sliding window
    not older than W keys back from there.  Tree attention (TensorFold PR #1619 names
    the paged tree-attention decode kernels of its drafted verify windows, body and
    review thread; the mask is our reading): the same keys before the window, L - n,
    and of the window's own keys L - n + j those whose bit j is set in the row's mask,
    again not older than the window's lower bound.  Causal is the mask of bits 0 .. i.
    """
    lo, hi = visible_range(L - n + 1 + i, window)
    if mask is None:
        return np.arange(lo, hi)
    start = L - n
    own = [start + j for j in range(n) if (mask >> j) & 1 and start + j >= lo]
    return np.concatenate([np.arange(lo, start), np.array(own, dtype=np.int64)]).astype(np.int64)


def decode_attention(wl) -> np.ndarray:
    """fp64 output of one decode step over the paged pool: [B][Hq][D], or
    [B][rows][Hq][D] when the workload has a window of several query rows.

    Query row i of a window of n rows sits at position L - n + i and attends causally:
    to the keys at positions before L - n + i + 1 (and, with a sliding window, not older
    than W keys back from there), or, given tree masks, as `window_row_positions`
    describes.  One row is ordinary decode.  A row that sees no key gets NaN (0 / 0).
    """
    G = wl.num_q_heads // wl.num_kv_heads
    n = getattr(wl, "num_rows", 1)
    masks = getattr(wl, "row_masks", None)
    q = wl.q if n > 1 else wl.q[:, None]
    out = np.empty((wl.batch, n, wl.num_q_heads, wl.head_dim), dtype=np.float64)
    for r in range(wl.batch):
        for i in range(n):
            mask = None if masks is None else int(masks[r][i])
            pos = window_row_positions(int(wl.seq_lens[r]), n, i, wl.window, mask)
            if pos.size == 0:
                out[r, i] = np.nan
                continue
            for g in range(wl.num_kv_heads):
                K, V = keys_values(wl, _stored_rows(wl, r, g, pos))
                heads = slice(g * G, (g + 1) * G)
                out[r, i, heads] = dense_attention(q[r, i, heads], K, V, wl.scale)
    return out if n > 1 else out[:, 0]


def prefill_row_index(wl) -> list[tuple[int, int]]:
    """(request, position) of every packed query row of a prefill workload."""
    out = []
    for r in range(wl.batch):
        L = int(wl.seq_lens[r])
        n = int(wl.q_lens[r])
        out.extend((r, L - n + i) for i in range(n))
    return out


def prefill_attention(wl, rows: Sequence[int] | None = None) -> np.ndarray:
    """fp64 output of paged prefill: [T][Hq][D] over the packed query rows (T = sum of
    the requests' new rows), or only the packed rows listed in ``rows``.

    A row of request r at position p attends to the keys at positions lo .. p of that
    request (lo = 0, or p + 1 - W with a sliding window W), through the page table.
    """
    G = wl.num_q_heads // wl.num_kv_heads
    index = prefill_row_index(wl)
    sel = range(len(index)) if rows is None else [int(t) for t in rows]
    out = np.empty((len(sel), wl.num_q_heads, wl.head_dim), dtype=np.float64)
    for k, t in enumerate(sel):
        r, p = index[t]
        lo, hi = visible_range(p + 1, wl.window)
        pos = np.arange(lo, hi)
        for g in range(wl.num_kv_heads):
            K, V = keys_values(wl, _stored_rows(wl, r, g, pos))
            heads = slice(g * G, (g + 1) * G)
            out[k, heads] = dense_attention(wl.q[t, heads], K, V, wl.scale)
    return out


# --------------------------------------------------------------------------------------
# split-KV algebra

@dataclasses.dataclass
class State:
    """Online-softmax state of a set of keys for one query head (natural-log units).

    m = max score, l = sum of e^(s - m), acc = sum of e^(s - m) v.
    The empty set is (-inf, 0, 0).
    """
    m: float
    l: float
    acc: np.ndarray


def empty_state(dv: int) -> State:
    return State(-math.inf, 0.0, np.zeros(dv, dtype=np.float64))


def validate(st: State) -> None:
    """Fail closed on states no finite key set produces."""
    if math.isnan(st.m) or st.m == math.inf:
        raise InvalidState("maximum is NaN or +inf")
    if not np.all(np.isfinite(st.acc)) or not math.isfinite(st.l):
        raise InvalidState("non-finite sum or numerator")
    if st.m == -math.inf:
        if st.l != 0.0 or np.any(st.acc != 0.0):
            raise InvalidState("empty state with a non-zero sum or numerator")
    elif st.l < 1.0:
        # the maximal key contributes e^0 = 1 to a non-empty state's sum
        raise InvalidState("non-empty state with sum below one")


def partial_state(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float) -> State:
    """State of one query vector q[D] over the keys K[n][D] / values V[n][Dv]."""
    if K.shape[0] == 0:
        return empty_state(V.shape[1])
    s = scale * (K @ np.asarray(q, dtype=np.float64))
    m = float(s.max())
    e = np.exp(s - m)
    return State(m, float(e.sum()), e @ V)


def merge(a: State, b: State) -> State:
    """Exact rescaling merge of two states; an empty side leaves the other unchanged."""
    validate(a)
    validate(b)
    M = max(a.m, b.m)
    if M == -math.inf:
        return empty_state(a.acc.shape[0])
    alpha = 0.0 if a.m == -math.inf else math.exp(a.m - M)
    beta = 0.0 if b.m == -math.inf else math.exp(b.m - M)
    return State(M, alpha * a.l + beta * b.l, alpha * a.acc + beta * b.acc)


def finalize(st: State) -> np.ndarray:
    validate(st)
    if st.l == 0.0:
        raise InvalidState("finalize of an empty state (no keys)")
    return st.acc / st.l


def fold(states: Sequence[State]) -> State:
    """Left-to-right merge of consecutive states."""
    acc = states[0]
    validate(acc)
    for st in states[1:]:
        acc = merge(acc, st)
    return acc


def split_kv_attention(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float,
                       cuts: Sequence[int], group: int) -> np.ndarray:
    """Attention of q[D] through chunk partials merged in two levels.

    ``cuts`` are chunk boundaries 0 = c0 <= c1 <= ... <= cn = n (equal cuts give
    empty chunks); level one folds each run of ``group`` consecutive chunk
    states, level two folds the group states, then O / S.
    """
    parts = [partial_state(q, K[a:b], V[a:b], scale) for a, b in zip(cuts[:-1], cuts[1:])]
    groups = [fold(parts[i:i + group]) for i in range(0, len(parts), group)]
    return finalize(fold(groups))


def paged_partials(wl, r: int, g: int, ranges: Sequence[tuple[int, int]],
                   row: int = 0) -> list[list[State]]:
    """Per-chunk states for the G query heads of KV head g of request r (query row
    `row` of a multi-row window).

    ``ranges`` are position intervals [a, b); positions outside the row's visible
    range are dropped.  Returns states[h_in_group][chunk].
    """
    G = wl.num_q_heads // wl.num_kv_heads
    n = getattr(wl, "num_rows", 1)
    q = wl.q if n > 1 else wl.q[:, None]
    lo, L = visible_range(int(wl.seq_lens[r]) - n + 1 + row, wl.window)
    out = [[] for _ in range(G)]
    for a, b in ranges:
        pos = np.arange(max(a, lo), min(b, L))
        K, V = keys_values(wl, _stored_rows(wl, r, g, pos))
        for i in range(G):
            out[i].append(partial_state(q[r, row, g * G + i], K, V, wl.scale))
    return out
