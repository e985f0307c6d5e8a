"""Seeded synthetic inputs for paged decode attention.

This module only *builds data*: query vectors, bf16 K/V rows scattered into a
paged pool through a shuffled page table, and the per-request lengths.  It holds
none of the attention arithmetic, so both the fp64 oracle (``oracle/``) and the
GPU path can consume the same bits without sharing any of the method's code.

Shapes and distributions follow the workloads on the pages:

* global layers of Gemma 4 31B: 32 query heads, 4 KV heads (eight query heads
  per KV head), head dim 512, pages of 256 positions, one decode token
  (pegainfer PR #1055, Description and Verification; TensorFold PR #1619, body);
* the split row is K[0:512] | V[0:512] (1024 bf16 columns); the folded row is
  the 128 rotated K columns followed by all of V (640 columns), with K's norm
  weight folded into the query at prep time (pegainfer PR #1055, Description);
* sliding layers: head dim 256, window 1024, pages of 64 (pegainfer PR #1057,
  Description).

q, K and V are N(0, 1); q stays fp32.  K/V are stored in the pool's element
type: bf16 or f16 (round-to-nearest-even), f32 (as drawn) or FP8 E4M3 codes of
x / scale (round-to-nearest-even, clamped to the largest finite code) with one
dequantisation factor for K and one for V.  Random numbers come from a seeded
torch CPU generator (Mersenne Twister stream, deterministic for a given seed on
any host); the same seed draws the same N(0, 1) values whatever the element type.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional, Sequence

import numpy as np
import torch

SPLIT = "split"
FOLDED = "folded"

HEAD_MAJOR = "head_major"    # pool[page][kv_head][slot][cols]
TOKEN_MAJOR = "token_major"  # pool[page][slot][kv_head][cols]

# Element types of the K/V pool (the C descriptor's kv_dtype codes).
BF16 = "bf16"
F16 = "f16"
FP8 = "fp8_e4m3"
F32 = "f32"
KV_DTYPES = {BF16: 0, F16: 1, FP8: 2, F32: 3}
KV_BYTES = {BF16: 2, F16: 2, FP8: 1, F32: 4}
KV_NUMPY = {BF16: np.uint16, F16: np.uint16, FP8: np.uint8, F32: np.uint32}
# Default dequantisation factors of FP8 pools (not powers of two, K != V).
FP8_K_SCALE = 0.0175
FP8_V_SCALE = 0.0225
FP8_MAX = 448.0

# Bit patterns used to make unused slots hostile: a quiet NaN, a huge finite value
# (about 1e30; the largest finite value for f16 and FP8) and zero.
BF16_QNAN = 0x7FC0
BF16_BIG = 0x7149
PADS = {"nan": BF16_QNAN, "big": BF16_BIG, "zero": 0x0000}
PADS_BY_DTYPE = {
    BF16: PADS,
    F16: {"nan": 0x7E00, "big": 0x7BFF, "zero": 0},
    FP8: {"nan": 0x7F, "big": 0x7E, "zero": 0},
    F32: {"nan": 0x7FC00000, "big": 0x7149F2CA, "zero": 0},
}


@dataclasses.dataclass
class Workload:
    """One decode step's inputs.  All arrays live on the host."""
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    fmt: str                 # SPLIT or FOLDED
    rot_cols: int            # folded: stored rotated K columns (128); split: 0
    page_size: int
    max_pages: int           # page-table row length
    window: int              # 0 = whole context
    scale: float
    layout: str
    num_pages: int
    row_cols: int            # stored columns (elements) per row
    page_stride: int         # elements between pages
    head_stride: int         # elements between KV heads inside a page
    row_stride: int          # elements between consecutive slots
    k_offset: int            # column where the K part starts
    v_offset: int            # column where V starts
    q: np.ndarray            # float32 [B][Hq][D]  (folded: the folded query)
    pool: np.ndarray         # element bit patterns (uint8/16/32), flat, num_pages * page_stride
    table: np.ndarray        # int32 [B][max_pages], -1 where no page
    seq_lens: np.ndarray     # int32 [B]
    fold_w: Optional[np.ndarray] = None   # float32 [D - rot_cols] (folded pair only)
    q_unfolded: Optional[np.ndarray] = None
    num_rows: int = 1        # query rows per request; > 1 makes q [B][rows][Hq][D]
    # Prefill: new query rows per request (ragged, 0 allowed); q is then packed
    # [sum(q_lens)][Hq][D], request r owning rows q_starts[r] .. q_starts[r + 1].
    q_lens: Optional[np.ndarray] = None
    kv_dtype: str = BF16     # element type of the pool
    k_scale: float = 1.0     # K = stored value * k_scale
    v_scale: float = 1.0     # V = stored value * v_scale
    # Tree attention over a window of several rows: parent window row of each row (-1:
    # hangs directly off the keys before the window) and its encoding as the kernels
    # take it, bit j of row_masks[r][i] set when row i sees window row j.
    tree_parents: Optional[np.ndarray] = None   # int32 [B][rows]
    row_masks: Optional[np.ndarray] = None      # uint64 [B][rows]

    @property
    def group_size(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    def rows_of(self, r: int) -> int:
        """Query rows of request r (its last positions)."""
        return int(self.q_lens[r]) if self.q_lens is not None else self.num_rows

    @property
    def q_starts(self) -> np.ndarray:
        """int32 [B + 1]: packed query rows of request r are q_starts[r] .. q_starts[r + 1]."""
        lens = self.q_lens if self.q_lens is not None else np.full(self.batch, self.num_rows)
        return np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)

    def visible(self, r: int) -> tuple[int, int]:
        """[lo, hi) of the key positions request r's rows attend to, together."""
        L = int(self.seq_lens[r])
        first = L - max(self.rows_of(r), 1) + 1   # keys the first query row sees: [.., first)
        lo = max(0, first - self.window) if self.window > 0 else 0
        return lo, L

    def desc_fields(self, num_chunks: int = 0, merge_group: int = 0) -> dict:
        """The pool/batch description as plain fields (names of the C descriptor)."""
        return dict(batch=self.batch, num_q_heads=self.num_q_heads,
                    num_kv_heads=self.num_kv_heads, head_dim=self.head_dim,
                    format=0 if self.fmt == SPLIT else 1, rot_cols=self.rot_cols,
                    page_size=self.page_size, max_pages_per_seq=self.max_pages,
                    window=self.window, num_chunks=num_chunks, merge_group=merge_group,
                    scale=self.scale, num_pages=self.num_pages, page_stride=self.page_stride,
                    head_stride=self.head_stride, row_stride=self.row_stride,
                    k_offset=self.k_offset, v_offset=self.v_offset,
                    num_rows=self.num_rows, kv_dtype=KV_DTYPES[self.kv_dtype],
                    k_scale=self.k_scale, v_scale=self.v_scale)

    def kv_bytes(self) -> int:
        """Bytes of K/V rows a decode step must stream (visible keys only)."""
        n = sum(self.visible(r)[1] - self.visible(r)[0] for r in range(self.batch))
        return n * self.num_kv_heads * self.row_cols * KV_BYTES[self.kv_dtype]


def _gen(seed: int) -> torch.Generator:
    return torch.Generator().manual_seed(int(seed))


def _normal_stored(gen: torch.Generator, shape, kv_dtype: str, k_scale: float,
                   v_scale: float, k_cols: slice) -> np.ndarray:
    """N(0,1) fp32 values in the pool's element type (bit patterns).  FP8 codes are
    x / scale, with K's factor on the ``k_cols`` columns and V's on the rest."""
    x = torch.randn(*shape, generator=gen, dtype=torch.float32)
    if kv_dtype == BF16:
        return x.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    if kv_dtype == F16:
        return x.to(torch.float16).view(torch.int16).numpy().view(np.uint16)
    if kv_dtype == F32:
        return x.numpy().view(np.uint32).copy()
    if kv_dtype == FP8:
        div = torch.full((shape[-1],), float(v_scale), dtype=torch.float32)
        div[k_cols] = float(k_scale)
        y = (x / div).clamp(-FP8_MAX, FP8_MAX)
        return y.to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()
    raise ValueError(kv_dtype)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (RNE) and return the bit patterns."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _strides(layout: str, num_kv_heads: int, page_size: int, row_cols: int):
    if layout == HEAD_MAJOR:
        row_stride = row_cols
        head_stride = page_size * row_cols
    elif layout == TOKEN_MAJOR:
        head_stride = row_cols
        row_stride = num_kv_heads * row_cols
    else:
        raise ValueError(layout)
    page_stride = num_kv_heads * page_size * row_cols
    return page_stride, head_stride, row_stride


def resident_pages(L: int, page_size: int, window: int, extra_page: bool) -> tuple[int, int]:
    """Logical pages [p0, p1) a request keeps resident.

    Whole context: every page up to the one holding position L-1.  Windowed:
    the pages overlapping [L-window, L), plus, when ``extra_page`` is set and
    one exists, the page before them (the resident pages may hold up to one
    page more than the window; pegainfer PR #1057, Description).
    """
    p1 = (L + page_size - 1) // page_size
    if window <= 0:
        return 0, p1
    lo = max(0, L - window)
    p0 = lo // page_size
    if extra_page and p0 > 0:
        p0 -= 1
    return p0, p1


def make_workload(seq_lens: Sequence[int], *, num_q_heads: int, num_kv_heads: int,
                  head_dim: int, page_size: int, window: int = 0, fmt: str = SPLIT,
                  rot_cols: int = 128, seed: int = 0, table_seed: Optional[int] = None,
                  layout: str = HEAD_MAJOR, spare_pages: int = 4, pad: str = "nan",
                  max_pages: Optional[int] = None, extra_page: bool = True,
                  scale: Optional[float] = None, num_rows: int = 1, kv_dtype: str = BF16,
                  k_scale: Optional[float] = None, v_scale: Optional[float] = None,
                  q_lens: Optional[Sequence[int]] = None) -> Workload:
    """Build a decode-step workload.

    Data is drawn per (request, logical page) in ascending order from ``seed``;
    physical placement comes from a permutation drawn from ``table_seed``
    (default ``seed + 1000``), so two workloads that differ only in
    ``table_seed`` hold the same logical rows at different physical pages.
    Slots outside a request's visible keys and unused pages hold ``pad``.
    ``num_rows`` > 1 gives every request a window of that many query rows (the last
    positions of the request), q shaped [B][rows][Hq][D].  ``kv_dtype`` picks the
    pool's element type; the dequantisation factors default to 1 (FP8: the
    FP8_K_SCALE / FP8_V_SCALE pair).  ``q_lens`` (prefill) gives every request its own
    number of query rows (0 .. L); q is then packed [sum(q_lens)][Hq][D].
    """
    seq_lens = [int(x) for x in seq_lens]
    B = len(seq_lens)
    D = head_dim
    if fmt == SPLIT:
        row_cols, k_off, v_off, rot = 2 * D, 0, D, 0
    elif fmt == FOLDED:
        row_cols, k_off, v_off, rot = rot_cols + D, 0, rot_cols, rot_cols
    else:
        raise ValueError(fmt)
    if kv_dtype not in KV_DTYPES:
        raise ValueError(kv_dtype)
    if k_scale is None:
        k_scale = FP8_K_SCALE if kv_dtype == FP8 else 1.0
    if v_scale is None:
        v_scale = FP8_V_SCALE if kv_dtype == FP8 else 1.0
    if max_pages is None:
        max_pages = max((L + page_size - 1) // page_size for L in seq_lens)
    if q_lens is not None:
        q_lens = [int(x) for x in q_lens]
        if len(q_lens) != B or any(n < 0 or n > L for n, L in zip(q_lens, seq_lens)):
            raise ValueError("q_lens must give 0 .. L rows per request")
        rows = [max(n, 1) for n in q_lens]
        num_rows = 1
    else:
        rows = [num_rows] * B
    if num_rows < 1 or any(L < n for L, n in zip(seq_lens, rows)):
        raise ValueError("every request needs at least num_rows keys")
    # the first row of a window sees keys [.., L - rows + 1): its window reaches furthest back
    spans = [resident_pages(L, page_size, window + n - 1 if window > 0 else 0, extra_page)
             for L, n in zip(seq_lens, rows)]
    needed = sum(p1 - p0 for p0, p1 in spans)
    num_pages = needed + spare_pages
    page_stride, head_stride, row_stride = _strides(layout, num_kv_heads, page_size, row_cols)

    gen = _gen(seed)
    tgen = _gen(seed + 1000 if table_seed is None else table_seed)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)

    if q_lens is not None:
        qshape = (sum(q_lens), num_q_heads, D)
    else:
        qshape = (B, num_q_heads, D) if num_rows == 1 else (B, num_rows, num_q_heads, D)
    q = torch.randn(*qshape, generator=gen, dtype=torch.float32).numpy()
    fold_w = None
    q_unfolded = None
    if fmt == FOLDED:
        fold_w = (torch.rand(D - rot, generator=gen, dtype=torch.float32) + 0.5).numpy()
        q_unfolded = q.copy()
        q = q.copy()
        q[..., rot:] = (q_unfolded[..., rot:] * fold_w).astype(np.float32)

    etype = KV_NUMPY[kv_dtype]
    padv = etype(PADS_BY_DTYPE[kv_dtype][pad])
    pool = np.full(num_pages * page_stride, padv, dtype=etype)
    k_cols = slice(k_off, k_off + (rot if fmt == FOLDED else D))
    perm = torch.randperm(num_pages, generator=tgen).numpy().astype(np.int32)
    table = np.full((B, max_pages), -1, dtype=np.int32)
    pool_pages = pool.reshape(num_pages, page_stride)

    k = 0
    for r, L in enumerate(seq_lens):
        p0, p1 = spans[r]
        lo = max(0, L - rows[r] + 1 - window) if window > 0 else 0
        for j in range(p0, p1):
            pid = int(perm[k]); k += 1
            table[r, j] = pid
            block = _normal_stored(gen, (num_kv_heads, page_size, row_cols), kv_dtype,
                                   k_scale, v_scale, k_cols)
            # positions of this page that are outside the visible range get the pad
            pos = j * page_size + np.arange(page_size)
            dead = (pos >= L) | (pos < lo)
            block[:, dead, :] = padv
            _store_page(pool_pages[pid], block, layout, num_kv_heads, page_size, row_cols)

    return Workload(batch=B, num_q_heads=num_q_heads, num_kv_heads=num_kv_heads,
                    head_dim=D, fmt=fmt, rot_cols=rot, page_size=page_size,
                    max_pages=max_pages, window=window, scale=scale, layout=layout,
                    num_pages=num_pages, row_cols=row_cols, page_stride=page_stride,
                    head_stride=head_stride, row_stride=row_stride, k_offset=k_off,
                    v_offset=v_off, q=q, pool=pool, table=table,
                    seq_lens=np.asarray(seq_lens, dtype=np.int32), fold_w=fold_w,
                    q_unfolded=q_unfolded, num_rows=num_rows, kv_dtype=kv_dtype,
                    k_scale=float(k_scale), v_scale=float(v_scale),
                    q_lens=None if q_lens is None else np.asarray(q_lens, dtype=np.int32))


def _store_page(dst: np.ndarray, block: np.ndarray, layout: str, hkv: int, ps: int, cols: int):
    if layout == HEAD_MAJOR:
        dst[:] = block.reshape(-1)
    else:
        dst[:] = block.transpose(1, 0, 2).reshape(-1)


def split_pair_of_folded(wl: Workload) -> Workload:
    """The split-row pool that a folded pool stands for.

    Row = [Krot | bf16(w * V[rot:]) | V]: the unrotated K columns are what the
    norm weight makes of V's columns, so the score against the folded row with
    the folded query equals the score against this row with the unfolded
    query, up to the bf16 rounding of w * V (pegainfer PR #1055, Description).
    """
    if wl.fmt != FOLDED:
        raise ValueError("need a folded workload")
    if wl.kv_dtype != BF16:
        raise ValueError("the split pair is defined for bf16 pools")
    D, rot = wl.head_dim, wl.rot_cols
    cols = 2 * D
    page_stride, head_stride, row_stride = _strides(wl.layout, wl.num_kv_heads, wl.page_size, cols)
    pool = np.empty(wl.num_pages * page_stride, dtype=np.uint16)
    src = wl.pool.reshape(wl.num_pages, -1)
    dst = pool.reshape(wl.num_pages, -1)
    for p in range(wl.num_pages):
        if wl.layout == HEAD_MAJOR:
            rows = src[p].reshape(wl.num_kv_heads, wl.page_size, wl.row_cols)
        else:
            rows = src[p].reshape(wl.page_size, wl.num_kv_heads, wl.row_cols).transpose(1, 0, 2)
        krot = rows[:, :, :rot]
        v = rows[:, :, rot:]
        vf = (v.astype(np.uint32) << 16).view(np.float32)
        kfold = f32_to_bf16_bits((vf[:, :, rot:] * wl.fold_w).astype(np.float32))
        out = np.concatenate([krot, kfold, v], axis=2)
        _store_page(dst[p], out, wl.layout, wl.num_kv_heads, wl.page_size, cols)
    return dataclasses.replace(wl, fmt=SPLIT, rot_cols=0, row_cols=cols, page_stride=page_stride,
                               head_stride=head_stride, row_stride=row_stride, k_offset=0,
                               v_offset=D, q=wl.q_unfolded.copy(), pool=pool)


# ---- the workloads the pages measure -------------------------------------------------

GLOBAL = dict(num_q_heads=32, num_kv_heads=4, head_dim=512, page_size=256)
SLIDING = dict(num_q_heads=32, num_kv_heads=16, head_dim=256, page_size=64, window=1024)


def tiny_ref(seed: int = 0, **kw) -> Workload:
    """1 token of decode over a 1024-token context, split rows, 4 pages drawn
    from a pool of 8 (the other 4 hold the pad), shuffled page table."""
    return make_workload([1024], **GLOBAL, seed=seed, **kw)


def global_decode(L: int, seed: int = 1, fmt: str = SPLIT, **kw) -> Workload:
    """Global-layer decode at context L (10,602 / 40,002 / 81,653 / 163,336)."""
    kw.setdefault("spare_pages", 1)
    return make_workload([L], **GLOBAL, fmt=fmt, seed=seed, **kw)


def global_streams(seed: int = 16, streams: int = 4, prompt: int = 9000, spread: int = 640,
                   fmt: str = SPLIT, **kw) -> Workload:
    """Global-layer decode of several concurrent streams: ``streams`` requests whose
    contexts are a ``prompt``-token prompt plus 0 .. spread - 1 decoded tokens (seeded),
    the four-stream, 9k-prompt serving case."""
    g = _gen(seed + 77)
    lens = (prompt + torch.randint(0, spread, (streams,), generator=g)).tolist()
    kw.setdefault("spare_pages", 1)
    return make_workload(lens, **GLOBAL, fmt=fmt, seed=seed, **kw)


def global_prefill(n: int, context: int = 0, seed: int = 11, fmt: str = SPLIT, **kw) -> Workload:
    """Global-layer prefill: a prompt of n new rows after ``context`` earlier tokens,
    one request (10,602 rows: the prompt length the pages measure)."""
    kw.setdefault("spare_pages", 1)
    return make_workload([context + n], **GLOBAL, fmt=fmt, seed=seed, q_lens=[n], **kw)


def sliding_prefill(seed: int = 12, batch: int = 16, max_len: int = 4096, **kw) -> Workload:
    """Sliding-layer varlen prefill: 16 ragged prompts, lengths drawn uniformly from
    1..4096, window 1024, every row of every prompt new."""
    g = _gen(seed + 77)
    lens = (torch.randint(1, max_len + 1, (batch,), generator=g)).tolist()
    kw.setdefault("max_pages", max_len // SLIDING["page_size"])
    return make_workload(lens, **SLIDING, seed=seed, q_lens=lens, **kw)


def sliding_batch(seed: int = 4, batch: int = 16, max_len: int = 4096, **kw) -> Workload:
    """16 ragged requests, lengths drawn uniformly from 1..4096, window 1024."""
    g = _gen(seed + 77)
    lens = (torch.randint(1, max_len + 1, (batch,), generator=g)).tolist()
    kw.setdefault("max_pages", max_len // SLIDING["page_size"])
    return make_workload(lens, **SLIDING, seed=seed, **kw)


def tree_masks(parents: np.ndarray) -> np.ndarray:
    """uint64 [B][rows] masks of a forest of window rows given by parent indices
    (parents[r][i] < i, or -1): bit j of row i is set when j is i or one of its
    ancestors.  Rows are at most 64."""
    parents = np.asarray(parents, dtype=np.int64)
    B, n = parents.shape
    if n > 64:
        raise ValueError("at most 64 window rows")
    masks = np.zeros((B, n), dtype=np.uint64)
    for r in range(B):
        for i in range(n):
            p = int(parents[r, i])
            if not -1 <= p < i:
                raise ValueError("a parent must be an earlier row or -1")
            masks[r, i] = np.uint64(1 << i) | (masks[r, p] if p >= 0 else np.uint64(0))
    return masks


def random_parents(batch: int, rows: int, seed: int) -> np.ndarray:
    """Seeded random forests: row 0 hangs off the prefix, row i > 0 off a uniformly
    drawn earlier row (or, one time in eight, off the prefix as a new root)."""
    rng = np.random.default_rng(seed)
    parents = np.full((batch, rows), -1, dtype=np.int32)
    for r in range(batch):
        for i in range(1, rows):
            parents[r, i] = -1 if rng.random() < 0.125 else int(rng.integers(0, i))
    return parents


def set_tree(wl: Workload, parents: np.ndarray) -> Workload:
    """Attach a tree (parent indices per request) and its masks to a multi-row workload."""
    parents = np.asarray(parents, dtype=np.int32)
    if parents.shape != (wl.batch, wl.num_rows):
        raise ValueError("parents must be [batch][rows]")
    wl.tree_parents = parents
    wl.row_masks = tree_masks(parents)
    return wl

