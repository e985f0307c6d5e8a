"""Reference for the step that feeds the decode path: writing new K/V rows into pages and
folding K's norm weight into the query.

TEST INFRASTRUCTURE ONLY (see the package docstring).

* TensorFold PR #1619, body: a kernel copies each forward's k/v rows into the pages of
  the pool (one launch per global layer), so the cache bits equal the linear cache's.
* pegainfer PR #1055, Description: the hd512 prep writes either row format; the folded
  row keeps only the rotated K columns and V in full, and K's norm weight is folded into
  the query at prep time.

Reading taken: the new rows arrive as float32 (the projection output) and are stored as
bf16 rounded to nearest, ties to even; the split row is [k[0:D] | v[0:D]], the folded row
[k_rot[0:rot] | v[0:D]]; request r's i-th new token goes to logical position
start_pos[r] + i.  The folded query is q'[d] = q[d] for d < rot and fl32(q[d] * w[d - rot])
otherwise (one float32 product, rounded to nearest).
"""
from __future__ import annotations

import numpy as np

__all__ = ["f32_to_bf16_rne", "write_rows", "fold_query"]


def f32_to_bf16_rne(x: np.ndarray) -> np.ndarray:
    """Round binary32 values to bfloat16 (nearest, ties to even); returns the 16-bit patterns.

    bf16 keeps the upper 16 bits of a binary32.  Rounding adds half an ulp of the kept
    part (0x7FFF) plus the kept part's lowest bit, so an exact half rounds to the even
    neighbour; NaN maps to a quiet NaN of the same sign.
    """
    bits = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (bits >> 16) & 1
    rounded = ((bits + 0x7FFF + lsb) >> 16).astype(np.uint16)
    nan = np.isnan(np.asarray(x, dtype=np.float32))
    quiet = ((bits >> 16).astype(np.uint16) & np.uint16(0x8000)) | np.uint16(0x7FC0)
    return np.where(nan, quiet, rounded).astype(np.uint16)


def write_rows(wl, k: np.ndarray, v: np.ndarray, start_pos: np.ndarray) -> np.ndarray:
    """The pool after writing new rows; returns a new flat uint16 array.

    k : float32 [B][n][Hkv][kc] with kc = D (split) or rot (folded)
    v : float32 [B][n][Hkv][D]
    Element (page p, KV head g, slot s, column c) is pool[p*page_stride + g*head_stride +
    s*row_stride + c]; logical position j of request r is slot j % page_size of page
    table[r][j // page_size].
    """
    pool = wl.pool.copy()
    B, n, hkv, kc = k.shape
    D = wl.head_dim
    for r in range(B):
        for i in range(n):
            j = int(start_pos[r]) + i
            page = int(wl.table[r][j // wl.page_size])
            if page < 0 or page >= wl.num_pages:
                raise IndexError("page table points outside the pool")
            for g in range(hkv):
                base = page * wl.page_stride + g * wl.head_stride + (j % wl.page_size) * wl.row_stride
                pool[base + wl.k_offset: base + wl.k_offset + kc] = f32_to_bf16_rne(k[r, i, g])
                pool[base + wl.v_offset: base + wl.v_offset + D] = f32_to_bf16_rne(v[r, i, g])
    return pool


def fold_query(q: np.ndarray, w: np.ndarray, rot: int) -> np.ndarray:
    """q' = q with the columns from `rot` on multiplied by the norm weight (float32)."""
    q = np.asarray(q, dtype=np.float32)
    out = q.copy()
    out[..., rot:] = (q[..., rot:] * np.asarray(w, dtype=np.float32)).astype(np.float32)
    return out
