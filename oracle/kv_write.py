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
start_pos[r] + i.

Other stored element types (the gem design note, "Fixed production shape", names F32 KV
as its production type and F16 / quantised KV as further axes; the decode path reads
stored values times one dequantisation factor per tensor, K = stored * k_scale and
V = stored * v_scale).  Reading taken for the write: a value x is first divided by its
factor (one float32 division, rounded to nearest), then encoded:
  * f32: the quotient as is;
  * f16: IEEE binary16, rounded to nearest with ties to even (overflow gives infinity);
  * FP8 E4M3 (OCP): the representable value nearest to the quotient, a tie going to the
    code whose mantissa is even; magnitudes beyond the largest finite value 448
    (infinities included) saturate to +-448; NaN gives the NaN code of its sign; the
    sign of a result that rounds to zero is kept (-0 is 0x80).
With factors of 1 (every pool but FP8 by default) the division is exact.  The folded query is q'[d] = q[d] for d < rot and fl32(q[d] * w[d - rot])
otherwise (one float32 product, rounded to nearest).
"""
from __future__ import annotations

import numpy as np

__all__ = ["f32_to_bf16_rne", "f32_to_f16_rne", "f32_to_e4m3", "encode_stored", "write_rows",
           "fold_query"]


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


def f32_to_f16_rne(x: np.ndarray) -> np.ndarray:
    """Round binary32 values to IEEE binary16 (nearest, ties to even; overflow to infinity);
    returns the 16-bit patterns.  numpy's half conversion is the rounding step."""
    with np.errstate(over="ignore"):  # overflow to infinity is the defined result
        return np.ascontiguousarray(x, dtype=np.float32).astype(np.float16).view(np.uint16)


# Non-negative finite E4M3 values in code order (codes 0x00 .. 0x7E: 0 .. 448, increasing).
def _e4m3_grid() -> np.ndarray:
    from .attention import e4m3_bits_to_f64
    return e4m3_bits_to_f64(np.arange(0x7F, dtype=np.uint8))


def f32_to_e4m3(x: np.ndarray) -> np.ndarray:
    """Encode binary32 values as OCP E4M3 codes: the nearest representable value, ties to
    the even code (even mantissa), saturating beyond 448 (infinities too); NaN gives
    S.1111.111; the sign is kept for values that round to zero."""
    x = np.asarray(x, dtype=np.float32)
    grid = _e4m3_grid()
    a = np.abs(x.astype(np.float64))
    sign = np.signbit(x).astype(np.uint8) << 7
    with np.errstate(invalid="ignore"):
        i = np.clip(np.searchsorted(grid, np.where(np.isnan(a), 0.0, a), side="right") - 1, 0, 0x7E)
    lo = grid[i]
    hi = grid[np.minimum(i + 1, 0x7E)]
    below, above = a - lo, hi - a
    up = (i < 0x7E) & ((above < below) | ((above == below) & (i % 2 == 1)))
    code = (i + up).astype(np.uint8) | sign
    return np.where(np.isnan(x), sign | np.uint8(0x7F), code).astype(np.uint8)


def encode_stored(x: np.ndarray, kv_dtype: str, factor: float = 1.0) -> np.ndarray:
    """Stored bit patterns of float32 values written into a pool of the given element
    type with the given dequantisation factor (x / factor in float32, then encoded)."""
    q = np.ascontiguousarray(x, dtype=np.float32) / np.float32(factor)
    if kv_dtype == "bf16":
        return f32_to_bf16_rne(q)
    if kv_dtype == "f16":
        return f32_to_f16_rne(q)
    if kv_dtype == "fp8_e4m3":
        return f32_to_e4m3(q)
    if kv_dtype == "f32":
        return q.view(np.uint32)
    raise ValueError(f"unknown element type {kv_dtype}")


def write_rows(wl, k: np.ndarray, v: np.ndarray, start_pos: np.ndarray) -> np.ndarray:
    """The pool after writing new rows; returns a new flat array of the pool's bit patterns
    (element type wl.kv_dtype, factors wl.k_scale / wl.v_scale; bf16 with factors 1 when the
    workload does not say).

    k : float32 [B][n][Hkv][kc] with kc = D (split) or rot (folded)
    v : float32 [B][n][Hkv][D]
    Element (page p, KV head g, slot s, column c) is pool[p*page_stride + g*head_stride +
    s*row_stride + c]; logical position j of request r is slot j % page_size of page
    table[r][j // page_size].
    """
    pool = wl.pool.copy()
    B, n, hkv, kc = k.shape
    D = wl.head_dim
    dt = getattr(wl, "kv_dtype", "bf16")
    ks = float(getattr(wl, "k_scale", 1.0))
    vs = float(getattr(wl, "v_scale", 1.0))
    for r in range(B):
        for i in range(n):
            j = int(start_pos[r]) + i
            page = int(wl.table[r][j // wl.page_size])
            if page < 0 or page >= wl.num_pages:
                raise IndexError("page table points outside the pool")
            for g in range(hkv):
                base = page * wl.page_stride + g * wl.head_stride + (j % wl.page_size) * wl.row_stride
                pool[base + wl.k_offset: base + wl.k_offset + kc] = encode_stored(k[r, i, g], dt, ks)
                pool[base + wl.v_offset: base + wl.v_offset + D] = encode_stored(v[r, i, g], dt, vs)
    return pool


def fold_query(q: np.ndarray, w: np.ndarray, rot: int) -> np.ndarray:
    """q' = q with the columns from `rot` on multiplied by the norm weight (float32)."""
    q = np.asarray(q, dtype=np.float32)
    out = q.copy()
    out[..., rot:] = (q[..., rot:] * np.asarray(w, dtype=np.float32)).astype(np.float32)
    return out
