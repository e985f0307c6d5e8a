"""Paged split-KV decode attention for MI355X (gfx950).

A thin ctypes binding of the C ABI in include/attn_decode.h: the same four
calls, argument marshalling only.  Every step of the computation runs in the
HIP library; if it is missing or cannot be loaded, importing this package
raises.  Device buffers are passed as torch tensors (their data_ptr) or as raw
integer addresses; ``stream`` defaults to torch's current stream.
"""
from __future__ import annotations

import ctypes
import os

from . import build as _build

__all__ = ["AttnDecodeDesc", "AttnDecodePlan", "AttnDecodeError", "attn_decode_plan",
           "attn_decode_split", "attn_decode_split_tree", "attn_decode_merge",
           "attn_decode_status_string", "make_desc",
           "attn_kv_write", "attn_query_fold", "AttnPrefillPlan", "attn_prefill_plan",
           "attn_prefill", "attn_stream_read", "STREAM_READ_GROUPS",
           "attn_decode_step_noalloc", "NOALLOC_SCRATCH_BYTES",
           "ATTN_KV_SPLIT", "ATTN_KV_FOLDED", "ATTN_KV_BF16", "ATTN_KV_F16", "ATTN_KV_FP8_E4M3",
           "ATTN_KV_F32", "STATUS", "LIB_PATH", "SYMBOLS"]

ATTN_KV_SPLIT = 0
ATTN_KV_FOLDED = 1
ATTN_KV_BF16 = 0
ATTN_KV_F16 = 1
ATTN_KV_FP8_E4M3 = 2
ATTN_KV_F32 = 3
STATUS = {"ATTN_OK": 0, "ATTN_E_INVALID_ARG": -1, "ATTN_E_UNSUPPORTED": -2,
          "ATTN_E_PAST_PAGES": -3, "ATTN_E_OVERFLOW": -4, "ATTN_E_WORKSPACE": -5,
          "ATTN_E_PLAN": -6, "ATTN_E_LAUNCH": -7, "ATTN_E_SCRATCH": -8}
SYMBOLS = ("attn_decode_plan", "attn_decode_split", "attn_decode_split_tree", "attn_decode_merge",
           "attn_decode_status_string", "attn_kv_write", "attn_query_fold",
           "attn_prefill_plan", "attn_prefill", "attn_stream_read", "attn_decode_step_noalloc")
STREAM_READ_GROUPS = 2048  # ATTN_STREAM_READ_GROUPS
NOALLOC_SCRATCH_BYTES = 32 << 20  # ATTN_NOALLOC_SCRATCH_BYTES
LIB_PATH = _build.LIB


class AttnDecodeDesc(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("num_q_heads", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("format", ctypes.c_int32), ("rot_cols", ctypes.c_int32),
                ("page_size", ctypes.c_int32), ("max_pages_per_seq", ctypes.c_int32),
                ("window", ctypes.c_int32), ("num_chunks", ctypes.c_int32),
                ("merge_group", ctypes.c_int32), ("num_rows", ctypes.c_int32),
                ("kv_dtype", ctypes.c_int32), ("scale", ctypes.c_float),
                ("k_scale", ctypes.c_float), ("v_scale", ctypes.c_float),
                ("num_pages", ctypes.c_int64), ("page_stride", ctypes.c_int64),
                ("head_stride", ctypes.c_int64), ("row_stride", ctypes.c_int64),
                ("k_offset", ctypes.c_int64), ("v_offset", ctypes.c_int64)]


class AttnDecodePlan(ctypes.Structure):
    _fields_ = [("magic", ctypes.c_uint64), ("desc", AttnDecodeDesc),
                ("group_size", ctypes.c_int32), ("tile", ctypes.c_int32),
                ("chunk_len", ctypes.c_int32), ("chunk_len_odd", ctypes.c_int32),
                ("num_chunks", ctypes.c_int32),
                ("merge_group", ctypes.c_int32), ("num_groups", ctypes.c_int32),
                ("max_span", ctypes.c_int32), ("num_rows", ctypes.c_int32),
                ("row_groups", ctypes.c_int32), ("grid_x", ctypes.c_int32),
                ("off_part_m", ctypes.c_uint64), ("off_part_l", ctypes.c_uint64),
                ("off_part_o", ctypes.c_uint64), ("workspace_bytes", ctypes.c_uint64)]


class AttnPrefillPlan(ctypes.Structure):
    _fields_ = [("magic", ctypes.c_uint64), ("desc", AttnDecodeDesc),
                ("group_size", ctypes.c_int32), ("key_tile", ctypes.c_int32),
                ("row_tile", ctypes.c_int32), ("total_rows", ctypes.c_int32),
                ("max_rows", ctypes.c_int32), ("grid_x", ctypes.c_int32)]


class AttnDecodeError(RuntimeError):
    def __init__(self, call: str, status: int):
        self.status = status
        super().__init__(f"{call}: {attn_decode_status_string(status)} ({status})")


def _load() -> ctypes.CDLL:
    # A library missing, or built from other sources than those in the tree, is rebuilt
    # first: a stale library is never loaded.
    if not _build.is_current():
        _build.build()
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.c_void_p
    lib.attn_decode_plan.argtypes = [ctypes.POINTER(AttnDecodeDesc), P, ctypes.POINTER(AttnDecodePlan)]
    lib.attn_decode_plan.restype = ctypes.c_int
    lib.attn_decode_split.argtypes = [ctypes.POINTER(AttnDecodePlan), P, P, P, P, P, ctypes.c_size_t, P]
    lib.attn_decode_split.restype = ctypes.c_int
    lib.attn_decode_split_tree.argtypes = [ctypes.POINTER(AttnDecodePlan), P, P, P, P, P, P,
                                           ctypes.c_size_t, P]
    lib.attn_decode_split_tree.restype = ctypes.c_int
    lib.attn_decode_merge.argtypes = [ctypes.POINTER(AttnDecodePlan), P, ctypes.c_size_t, P, P]
    lib.attn_decode_merge.restype = ctypes.c_int
    lib.attn_kv_write.argtypes = [ctypes.POINTER(AttnDecodePlan), P, P, ctypes.c_int32, P, P, P, P, P]
    lib.attn_kv_write.restype = ctypes.c_int
    lib.attn_query_fold.argtypes = [ctypes.POINTER(AttnDecodePlan), P, P, P, P]
    lib.attn_query_fold.restype = ctypes.c_int
    lib.attn_prefill_plan.argtypes = [ctypes.POINTER(AttnDecodeDesc), P, P,
                                      ctypes.POINTER(AttnPrefillPlan)]
    lib.attn_prefill_plan.restype = ctypes.c_int
    lib.attn_prefill.argtypes = [ctypes.POINTER(AttnPrefillPlan), P, P, P, P, P, P, P]
    lib.attn_prefill.restype = ctypes.c_int
    lib.attn_stream_read.argtypes = [P, ctypes.c_size_t, P, P]
    lib.attn_stream_read.restype = ctypes.c_int
    lib.attn_decode_step_noalloc.argtypes = [ctypes.POINTER(AttnDecodePlan), P, P, P, P, P, P, P]
    lib.attn_decode_step_noalloc.restype = ctypes.c_int
    lib.attn_decode_status_string.argtypes = [ctypes.c_int]
    lib.attn_decode_status_string.restype = ctypes.c_char_p
    return lib


_lib = _load()


def _ptr(x) -> int:
    """Device/host address of a torch tensor, numpy array or raw integer."""
    if x is None:
        return 0
    if isinstance(x, int):
        return x
    if hasattr(x, "data_ptr"):
        return int(x.data_ptr())
    if hasattr(x, "ctypes"):
        return int(x.ctypes.data)
    raise TypeError(f"cannot take the address of {type(x).__name__}")


def _nbytes(x) -> int:
    if hasattr(x, "untyped_storage"):
        return int(x.numel() * x.element_size())
    return int(x.nbytes)


def _stream(stream) -> int:
    if stream is None:
        import torch
        return int(torch.cuda.current_stream().cuda_stream)
    if hasattr(stream, "cuda_stream"):
        return int(stream.cuda_stream)
    return int(stream)


def make_desc(**fields) -> AttnDecodeDesc:
    """An attn_decode_desc from keyword fields (missing fields are 0, except the
    dequantisation factors k_scale and v_scale, which default to 1)."""
    d = AttnDecodeDesc()
    d.k_scale = 1.0
    d.v_scale = 1.0
    for k, v in fields.items():
        setattr(d, k, v)
    return d


def attn_decode_status_string(status: int) -> str:
    return _lib.attn_decode_status_string(int(status)).decode()


def attn_decode_plan(desc: AttnDecodeDesc, seq_lens_host) -> AttnDecodePlan:
    """Validate and plan; ``seq_lens_host`` is a host int32 array (numpy) of length batch."""
    import numpy as np
    lens = np.ascontiguousarray(seq_lens_host, dtype=np.int32)
    if lens.ndim != 1 or lens.size != desc.batch:
        raise ValueError("seq_lens needs batch entries")
    plan = AttnDecodePlan()
    rc = _lib.attn_decode_plan(ctypes.byref(desc), lens.ctypes.data, ctypes.byref(plan))
    if rc != 0:
        raise AttnDecodeError("attn_decode_plan", rc)
    return plan


def attn_decode_split(plan: AttnDecodePlan, q, kv_pool, page_table, seq_lens, workspace,
                      workspace_bytes=None, stream=None) -> None:
    nbytes = _nbytes(workspace) if workspace_bytes is None else int(workspace_bytes)
    rc = _lib.attn_decode_split(ctypes.byref(plan), _ptr(q), _ptr(kv_pool), _ptr(page_table),
                                _ptr(seq_lens), _ptr(workspace), nbytes, _stream(stream))
    if rc != 0:
        raise AttnDecodeError("attn_decode_split", rc)


def attn_decode_split_tree(plan: AttnDecodePlan, q, kv_pool, page_table, seq_lens, row_masks,
                           workspace, workspace_bytes=None, stream=None) -> None:
    """attn_decode_split for a window of rows forming a tree: row_masks is a device
    uint64 [batch][rows] (int64 tensors are taken as the same bits)."""
    nbytes = _nbytes(workspace) if workspace_bytes is None else int(workspace_bytes)
    rc = _lib.attn_decode_split_tree(ctypes.byref(plan), _ptr(q), _ptr(kv_pool),
                                     _ptr(page_table), _ptr(seq_lens), _ptr(row_masks),
                                     _ptr(workspace), nbytes, _stream(stream))
    if rc != 0:
        raise AttnDecodeError("attn_decode_split_tree", rc)


def attn_decode_merge(plan: AttnDecodePlan, workspace, out, workspace_bytes=None,
                      stream=None) -> None:
    nbytes = _nbytes(workspace) if workspace_bytes is None else int(workspace_bytes)
    rc = _lib.attn_decode_merge(ctypes.byref(plan), _ptr(workspace), nbytes, _ptr(out),
                                _stream(stream))
    if rc != 0:
        raise AttnDecodeError("attn_decode_merge", rc)


def attn_decode_step_noalloc(plan: AttnDecodePlan, q, kv_pool, page_table, seq_lens, out,
                             row_masks=None, stream=None) -> None:
    """A whole decode step (split, or split_tree with row_masks, then merge) with the chunk
    states in the library's static per-GPU array: no workspace argument, nothing
    allocated.  Calls that overlap on one GPU race (they share the array)."""
    rc = _lib.attn_decode_step_noalloc(ctypes.byref(plan), _ptr(q), _ptr(kv_pool),
                                       _ptr(page_table), _ptr(seq_lens), _ptr(row_masks),
                                       _ptr(out), _stream(stream))
    if rc != 0:
        raise AttnDecodeError("attn_decode_step_noalloc", rc)


def attn_kv_write(plan: AttnDecodePlan, k, v, num_new: int, start_pos, kv_pool, page_table,
                  bad_rows=None, stream=None) -> None:
    rc = _lib.attn_kv_write(ctypes.byref(plan), _ptr(k), _ptr(v), int(num_new), _ptr(start_pos),
                            _ptr(kv_pool), _ptr(page_table), _ptr(bad_rows), _stream(stream))
    if rc != 0:
        raise AttnDecodeError("attn_kv_write", rc)


def attn_prefill_plan(desc: AttnDecodeDesc, seq_lens_host, q_starts_host) -> AttnPrefillPlan:
    """Validate and plan a prefill; host int32 arrays of length batch and batch + 1."""
    import numpy as np
    lens = np.ascontiguousarray(seq_lens_host, dtype=np.int32)
    starts = np.ascontiguousarray(q_starts_host, dtype=np.int32)
    if lens.size != desc.batch or starts.size != desc.batch + 1:
        raise ValueError("seq_lens needs batch entries and q_starts batch + 1")
    plan = AttnPrefillPlan()
    rc = _lib.attn_prefill_plan(ctypes.byref(desc), lens.ctypes.data, starts.ctypes.data,
                                ctypes.byref(plan))
    if rc != 0:
        raise AttnDecodeError("attn_prefill_plan", rc)
    return plan


def attn_prefill(plan: AttnPrefillPlan, q, kv_pool, page_table, seq_lens, q_starts, out,
                 stream=None) -> None:
    rc = _lib.attn_prefill(ctypes.byref(plan), _ptr(q), _ptr(kv_pool), _ptr(page_table),
                           _ptr(seq_lens), _ptr(q_starts), _ptr(out), _stream(stream))
    if rc != 0:
        raise AttnDecodeError("attn_prefill", rc)


def attn_stream_read(buf, nbytes: int, partial, stream=None) -> None:
    """Measurement aid: read ``nbytes`` of ``buf`` once (the read ceiling a decode step is
    compared against); ``partial`` (uint32 [STREAM_READ_GROUPS][4]) receives per-workgroup
    XORs of the 16-byte words read."""
    rc = _lib.attn_stream_read(_ptr(buf), int(nbytes), _ptr(partial), _stream(stream))
    if rc != 0:
        raise AttnDecodeError("attn_stream_read", rc)


def attn_query_fold(plan: AttnDecodePlan, q, norm_w, q_out, stream=None) -> None:
    rc = _lib.attn_query_fold(ctypes.byref(plan), _ptr(q), _ptr(norm_w), _ptr(q_out),
                              _stream(stream))
    if rc != 0:
        raise AttnDecodeError("attn_query_fold", rc)

