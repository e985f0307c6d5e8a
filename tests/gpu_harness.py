"""Run one decode step of a synth.Workload through the C ABI on cuda:0."""
from __future__ import annotations

import sys

import numpy as np
import torch

import paged_split_kv_02_amd as K

GUARD = 4096          # float32 sentinels on each side of `out`
WS_GUARD = 1 << 16    # bytes of sentinel past the workspace
SENTINEL = 0x7FBADBAD  # an unusual NaN bit pattern


def note(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def fnv1a(a: np.ndarray) -> int:
    """FNV-1a (64-bit) over the bytes of an array."""
    h = 0xCBF29CE484222325
    for byte in np.ascontiguousarray(a).view(np.uint8).tobytes():
        h ^= byte
        h = (h * 0x100000001B3) & 0xFFFFFFFFFFFFFFFF
    return h


class Device:
    """Workload buffers resident on the GPU plus a plan."""

    def __init__(self, wl, num_chunks=0, merge_group=0, seq_lens_dev=None):
        self.wl = wl
        dev = torch.device("cuda:0")
        self.desc = K.make_desc(**wl.desc_fields(num_chunks, merge_group))
        self.plan = K.attn_decode_plan(self.desc, wl.seq_lens)
        self.q = torch.from_numpy(np.ascontiguousarray(wl.q, dtype=np.float32)).to(dev)
        self.pool = torch.from_numpy(wl.pool.view(np.uint8)).to(dev)
        self.table = torch.from_numpy(wl.table).to(dev)
        lens = wl.seq_lens if seq_lens_dev is None else np.asarray(seq_lens_dev, dtype=np.int32)
        self.lens = torch.from_numpy(lens).to(dev)
        nws = int(self.plan.workspace_bytes)
        self.ws_buf = torch.full((nws + WS_GUARD,), 0xA5, dtype=torch.uint8, device=dev)
        self.ws = self.ws_buf[:nws]
        n = wl.batch * wl.num_rows * wl.num_q_heads * wl.head_dim
        self.out_buf = torch.full((n + 2 * GUARD,), 0, dtype=torch.int32, device=dev)
        self.out_buf.fill_(SENTINEL)
        self.out_f = self.out_buf.view(torch.float32)
        self.out = self.out_f[GUARD:GUARD + n]

    def step(self, stream=None):
        K.attn_decode_split(self.plan, self.q, self.pool, self.table, self.lens, self.ws,
                            stream=stream)
        K.attn_decode_merge(self.plan, self.ws, self.out, stream=stream)

    def run(self) -> np.ndarray:
        self.step()
        torch.cuda.synchronize()
        return self.result()

    def result(self) -> np.ndarray:
        wl = self.wl
        shape = (wl.batch, wl.num_q_heads, wl.head_dim) if wl.num_rows == 1 else \
            (wl.batch, wl.num_rows, wl.num_q_heads, wl.head_dim)
        return self.out.cpu().numpy().reshape(shape).copy()

    def guards_intact(self) -> bool:
        ob = self.out_buf.cpu().numpy()
        wsg = self.ws_buf[int(self.plan.workspace_bytes):].cpu().numpy()
        return (np.all(ob[:GUARD] == SENTINEL) and np.all(ob[-GUARD:] == SENTINEL)
                and np.all(wsg == 0xA5))

    def partials(self):
        """(m, l, o) chunk states as numpy: [B][Hq][n], [B][Hq][n], [B][Hq][n][D]."""
        p, wl = self.plan, self.wl
        ws = self.ws.cpu().numpy()
        B, H, n, D = wl.batch * wl.num_rows, wl.num_q_heads, p.num_chunks, wl.head_dim

        def region(off, count):
            return ws[off:off + 4 * count].view(np.float32)
        m = region(p.off_part_m, B * H * n).reshape(B, H, n)
        l = region(p.off_part_l, B * H * n).reshape(B, H, n)
        o = region(p.off_part_o, B * H * n * D).reshape(B, H, n, D)
        return m, l, o

    def chunk_ranges(self, r):
        p = self.plan
        L = int(self.wl.seq_lens[r])
        first_hi = L - self.wl.num_rows + 1
        lo = max(0, first_hi - p.desc.window) if p.desc.window > 0 else 0
        start = lo // p.tile * p.tile
        return plan_chunk_ranges(p, start)


def plan_chunk_ranges(p, start: int) -> list:
    """[a, b) of every chunk of a plan from a request's start: even-numbered chunks hold
    chunk_len keys, odd-numbered ones chunk_len_odd (the header's chunk layout)."""
    out, a = [], start
    for c in range(p.num_chunks):
        n = p.chunk_len if c % 2 == 0 else p.chunk_len_odd
        out.append((a, a + n))
        a += n
    return out


def compare(got: np.ndarray, ref: np.ndarray) -> dict:
    err = got.astype(np.float64) - ref
    return dict(max_abs=float(np.max(np.abs(err))),
                max_ref=float(np.max(np.abs(ref))),
                nmse=float(np.sum(err ** 2) / np.sum(ref ** 2)),
                corr=float(np.corrcoef(got.reshape(-1).astype(np.float64), ref.reshape(-1))[0, 1]),
                finite=bool(np.all(np.isfinite(got))))
