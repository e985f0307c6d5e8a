"""Benchmark: one decode step of paged split-KV attention on one MI355X.

A step is the whole hot path for one global-layer decode token: attn_decode_split
(page-table gather, K/V streaming, scores, online softmax, PV, partial write)
followed by attn_decode_merge (level-1 and level-2 merge, O / S), at 163,336
tokens of context, 32 query / 4 KV heads, head dim 512, split 1024-column rows
in pages of 256 with a shuffled page table.  Inputs are synthetic N(0, 1) data
already resident in HBM when timing starts.

Prints one JSON line.  `value` is effective GB/s: K/V row bytes the step must
read divided by the step time.  `roofline` reports the partial kernel's own
algorithmic bytes over its average duration (HIP events on its stream).
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode-attention µs/step + effective HBM GB/s (% peak) at 163K ctx, hd512"
HBM_PEAK_GBS = 8000.0
BF16_MFMA_PEAK_TFLOPS = 2500.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "pmc_traffic_global163k_split.txt")


def parse_args():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--context", type=int, default=163336)
    ap.add_argument("--fmt", choices=["split", "folded"], default="split")
    ap.add_argument("--num-chunks", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-variants", action="store_true")
    ap.add_argument("--variants", default="",
                    help="comma-separated substrings: time only the variants whose names hold one")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (reference kernel for counters)")
    return ap.parse_args()


def kernel_source_digest() -> str:
    import hashlib
    h = hashlib.sha256()
    for name in ("attn_decode.hip", "plan.cpp", "plan_internal.h"):
        with open(os.path.join(ROOT, "paged_split_kv_02_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def read_traffic(launch_bytes: int):
    """HBM bytes per partial-kernel launch from the committed counter summary, if it was
    taken on the current kernel source (else None)."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    kv = {}
    with open(TRAFFIC_FILE) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
    if kv.get("kernel_source_digest") != kernel_source_digest():
        return None
    try:
        return int(float(kv["hbm_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


class Resident:
    """A workload's buffers on the GPU and its plan."""

    def __init__(self, wl, num_chunks=0):
        import numpy as np
        import torch
        import paged_split_kv_02_amd as K
        dev = torch.device("cuda:0")
        self.wl = wl
        self.K = K
        self.plan = K.attn_decode_plan(K.make_desc(**wl.desc_fields(num_chunks)), wl.seq_lens)
        self.q = torch.from_numpy(np.ascontiguousarray(wl.q, dtype=np.float32)).to(dev)
        self.pool = torch.from_numpy(wl.pool.view(np.uint8)).to(dev)
        self.table = torch.from_numpy(wl.table).to(dev)
        self.lens = torch.from_numpy(wl.seq_lens).to(dev)
        self.ws = torch.empty(int(self.plan.workspace_bytes), dtype=torch.uint8, device=dev)
        self.out = torch.empty(wl.batch * wl.num_rows, wl.num_q_heads, wl.head_dim,
                               dtype=torch.float32, device=dev)
        self.masks = None
        if getattr(wl, "row_masks", None) is not None:   # tree attention over the rows
            self.masks = torch.from_numpy(np.ascontiguousarray(wl.row_masks).view(np.int64)).to(dev)

    def split(self):
        if self.masks is not None:
            self.K.attn_decode_split_tree(self.plan, self.q, self.pool, self.table, self.lens,
                                          self.masks, self.ws)
            return
        self.K.attn_decode_split(self.plan, self.q, self.pool, self.table, self.lens, self.ws)

    def merge(self):
        self.K.attn_decode_merge(self.plan, self.ws, self.out)

    def kernel_bytes(self) -> int:
        """Algorithmic bytes of one partial-kernel launch: K/V rows read, q, page-table
        entries, and the chunk states written."""
        wl, p = self.wl, self.plan
        pages = sum(-(-int(L) // wl.page_size) for L in wl.seq_lens)
        states = wl.batch * wl.num_rows * wl.num_q_heads * p.num_chunks
        return (wl.kv_bytes() + wl.q.size * 4 + pages * 4 + states * (wl.head_dim + 2) * 4)


def time_steps(res, steps, warmup, flush=None):
    """Time `steps` decode steps (split + merge).

    Without ``flush``: region A brackets all steps with one pair of events (the
    step time); region B repeats the steps with events around each partial-kernel
    launch (its duration, for the roofline).  With ``flush`` (inputs that fit the
    256 MB infinity cache): every step is preceded by an untimed 1 GiB write and
    timed on its own (two events around split + merge), alternating with a partial-kernel
    launch timed on its own after a flush of its own.
    """
    import torch
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        res.split()
        res.merge()
    torch.cuda.synchronize()
    E = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    if flush is None:
        first, last = E(), E()
        t0 = time.perf_counter()
        first.record(stream)
        for _ in range(steps):
            res.split()
            res.merge()
        last.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        total_ms = first.elapsed_time(last)
        ev = [(E(), E(), E()) for _ in range(steps)]
        for a, b, c in ev:
            a.record(stream)
            res.split()
            b.record(stream)
            res.merge()
            c.record(stream)
        torch.cuda.synchronize()
        split_ms = [a.elapsed_time(b) for a, b, _ in ev]
        each_step_ms = [a.elapsed_time(c) for a, _, c in ev]
        return dict(total_ms=total_ms, wall_s=wall, split_ms=split_ms,
                    step_ms=[total_ms / steps] * steps, each_step_ms=each_step_ms)
    # Alternating: a step bracketed by two events only (split and merge back to back, as a
    # caller runs them), then a partial-kernel launch bracketed on its own.
    step_ms, split_ms = [], []
    for _ in range(steps):
        flush()
        a, c = E(), E()
        a.record(stream)
        res.split()
        res.merge()
        c.record(stream)
        torch.cuda.synchronize()
        step_ms.append(a.elapsed_time(c))
        flush()
        a, b = E(), E()
        a.record(stream)
        res.split()
        b.record(stream)
        torch.cuda.synchronize()
        split_ms.append(a.elapsed_time(b))
    return dict(total_ms=sum(step_ms), wall_s=None, split_ms=split_ms, step_ms=step_ms)


def time_stream_read(buf, nbytes: int, reps: int = 20) -> float:
    """Median duration (ms) of the plain streaming read over the first ``nbytes`` of buf:
    the practical read ceiling beside a decode step over the same bytes."""
    import torch
    import paged_split_kv_02_amd as K
    part = torch.empty(K.STREAM_READ_GROUPS * 4, dtype=torch.int32, device=buf.device)
    stream = torch.cuda.current_stream()
    for _ in range(3):
        K.attn_stream_read(buf, nbytes, part)
    times = []
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        K.attn_stream_read(buf, nbytes, part)
        b.record(stream)
        torch.cuda.synchronize()
        times.append(a.elapsed_time(b))
    return median(times)


def prefill_flops(wl) -> int:
    """Algorithmic FLOPs of a prefill: 4 * D per (row, query head, visible key) (QK^T and
    PV, one multiply-add each), a row at position p seeing min(p + 1, window) keys."""
    total_keys = 0
    for r in range(wl.batch):
        L, n = int(wl.seq_lens[r]), int(wl.q_lens[r])
        for p in range(L - n, L):
            total_keys += min(p + 1, wl.window) if wl.window > 0 else p + 1
    return 4 * wl.head_dim * wl.num_q_heads * total_keys


def time_prefill(wl, launches=10, warmup=2, flush=None):
    """Median duration of attn_prefill launches (events on the launch stream)."""
    import numpy as np
    import torch
    import paged_split_kv_02_amd as K
    dev = torch.device("cuda:0")
    plan = K.attn_prefill_plan(K.make_desc(**wl.desc_fields()), wl.seq_lens, wl.q_starts)
    q = torch.from_numpy(np.ascontiguousarray(wl.q, dtype=np.float32)).to(dev)
    pool = torch.from_numpy(wl.pool.view(np.uint8)).to(dev)
    table = torch.from_numpy(wl.table).to(dev)
    lens = torch.from_numpy(wl.seq_lens).to(dev)
    starts = torch.from_numpy(wl.q_starts).to(dev)
    out = torch.empty_like(q)
    stream = torch.cuda.current_stream()
    times = []
    for it in range(warmup + launches):
        if flush is not None:
            flush()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        K.attn_prefill(plan, q, pool, table, lens, starts, out)
        b.record(stream)
        torch.cuda.synchronize()
        if it >= warmup:
            times.append(a.elapsed_time(b))
    return median(times), plan


def median(xs):
    s = sorted(xs)
    n = len(s)
    return s[n // 2] if n % 2 else 0.5 * (s[n // 2 - 1] + s[n // 2])


def percentile(xs, p):
    """Linear interpolation between the closest ranks."""
    s = sorted(xs)
    x = (len(s) - 1) * p / 100.0
    i = int(x)
    return s[i] if i + 1 >= len(s) else s[i] + (s[i + 1] - s[i]) * (x - i)


def cpu_baseline(wl, budget_s=10.0, single_s=5.0):
    """Time the fp64 oracle on the host over the same step, repeated until the budget
    is spent (KV heads one after another, at least one); GB/s of K/V rows consumed.
    Then the same with the numeric library held to one thread (``single_thread``)."""
    from threadpoolctl import threadpool_limits
    out = _oracle_rate(wl, budget_s)
    with threadpool_limits(limits=1):
        one = _oracle_rate(wl, single_s)
    out["single_thread"] = {k: one[k] for k in ("value", "unit", "cores", "sample", "seconds",
                                                 "us_per_step_equiv")}
    return out


def _oracle_rate(wl, budget_s):
    import numpy as np
    import oracle
    from threadpoolctl import threadpool_info
    G = wl.num_q_heads // wl.num_kv_heads
    done_heads = 0
    total_heads = wl.batch * wl.num_kv_heads
    # one untimed pass first (first touches of the host arrays, library start-up)
    lo, L = oracle.visible_range(int(wl.seq_lens[0]), wl.window)
    Kx, Vx = oracle.keys_values(wl, oracle.bf16_bits_to_f64(oracle.gather_rows(wl, 0, 0, np.arange(lo, L))))
    oracle.dense_attention(wl.q[0, 0:G], Kx, Vx, wl.scale)
    t0 = time.perf_counter()
    while True:
        for r in range(wl.batch):
            lo, L = oracle.visible_range(int(wl.seq_lens[r]), wl.window)
            pos = np.arange(lo, L)
            for g in range(wl.num_kv_heads):
                Kx, Vx = oracle.keys_values(
                    wl, oracle.bf16_bits_to_f64(oracle.gather_rows(wl, r, g, pos)))
                oracle.dense_attention(wl.q[r, g * G:(g + 1) * G], Kx, Vx, wl.scale)
                done_heads += 1
                if time.perf_counter() - t0 > budget_s:
                    break
            if time.perf_counter() - t0 > budget_s:
                break
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    bytes_done = wl.kv_bytes() * done_heads / total_heads
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    return {"value": round(bytes_done / dt / 1e9, 4), "unit": "GB/s", "cores": threads,
            "kind": "oracle",
            "sample": f"{done_heads} KV-head passes ({done_heads / total_heads:.2f} steps) of the "
                      f"same {wl.seq_lens[0]}-token step, fp64 numpy oracle, {dt:.1f} s wall",
            "seconds": round(dt, 2),
            "us_per_step_equiv": round(dt / done_heads * total_heads * 1e6, 1),
            "cores_note": "threads of the numeric library (the score and output products); "
                          "the row gather and the bf16 widening run on one thread",
            "host_cpu": host_cpu_model(), "host_nproc": os.cpu_count()}


def host_cpu_model() -> str:
    """The host CPU's model name as the kernel reports it."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


def main():
    args = parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported here "
              "(the decode step shards across GPUs without this process).", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch
    import synth
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    import paged_split_kv_02_amd  # noqa: F401  (raises if the HIP library is missing)

    t_gen = time.perf_counter()
    wl = synth.global_decode(args.context, seed=2, fmt=args.fmt)
    print(f"# generated {args.context}-token {args.fmt} workload in {time.perf_counter() - t_gen:.1f} s",
          file=sys.stderr, flush=True)
    res = Resident(wl, args.num_chunks)
    if args.copy_calibration:
        a = torch.empty(1 << 28, dtype=torch.float32, device="cuda:0")
        b = torch.empty_like(a)
        a.fill_(1.0)
        torch.cuda.synchronize()
        b.copy_(a)  # reads 1 GiB, writes 1 GiB
        torch.cuda.synchronize()
        del a, b

    t = time_steps(res, args.steps, args.warmup)
    # the same step, each one after an untimed 1 GiB write that evicts the caches
    flush_buf = torch.empty(1 << 28, dtype=torch.float32, device="cuda:0")

    def flush():
        flush_buf.zero_()  # 1 GiB of writes evicts the 256 MB infinity cache
    tf = time_steps(res, args.steps, 2, flush=flush)
    # the plain streaming read over the step's own K/V bytes (the pool's leading pages)
    read_bytes = wl.kv_bytes() // 16 * 16
    read_ms = time_stream_read(res.pool, read_bytes)
    ms_per_step = t["total_ms"] / args.steps
    kv = wl.kv_bytes()
    gbs = kv / (ms_per_step * 1e-3) / 1e9
    split_avg_ms = sum(t["split_ms"]) / len(t["split_ms"])
    kb = res.kernel_bytes()
    achieved = kb / (split_avg_ms * 1e-3) / 1e9
    traffic = read_traffic(kb)

    line = {
        "metric": METRIC,
        "value": round(gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "us_per_step": round(ms_per_step * 1e3, 2),
        "us_per_step_median": round(median(t["step_ms"]) * 1e3, 2),
        "pct_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
        "flushed": {"us_per_step_median": round(median(tf["step_ms"]) * 1e3, 2),
                    "partial_kernel_us_median": round(median(tf["split_ms"]) * 1e3, 2),
                    "effective_gbs": round(kv / (median(tf["step_ms"]) * 1e-3) / 1e9, 1),
                    "timing": f"median of {args.steps} steps, each after an untimed 1 GiB write"},
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"global-decode-{args.context}-{args.fmt}", "context": args.context,
                   "batch": 1, "q_heads": 32, "kv_heads": 4, "head_dim": 512, "page_size": 256,
                   "row_cols": wl.row_cols, "num_chunks": res.plan.num_chunks,
                   "chunk_len": res.plan.chunk_len, "merge_group": res.plan.merge_group,
                   "kv_bytes": kv, "parallelism": "single-gpu"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "kernel": "split_partial_kernel",
                     "kernel_us": round(split_avg_ms * 1e3, 2), "algorithmic_bytes": kb},
        "merge_us": round((ms_per_step - split_avg_ms) * 1e3, 2),
        "kernel_us_p10_p90": [round(percentile(t["split_ms"], 10) * 1e3, 2),
                              round(percentile(t["split_ms"], 90) * 1e3, 2)],
        "step_us_p10_p90": [round(percentile(t["each_step_ms"], 10) * 1e3, 2),
                            round(percentile(t["each_step_ms"], 90) * 1e3, 2)],
        "read_ceiling": {"kernel": "attn_stream_read", "bytes": read_bytes,
                         "us": round(read_ms * 1e3, 2),
                         "gbs": round(read_bytes / (read_ms * 1e-3) / 1e9, 1),
                         "step_pct_of_ceiling": round(100 * (read_ms / ms_per_step), 2),
                         "kernel_pct_of_ceiling": round(100 * (read_ms / split_avg_ms), 2)},
    }
    print(f"# step {ms_per_step * 1e3:.1f} us, partial kernel {split_avg_ms * 1e3:.1f} us",
          file=sys.stderr, flush=True)
    del res

    if not args.no_variants:
        variants = {}
        pick = [x for x in args.variants.split(",") if x]

        def wanted(name):
            return not pick or any(x in name for x in pick)
        for name, maker, n_steps in (
                ("global-decode-10602-split", lambda: synth.global_decode(10602, seed=13), 20),
                ("global-decode-40002-split", lambda: synth.global_decode(40002, seed=14), 20),
                ("global-decode-81653-split", lambda: synth.global_decode(81653, seed=15), 20),
                ("global-decode-163336-folded", lambda: synth.global_decode(163336, seed=3, fmt="folded"), 20),
                # the headline's workload with 64 chunks of equal length: the automatic plan
                # gives even-numbered chunks (on the even XCDs) more keys than odd ones, and
                # this line shows whether that still pays on the part the bench runs on
                ("global-decode-163336-split-equal-chunks",
                 lambda: synth.global_decode(163336, seed=2), 20),
                ("global-decode-4streams-9k-split", lambda: synth.global_streams(seed=16), 20),
                # one GPU's share of the headline step if it were sharded over GPUs: by KV
                # head (one of the four, its 8 query heads) or by sequence (1/8 of the keys)
                ("shard-kvhead-163336-split-8q1kv",
                 lambda: synth.make_workload([163336], num_q_heads=8, num_kv_heads=1, head_dim=512,
                                             page_size=256, seed=17), 20),
                ("shard-seq-20417-split", lambda: synth.global_decode(20417, seed=18), 20),
                ("sliding-hd256-16ragged-w1024", lambda: synth.sliding_batch(seed=4), 20),
                ("global-decode-163336-split-4rows",
                 lambda: synth.make_workload([163336], **synth.GLOBAL, seed=6, num_rows=4,
                                             spare_pages=1), 20),
                ("global-decode-163336-split-4rows-tree",
                 lambda: synth.set_tree(synth.make_workload([163336], **synth.GLOBAL, seed=6,
                                                            num_rows=4, spare_pages=1),
                                        np.array([[-1, 0, 0, 1]], dtype=np.int32)), 20),
                ("global-decode-163336-split-fp8e4m3-4rows",
                 lambda: synth.make_workload([163336], **synth.GLOBAL, seed=7, num_rows=4,
                                             kv_dtype=synth.FP8, spare_pages=1), 20),
                ("global-decode-163336-split-fp8e4m3",
                 lambda: synth.global_decode(163336, seed=7, kv_dtype=synth.FP8), 20),
                ("global-decode-163336-folded-fp8e4m3",
                 lambda: synth.global_decode(163336, seed=8, fmt="folded", kv_dtype=synth.FP8), 20),
                ("global-decode-163336-split-f16",
                 lambda: synth.global_decode(163336, seed=9, kv_dtype=synth.F16), 20),
                ("sliding-hd256-16ragged-w1024-fp8e4m3",
                 lambda: synth.sliding_batch(seed=4, kv_dtype=synth.FP8), 20),
                ("global-decode-163336-split-f32",
                 lambda: synth.global_decode(163336, seed=10, kv_dtype=synth.F32), 20),
                ("global-decode-163336-folded-f32",
                 lambda: synth.global_decode(163336, seed=10, fmt="folded", kv_dtype=synth.F32), 20),
                ("global-decode-163336-split-f32-4rows",
                 lambda: synth.make_workload([163336], **synth.GLOBAL, seed=10, num_rows=4,
                                             kv_dtype=synth.F32, spare_pages=1), 20)):
            if not wanted(name):
                continue
            vwl = maker()
            vres = Resident(vwl, 64 if name.endswith("equal-chunks") else 0)
            vt = time_steps(vres, n_steps, 3, flush=flush)
            vms = median(vt["step_ms"])
            vsplit = median(vt["split_ms"])
            variants[name] = {"us_per_step": round(vms * 1e3, 2), "query_rows": vwl.num_rows,
                              "kv_dtype": vwl.kv_dtype,
                              "partial_kernel_us": round(vsplit * 1e3, 2),
                              "merge_us": round((vms - vsplit) * 1e3, 2),
                              "kv_bytes": vwl.kv_bytes(),
                              "effective_gbs": round(vwl.kv_bytes() / (vms * 1e-3) / 1e9, 1),
                              "pct_hbm_peak": round(100 * vwl.kv_bytes() / (vms * 1e-3) / 1e9
                                                    / HBM_PEAK_GBS, 2),
                              "partial_kernel_gbs": round(vres.kernel_bytes() / (vsplit * 1e-3) / 1e9, 1),
                              "num_chunks": vres.plan.num_chunks,
                              "chunk_len_even_odd": [vres.plan.chunk_len, vres.plan.chunk_len_odd],
                              "timing": "median, cache flushed"}
            print(f"# {name}: {vms * 1e3:.1f} us/step", file=sys.stderr, flush=True)
            del vres
        # the step that feeds decode: a 10,602-token prompt's K/V rows written into pages
        # (fp32 in, bf16 rows out), and a single decode-token append
        import paged_split_kv_02_amd as K
        wlw = synth.global_decode(10602, seed=5)
        wres = Resident(wlw)
        gen = torch.Generator(device="cuda:0").manual_seed(5)
        for name, n in (("kv-write-prompt-10602-split", 10602), ("kv-write-append-1-split", 1)):
            if not wanted(name):
                continue
            kk = torch.randn(1, n, 4, 512, generator=gen, device="cuda:0")
            vv = torch.randn(1, n, 4, 512, generator=gen, device="cuda:0")
            start = torch.tensor([10602 - n], dtype=torch.int32, device="cuda:0")
            times = []
            for it in range(23):
                flush()
                torch.cuda.synchronize()
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record()
                K.attn_kv_write(wres.plan, kk, vv, n, start, wres.pool, wres.table)
                b.record()
                torch.cuda.synchronize()
                if it >= 3:
                    times.append(a.elapsed_time(b))
            t = median(times)
            moved = kk.numel() * 4 + vv.numel() * 4 + n * 4 * 1024 * 2
            variants[name] = {"us": round(t * 1e3, 2), "bytes": moved,
                              "gbs": round(moved / (t * 1e-3) / 1e9, 1),
                              "timing": "median of 20, cache flushed"}
            print(f"# {name}: {t * 1e3:.1f} us", file=sys.stderr, flush=True)
        del wres
        # paged prefill: a 10,602-token global prompt (split and folded rows, and split rows
        # over an FP8 pool) and the sliding layers' 16 ragged prompts; compute-bound (MFMA),
        # reported in TFLOP/s
        for name, maker in (("global-prefill-10602-split", lambda: synth.global_prefill(10602, seed=11)),
                            ("global-prefill-10602-folded",
                             lambda: synth.global_prefill(10602, seed=11, fmt="folded")),
                            ("global-prefill-10602-split-fp8",
                             lambda: synth.global_prefill(10602, seed=11, kv_dtype=synth.FP8)),
                            ("global-prefill-10602-split-f16",
                             lambda: synth.global_prefill(10602, seed=11, kv_dtype=synth.F16)),
                            ("global-prefill-10602-split-f32",
                             lambda: synth.global_prefill(10602, seed=11, kv_dtype=synth.F32)),
                            ("sliding-prefill-16ragged-w1024-f32",
                             lambda: synth.sliding_prefill(seed=12, kv_dtype=synth.F32)),
                            ("sliding-prefill-16ragged-w1024", lambda: synth.sliding_prefill(seed=12))):
            if not wanted(name):
                continue
            pwl = maker()
            t, plan = time_prefill(pwl, flush=flush)
            fl = prefill_flops(pwl)
            tf = fl / (t * 1e-3) / 1e12
            variants[name] = {"us": round(t * 1e3, 1), "rows": int(pwl.q_starts[-1]),
                              "algorithmic_flops": fl, "tflops": round(tf, 1),
                              "frac_bf16_mfma_peak": round(tf / BF16_MFMA_PEAK_TFLOPS, 4),
                              "mfma_issued_tflops": round(2 * tf, 1),
                              "note": "query and probabilities enter the MFMA as high+low bf16 "
                                      "parts: the MFMA work issued is twice the algorithmic",
                              "timing": "median of 10 launches, cache flushed"}
            print(f"# {name}: {t * 1e3:.1f} us, {tf:.1f} TFLOP/s algorithmic", file=sys.stderr,
                  flush=True)
            del pwl
        line["variants"] = variants
    del flush_buf

    if not args.no_cpu_baseline:
        print("# timing the fp64 oracle on the host", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(wl)
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
