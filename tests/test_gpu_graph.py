"""The launches under HIP graph capture: a captured decode step (split + merge), a
captured multi-row step and a captured prefill are replayed several times, with new
query values written eagerly between the replays, and every replay must equal the eager
run on the same inputs bit for bit.  Nothing in these paths allocates, synchronises or
records a memset."""
import numpy as np
import pytest
import torch

import synth
from tests.gpu_harness import Device, note
from tests.test_gpu_prefill import PrefillDevice

pytestmark = pytest.mark.gpu


def _capture(fn):
    """Warm up on a side stream, then capture fn() into a graph."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def _replay_matches_eager(q, run_eager, replay, read, what, seed):
    rng = np.random.default_rng(seed)
    qs = [torch.from_numpy(rng.standard_normal(tuple(q.shape)).astype(np.float32)).to(q.device)
          for _ in range(3)]
    eager = []
    for qv in qs:
        q.copy_(qv)
        run_eager()
        torch.cuda.synchronize()
        eager.append(read())
    for rep in range(3):
        for i, qv in enumerate(qs):
            q.copy_(qv)                     # eager work between the replays
            torch.cuda.synchronize()
            replay()
            torch.cuda.synchronize()
            got = read()
            assert np.array_equal(got.view(np.uint32), eager[i].view(np.uint32)), \
                f"{what}: replay {rep} input {i} differs from the eager run"
    note(f"  {what}: 9 replays equal the eager runs")


@pytest.mark.parametrize("rows,dt,fmt", [(1, synth.BF16, "split"), (4, synth.BF16, "split"),
                                         (1, synth.FP8, "split"), (1, synth.FP8, "folded"),
                                         (4, synth.FP8, "split"), (1, synth.F32, "split")])
def test_decode_step_in_a_graph(rows, dt, fmt):
    wl = synth.make_workload([3000, 1200], **synth.GLOBAL, fmt=fmt, seed=90 + rows,
                             num_rows=rows, kv_dtype=dt)
    what = f"decode rows={rows} {dt} {fmt}"
    note(f"[gpu] graph capture of a {what}")
    dev = Device(wl)
    g = _capture(dev.step)
    _replay_matches_eager(dev.q, dev.step, g.replay, dev.result, what, 7)


def test_prefill_in_a_graph():
    wl = synth.make_workload([700, 300], **synth.SLIDING, seed=95, q_lens=[400, 64],
                             max_pages=16)
    note("[gpu] graph capture of a prefill")
    dev = PrefillDevice(wl)
    g = _capture(dev.launch)
    read = lambda: dev.out.cpu().numpy().copy()  # noqa: E731
    _replay_matches_eager(dev.q, dev.launch, g.replay, read, "prefill", 8)

