"""GPU parity at the full context lengths of the global-layer workloads, in the launch
configuration bench.py times (automatic chunking).  The fp64 oracle computes every
output here (one dense matmul per KV head), so the whole output is compared."""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_harness import Device, note
from tests.test_gpu_parity import check

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("L,fmt", [(163336, "split"), (163336, "folded"), (81653, "split")])
def test_full_length(L, fmt):
    note(f"[gpu] full size L={L} {fmt}: generating")
    wl = synth.global_decode(L, seed=2 if fmt == "split" else 3, fmt=fmt)
    note(f"[gpu] full size L={L} {fmt}: running")
    dev = Device(wl)
    got = dev.run()
    assert dev.guards_intact()
    note(f"[gpu] full size L={L} {fmt}: oracle (n={dev.plan.num_chunks})")
    ref = oracle.decode_attention(wl)
    check(got, ref, f"L={L} {fmt}")
