"""GPU test of the allocation-free decode step (attn_decode_step_noalloc) through the C ABI.

Its output must equal, bit for bit, the output of attn_decode_split (attn_decode_split_tree
with masks) + attn_decode_merge with a caller's workspace on the same plan and inputs: the
same kernels run, only the chunk states live in the library's static per-GPU array.  Two
calls in a row, the second on a smaller input; each output is also held to the decode
bar against the fp64 oracle.  Collected last (a failure here must not hide other tests).
"""
import numpy as np
import pytest
import torch

import oracle
import paged_split_kv_02_amd as K
import synth
from tests.gpu_harness import Device, note
from tests.test_gpu_parity import check

pytestmark = pytest.mark.gpu


def _noalloc(dev: Device) -> np.ndarray:
    """Run the allocation-free step on a Device's buffers into a fresh guarded output."""
    wl = dev.wl
    n = wl.batch * wl.num_rows * wl.num_q_heads * wl.head_dim
    guard = 1024
    buf = torch.full((n + 2 * guard,), 0x7FBADBAD, dtype=torch.int32, device="cuda:0")
    out = buf.view(torch.float32)[guard:guard + n]
    masks = None
    if getattr(wl, "row_masks", None) is not None:
        masks = torch.from_numpy(np.ascontiguousarray(wl.row_masks).view(np.int64)).to("cuda:0")
    K.attn_decode_step_noalloc(dev.plan, dev.q, dev.pool, dev.table, dev.lens, out, row_masks=masks)
    torch.cuda.synchronize()
    b = buf.cpu().numpy()
    assert np.all(b[:guard] == 0x7FBADBAD) and np.all(b[-guard:] == 0x7FBADBAD), "wrote outside out"
    return out.cpu().numpy().reshape(dev.result().shape)


def _with_workspace(dev: Device) -> np.ndarray:
    wl = dev.wl
    if getattr(wl, "row_masks", None) is not None:
        masks = torch.from_numpy(np.ascontiguousarray(wl.row_masks).view(np.int64)).to("cuda:0")
        K.attn_decode_split_tree(dev.plan, dev.q, dev.pool, dev.table, dev.lens, masks, dev.ws)
        K.attn_decode_merge(dev.plan, dev.ws, dev.out)
        torch.cuda.synchronize()
        return dev.result()
    return dev.run()


def _pair(wl, what, **kw):
    note(f"[gpu] noalloc {what}")
    dev = Device(wl, **kw)
    ref = _with_workspace(dev)
    got = _noalloc(dev)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), f"{what}: differs from split+merge"
    check(got, oracle.decode_attention(wl), f"noalloc {what}")
    return got


def test_noalloc_equals_split_merge_twice_smaller_second():
    """A 10,602-token global step, then the 1,024-token tiny step (fewer chunk states):
    each equals split + merge bit for bit; the second is not disturbed by the first's
    states left in the array."""
    _pair(synth.global_decode(10602, seed=301), "global 10602 split")
    _pair(synth.tiny_ref(seed=302), "tiny 1024 n=8", num_chunks=8)


def test_noalloc_other_shapes():
    """The sliding batch (head dim 256, window), a folded row, a 3-row causal window, a tree
    window and FP8 / f32 pools, one after another on the same array."""
    _pair(synth.make_workload([5000, 333], **synth.GLOBAL, seed=303, num_rows=3), "rows=3")
    wl = synth.make_workload([900, 40], **synth.GLOBAL, seed=304, num_rows=4)
    synth.set_tree(wl, np.array([[-1, 0, 0, 1], [-1, 0, 1, 1]], dtype=np.int32))
    _pair(wl, "tree rows=4")
    _pair(synth.sliding_batch(seed=305), "sliding batch")
    _pair(synth.make_workload([3000], **synth.GLOBAL, fmt="folded", seed=306), "folded 3000")
    _pair(synth.make_workload([3000, 700], **synth.GLOBAL, seed=307, kv_dtype=synth.FP8),
          "fp8 split 3000,700")
    _pair(synth.make_workload([2000], **synth.GLOBAL, seed=308, kv_dtype=synth.F32), "f32 2000")


def test_noalloc_refuses_plan_beyond_the_array():
    """A plan whose chunk states exceed the static array is refused with ATTN_E_SCRATCH and
    launches nothing (the output keeps its contents)."""
    lens = np.array([163336] * 16, dtype=np.int32)
    f = dict(batch=16, num_q_heads=32, num_kv_heads=4, head_dim=512, format=0, rot_cols=0,
             page_size=256, max_pages_per_seq=639, window=0, num_chunks=64, merge_group=0,
             scale=1 / np.sqrt(512), num_pages=1, page_stride=4 * 256 * 1024,
             head_stride=256 * 1024, row_stride=1024, k_offset=0, v_offset=512)
    plan = K.attn_decode_plan(K.make_desc(**f), lens)
    assert plan.workspace_bytes > K.NOALLOC_SCRATCH_BYTES
    small = torch.zeros(4096, dtype=torch.float32, device="cuda:0")
    table = torch.zeros(16 * 639, dtype=torch.int32, device="cuda:0")
    dlens = torch.from_numpy(lens).to("cuda:0")
    out = torch.full((64,), 3.0, dtype=torch.float32, device="cuda:0")
    with pytest.raises(K.AttnDecodeError) as e:
        K.attn_decode_step_noalloc(plan, small, small, table, dlens, out)
    assert e.value.status == K.STATUS["ATTN_E_SCRATCH"]
    torch.cuda.synchronize()
    assert torch.all(out == 3.0)
