"""The streaming-read measurement aid (attn_stream_read through the C ABI): every 16-byte
word of the buffer is read exactly once, shown by the XOR of the per-workgroup results
against numpy's XOR of the words; an empty read writes zeros; nothing past the partial
results is written."""
import numpy as np
import pytest
import torch

import paged_split_kv_02_amd as K
from tests.gpu_harness import SENTINEL, note

pytestmark = pytest.mark.gpu


def xor_words(u8: np.ndarray) -> np.ndarray:
    return np.bitwise_xor.reduce(u8.view(np.uint32).reshape(-1, 4), axis=0)


@pytest.mark.parametrize("nbytes", [0, 16, 48 * 1024 + 16, (64 << 20) + 48])
def test_every_word_read_once(nbytes):
    note(f"[gpu] stream read {nbytes} bytes")
    rng = np.random.default_rng(nbytes)
    host = rng.integers(0, 256, size=max(nbytes, 16), dtype=np.uint8)[:nbytes]
    dev = torch.device("cuda:0")
    buf = torch.from_numpy(host.copy() if nbytes else np.zeros(16, np.uint8)).to(dev)
    G = K.STREAM_READ_GROUPS
    part = torch.full((G * 4 + 64,), SENTINEL, dtype=torch.int32, device=dev)
    K.attn_stream_read(buf, nbytes, part)
    torch.cuda.synchronize()
    got = part.cpu().numpy()
    assert np.all(got[G * 4:] == SENTINEL), "wrote past the partial results"
    total = np.bitwise_xor.reduce(got[:G * 4].view(np.uint32).reshape(G, 4), axis=0)
    want = xor_words(host) if nbytes else np.zeros(4, np.uint32)
    assert np.array_equal(total, want)
    if nbytes == 0:
        assert not np.any(got[:G * 4])
