"""Build the HIP library in-tree: paged_split_kv_02_amd/libattn_decode.so (gfx950)."""
from __future__ import annotations

import os
import shutil
import subprocess
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libattn_decode.so")
SOURCES = [os.path.join(CSRC, "attn_decode.hip"), os.path.join(CSRC, "plan.cpp")]
# Packed fp32 VALU forms are kept out of the generated code.  MFMA accumulators are
# allocated as VGPRs (not AGPRs), so the softmax rescale touches them in place
# instead of copying them across register files every tile.
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-mllvm", "-amdgpu-mfma-vgpr-form",
         "-Wall", "-Wno-unused-function"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP library cannot be built")


def build(verbose: bool = False) -> str:
    """Compile the library; always recompiles.  Returns the path of the .so."""
    fd, tmp = tempfile.mkstemp(prefix="libattn_decode.", suffix=".so.tmp", dir=HERE)
    os.close(fd)
    cmd = [hipcc(), *FLAGS, *SOURCES, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        os.unlink(tmp)
        raise RuntimeError("HIP build failed:\n" + " ".join(cmd) + "\n" + res.stdout + res.stderr)
    if verbose:
        print(" ".join(cmd))
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
