"""Build the HIP library in-tree: paged_split_kv_02_amd/libattn_decode.so (gfx950)."""
from __future__ import annotations

import os
import shutil
import subprocess
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libattn_decode.so")
# Packed fp32 VALU forms are kept out of all generated code.
COMMON = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Wall", "-Wno-unused-function"]
# MFMA accumulators are allocated as VGPRs (not AGPRs): the decode kernels' softmax
# rescale then touches them in place instead of copying them across register files every
# tile, and the 32-key tile kernels (prompt rows, windows of several rows) read their
# scores without copies and stop moving output accumulators between the two files around
# each tile's score products (the query operands stay parked in the AGPRs).
UNITS = [("attn_decode.hip", ["-mllvm", "-amdgpu-mfma-vgpr-form"]),
         ("prefill.hip", ["-mllvm", "-amdgpu-mfma-vgpr-form"]),
         ("stream_read.hip", []),
         ("plan.cpp", [])]
SOURCES = [os.path.join(CSRC, name) for name, _ in UNITS]
INCLUDE = os.path.join(os.path.dirname(HERE), "include")
# Digest of the sources a library was built from, written beside it by build().
DIGEST = LIB + ".digest"


def source_digest() -> str:
    """SHA-256 over the library's sources, headers, build flags and this script."""
    import hashlib
    h = hashlib.sha256()
    files = sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC)) + \
        sorted(os.path.join(INCLUDE, f) for f in os.listdir(INCLUDE)) + [os.path.abspath(__file__)]
    for path in files:
        if os.path.isfile(path):
            h.update(os.path.basename(path).encode() + b"\0")
            with open(path, "rb") as f:
                h.update(f.read())
    h.update(repr((COMMON, UNITS)).encode())
    return h.hexdigest()


def built_digest() -> str | None:
    """Digest recorded for the library on disk (None if there is none)."""
    try:
        with open(DIGEST) as f:
            return f.read().strip()
    except OSError:
        return None


def is_current() -> bool:
    """True if the library exists and was built from the sources as they are now."""
    return os.path.exists(LIB) and built_digest() == source_digest()


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP library cannot be built")


def build(verbose: bool = False) -> str:
    """Compile the library; always recompiles.  Returns the path of the .so."""
    cc = hipcc()
    digest = source_digest()
    with tempfile.TemporaryDirectory(prefix="attn_build.") as tmpdir:
        objs = []
        for name, extra in UNITS:
            obj = os.path.join(tmpdir, name + ".o")
            _run([cc, *COMMON, *extra, "-c", os.path.join(CSRC, name), "-o", obj], verbose)
            objs.append(obj)
        fd, tmp = tempfile.mkstemp(prefix="libattn_decode.", suffix=".so.tmp", dir=HERE)
        os.close(fd)
        try:
            _run([cc, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
        except RuntimeError:
            os.unlink(tmp)
            raise
        os.replace(tmp, LIB)
    with open(DIGEST + ".tmp", "w") as f:
        f.write(digest + "\n")
    os.replace(DIGEST + ".tmp", DIGEST)
    return LIB


def _run(cmd, verbose):
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("HIP build failed:\n" + " ".join(cmd) + "\n" + res.stdout + res.stderr)
    if verbose:
        print(" ".join(cmd))


if __name__ == "__main__":
    print(build(verbose=True))
