"""Builds libgdn.so (the HIP library behind include/gdn.h) in-tree with hipcc for gfx950."""
from __future__ import annotations

import os
import shutil
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libgdn.so")
# the measurement library (include/gdn_stream.h): a streaming copy that bench.py times
STREAM_LIB = os.path.join(PKG, "libgdn_stream.so")
STREAM_SOURCES = [os.path.join(CSRC, "gdn_stream.hip")]
SOURCES = [os.path.join(CSRC, f) for f in ("gdn_kernels.hip", "gdn_conv.hip", "gdn_prefill.hip", "gdn_noalloc.hip",
                                            "gdn_api.cpp")]

# gfx950 only. Packed fp32 ops are switched off for every HIP translation unit. Matrix-core
# results go to ordinary VGPRs (the prefill scan converts and rescales its accumulators
# every chunk; accumulation registers would add a copy each way); only the prefill uses
# the matrix cores.
HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-fvisibility=hidden", "-Wall", "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-I", os.path.join(ROOT, "include"),
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the gfx950 library cannot be built")


def _hipcc(sources: list[str], out: str, extra_flags: list[str] | None, quiet: bool) -> str:
    tmp = out + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, *(extra_flags or []), "-o", tmp, *sources]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + res.stdout + res.stderr)
    if not quiet:
        print(res.stderr)
    os.replace(tmp, out)
    return out


def build(extra_flags: list[str] | None = None, out: str = LIB, quiet: bool = True) -> str:
    """Builds libgdn.so (to `out`) and, for the default output, the measurement library."""
    _hipcc(SOURCES, out, extra_flags, quiet)
    if out == LIB:
        _hipcc(STREAM_SOURCES, STREAM_LIB, None, quiet)
    return out


if __name__ == "__main__":
    print(build(quiet=False))
