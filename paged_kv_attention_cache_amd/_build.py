"""Build libtl.so (the HIP kernels and the C ABI) in-tree for gfx950 with hipcc."""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libtl.so")
SOURCES = ["tl_api.hip", "tl_write.hip", "tl_decode.hip", "tl_prefill.hip", "tl_gdn.hip", "tl_alloc.hip"]
STREAM_SOURCE = "tl_stream.hip"  # measurement support: built as libtl_stream.so
STREAM_LIB = os.path.join(HERE, "libtl_stream.so")

# -packed-fp32-ops off: no v_pk_{add,mul,fma}_f32 in the device code.
# The atomic optimizer off: it turns a one-lane atomic whose result is read later (the
# decode kernels' work claim, issued a tile before the claimed number is needed) into
# a wave-wide form that reads the result at once, so the round trip was waited on in
# place.  Every atomic in these kernels is issued by one lane.
HIP_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-mllvm", "-amdgpu-atomic-optimizer-strategy=None",
    "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libtl.so)")


def _run(cmd):
    p = subprocess.run(cmd, capture_output=True, text=True)
    if p.returncode != 0:
        raise RuntimeError(f"build step failed: {' '.join(cmd)}\n{p.stdout}\n{p.stderr}")
    return p


def build(verbose: bool = False, extra_flags=(), out: str | None = None, build_dir: str | None = None) -> str:
    """Compile every source for gfx950 and link libtl.so next to this file."""
    bdir = build_dir or BUILD
    lib = out or LIB
    os.makedirs(bdir, exist_ok=True)
    cc = hipcc()
    objs = []

    def one(src):
        obj = os.path.join(bdir, src.replace(".hip", ".o"))
        cmd = [cc, *HIP_FLAGS, *extra_flags, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), file=sys.stderr)
        _run(cmd)
        return obj

    with ThreadPoolExecutor(max_workers=min(4, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(one, SOURCES + [STREAM_SOURCE]))
    tmp = lib + ".tmp"
    _run([cc, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs[:-1]])
    os.replace(tmp, lib)
    if out is None:  # the HBM streaming-read measurement library (bench.py --hbm-ceiling)
        _run([cc, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", STREAM_LIB + ".tmp", objs[-1]])
        os.replace(STREAM_LIB + ".tmp", STREAM_LIB)
    return lib


if __name__ == "__main__":
    print(build(verbose=True))
