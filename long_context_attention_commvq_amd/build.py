"""Build libcommvq.so (HIP for gfx950) in place, next to this file.

    python -m long_context_attention_commvq_amd.build
"""

from __future__ import annotations

import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libcommvq.so")
SOURCES = ["api.cpp", "encode.hip", "decode.hip", "decode_fast.hip", "decode_merge.hip", "decode_bitv.hip", "naive.hip", "em.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# Packed-fp32 instructions are switched off for all device code.
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", os.path.join(os.path.dirname(HERE), "include")]


def _run(cmd: list[str], verbose: bool) -> None:
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed building libcommvq.so")


def build(verbose: bool = False, jobs: int | None = None) -> str:
    """Compile every source to an object (in parallel), then link the library."""
    jobs = jobs or min(len(SOURCES), max(1, min(8, os.cpu_count() or 1)))
    with tempfile.TemporaryDirectory(prefix="commvq_build_") as tmpdir:
        objs = [os.path.join(tmpdir, os.path.splitext(s)[0] + ".o") for s in SOURCES]
        cmds = [[HIPCC, *FLAGS, "-c", os.path.join(CSRC, s), "-o", o] for s, o in zip(SOURCES, objs)]
        with ThreadPoolExecutor(max_workers=jobs) as ex:
            for f in [ex.submit(_run, c, verbose) for c in cmds]:
                f.result()
        tmp = LIB + ".tmp"
        _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
