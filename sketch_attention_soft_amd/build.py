"""Build librace_attn.so (HIP, gfx950) in-tree with hipcc."""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(HERE, "csrc", "race_attn.hip")
HEADERS = [os.path.join(HERE, "csrc", f) for f in ("race_common.h", "race_fwd.h", "race_bwd.h",
                                                   "race_squash.h", "race_walk.h")]
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "librace_attn.so")

ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def command(out: str, extra=()) -> list:
    return [
        hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
        # no packed-fp32 VALU instructions in device code
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", INCLUDE, *extra, SRC, "-o", out,
    ]


def build(verbose: bool = False, extra=()) -> str:
    """Compile unconditionally; returns the library path."""
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = command(tmp, extra)
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed building librace_attn.so")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
