"""Build librace_attn.so (HIP, gfx950) in-tree with hipcc.

Every csrc/*.hip file is one translation unit: the C ABI (race_attn.hip) and
the launch sequences instantiated per row type and direction
(race_inst_*.hip).  They are compiled to objects in parallel under _build/
and linked into one shared library next to this file.
"""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
SOURCES = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
INCLUDE = os.path.join(ROOT, "include")
OBJDIR = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "librace_attn.so")

ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # no packed-fp32 VALU instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def compile_command(src: str, obj: str, extra=()) -> list:
    return [hipcc(), *FLAGS, "-I", INCLUDE, *extra, "-c", src, "-o", obj]


def link_command(objs, out: str, extra=()) -> list:
    return [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *extra, *objs, "-o", out]


def _jobs() -> int:
    n = os.environ.get("MAX_JOBS")
    if n and n.isdigit():
        return max(1, min(int(n), 16))
    return max(1, min(len(os.sched_getaffinity(0)), 16))


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    return res.returncode, res.stdout + res.stderr


def build(verbose: bool = False, extra=(), out: str = LIB, link_extra=()) -> str:
    """Compile every translation unit and link, unconditionally; returns the
    library path.  extra / link_extra: more compiler / linker flags; out:
    where the library goes (another build of the same sources, e.g. one
    instrumented for a test, goes elsewhere)."""
    os.makedirs(OBJDIR, exist_ok=True)
    tag = "%d_%d" % (os.getpid(), abs(hash(out)) % 100000)
    objs = [os.path.join(OBJDIR, os.path.basename(s)[:-4] + f".{tag}.o") for s in SOURCES]
    with ThreadPoolExecutor(_jobs()) as ex:
        results = list(ex.map(lambda so: _run(compile_command(so[0], so[1], extra), verbose),
                              zip(SOURCES, objs)))
    failed = [(s, out) for s, (rc, out) in zip(SOURCES, results) if rc != 0]
    if failed:
        for s, out in failed:
            sys.stderr.write(f"--- {os.path.basename(s)}\n{out}")
        raise RuntimeError("hipcc failed compiling " + ", ".join(os.path.basename(s) for s, _ in failed))
    tmp = out + ".tmp" + tag
    rc, log = _run(link_command(objs, tmp, link_extra), verbose)
    for o in objs:
        os.remove(o)
    if rc != 0:
        sys.stderr.write(log)
        raise RuntimeError("hipcc failed linking " + os.path.basename(out))
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
