"""The oracle and the library's host-side code under AddressSanitizer and
UndefinedBehaviorSanitizer (CPU only, no GPU):

* the fp64 oracle (oracle/race_oracle.c) built with gcc and both sanitizers,
  driven by tests/sanitize/oracle_check.c over every entry point (small shapes
  across one and several row blocks, P = 1 to 4, causal and not, soft and
  hard, a zero row, the streaming entry points against the one-shot ones);
* the C ABI library rebuilt from the same sources with the sanitizers on its
  host code (device code is compiled as usual and never runs here), and
  tests/test_abi.py run against that build in a child process with the
  sanitizer runtime preloaded: argument validation, workspace sizing, status
  strings and the host-fitted squash polynomial, with any invalid access or
  undefined operation ending the run.
"""
import glob
import os
import shutil
import subprocess
import sys

import pytest

from sketch_attention_soft_amd import build as hip_build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.dirname(os.path.abspath(__file__))
SAN = "address,undefined"


def _clang_asan_runtime():
    found = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return found[-1] if found else None


@pytest.mark.timeout(300)
def test_oracle_under_sanitizers(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    exe = str(tmp_path / "oracle_check")
    cmd = ["gcc", "-O1", "-g", "-fopenmp", "-fno-omit-frame-pointer", "-fsanitize=" + SAN,
           "-fno-sanitize-recover=all", os.path.join(ROOT, "oracle", "race_oracle.c"),
           os.path.join(HERE, "sanitize", "oracle_check.c"), "-lm", "-o", exe]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", OMP_NUM_THREADS="2")
    res = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=240)
    print(res.stdout, res.stderr)
    assert res.returncode == 0, res.stderr
    assert "runtime error" not in res.stderr and "ERROR: AddressSanitizer" not in res.stderr


@pytest.mark.timeout(900)
def test_abi_host_code_under_sanitizers(tmp_path):
    rt = _clang_asan_runtime()
    if rt is None:
        pytest.skip("clang sanitizer runtime not found")
    lib = str(tmp_path / "librace_attn_san.so")
    flags = ["-Xarch_host", "-fsanitize=" + SAN, "-Xarch_host", "-fno-sanitize-recover=all",
             "-Xarch_host", "-fno-omit-frame-pointer"]
    hip_build.build(extra=flags, out=lib, link_extra=["-shared-libasan", *flags[:2]])
    env = dict(os.environ, LD_PRELOAD=rt, ASAN_OPTIONS="detect_leaks=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", RACE_ABI_TEST_LIB=lib)
    res = subprocess.run([sys.executable, "-m", "pytest", os.path.join(HERE, "test_abi.py"), "-q",
                          "-s", "-p", "no:cacheprovider", "-m", "not gpu"],
                         capture_output=True, text=True, env=env, cwd=ROOT, timeout=600)
    print(res.stdout[-3000:], res.stderr[-3000:])
    assert res.returncode == 0
    assert "runtime error" not in res.stdout + res.stderr
    assert "ERROR: AddressSanitizer" not in res.stdout + res.stderr
