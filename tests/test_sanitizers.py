"""The host code under AddressSanitizer and UndefinedBehaviorSanitizer, on the
CPU: the C oracle driven through every function and its edge cases, and the
C ABI's host side (all validation paths and the act-order permutation) built
as plain C++ with the kernel launchers stubbed out (nothing reaches them
without a GPU).  Any sanitizer report fails the run."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1")
CLANG = "/opt/rocm/llvm/bin/clang++"


def _run(cmd, cwd):
    r = subprocess.run(cmd, cwd=cwd, capture_output=True, text=True, env=ENV, timeout=300)
    assert r.returncode == 0, "%s\n%s\n%s" % (" ".join(cmd), r.stdout[-3000:], r.stderr[-3000:])
    return r.stdout


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc missing")
def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    _run(["gcc", "-std=c11", "-fopenmp"] + SAN + [os.path.join(HERE, "oracle_driver.c"),
                                                   os.path.join(ROOT, "oracle", "mnb_oracle.c"), "-o", exe, "-lm"],
         ROOT)
    assert _run([exe], ROOT).strip().endswith("ok")


@pytest.mark.skipif(not os.path.exists(CLANG), reason="ROCm clang++ missing")
def test_c_abi_host_side_under_sanitizers(tmp_path):
    exe = str(tmp_path / "api_driver")
    inc = ["-I" + os.path.join(ROOT, "include"), "-I" + os.path.join(ROOT, "block_wise_int4_amd", "csrc"),
           "-I/opt/rocm/include", "-D__HIP_PLATFORM_AMD__"]
    _run([CLANG, "-x", "c++", "-std=c++17"] + SAN + inc +
         [os.path.join(ROOT, "block_wise_int4_amd", "csrc", "mnb_api.cpp"), os.path.join(HERE, "api_driver.cpp"),
          "-o", exe, "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib"], ROOT)
    out = _run([exe], ROOT)
    assert out.strip().endswith("ok: 0 failures"), out
