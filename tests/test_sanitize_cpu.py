"""Host-side sanitizer runs (AddressSanitizer + UndefinedBehaviorSanitizer).

Two separate binaries, built with g++ from source: the CPU oracle with a
driver that calls every oracle entry point (tests/sanitize/oracle_san.cpp),
and the library's host-side packers with a driver that calls them and every
argument check (tests/sanitize/pack_san.cpp). The packers' source is copied to
a .cpp file first and compiled as host C++ against the HIP headers; no device
code is involved. Any sanitizer report aborts the binary.
"""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SAN = ["-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
       "-fsanitize=address,undefined", "-fno-sanitize-recover=all"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1",
           UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")

pytestmark = pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")


def _build_and_run(tmp_path, name, args):
    exe = str(tmp_path / name)
    r = subprocess.run(["g++"] + SAN + args + ["-o", exe], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-4000:]
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=ENV)
    assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr[-4000:]
    return r.stdout


def test_oracle_under_sanitizers(tmp_path):
    out = _build_and_run(tmp_path, "oracle_san", [
        "-fopenmp", os.path.join(HERE, "sanitize", "oracle_san.cpp"), os.path.join(ROOT, "oracle", "oracle.cpp")])
    assert "clean" in out


def test_packers_under_sanitizers(tmp_path):
    src = tmp_path / "pack_host.cpp"
    text = open(os.path.join(ROOT, "int4_grouped_gemm_router_amd", "csrc", "pack.hip")).read()
    src.write_text(text.replace('#include "../../include/moe_int4.h"', '#include "moe_int4.h"')
                   .replace('#include "layout.h"', '#include "' + os.path.join(
                       ROOT, "int4_grouped_gemm_router_amd", "csrc", "layout.h") + '"'))
    out = _build_and_run(tmp_path, "pack_san", [
        "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-I" + os.path.join(ROOT, "include"),
        str(src), os.path.join(HERE, "sanitize", "pack_san.cpp")])
    assert "clean" in out
