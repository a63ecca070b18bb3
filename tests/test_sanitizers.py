"""Host code under the address and undefined-behaviour sanitizers (CPU only).

Two programs are built and run:
  - the CPU oracle, every routine once on small seeded inputs
    (tests/sanitize/oracle_driver.c);
  - libkvq's host side (kvq_host.cpp, kvq_layout.cpp: context creation, the
    Lloyd-Max table builders, SplitMix64 signs, workspace layouts and the
    validation of every entry point) on a fake device whose HIP calls and
    kernel launches are host stand-ins (tests/sanitize/host_driver.cpp,
    hip_stubs.cpp).  No GPU code is built or run.
Any invalid access, leak or undefined operation aborts the program."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
CSRC = os.path.join(ROOT, "calibration_free_kv_amd", "csrc")
CLANGXX = "/opt/rocm/llvm/bin/clang++"
FLAGS = ["-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")


def _run(cmd, tmp_path, exe):
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    r = subprocess.run([exe], capture_output=True, text=True, env=ENV, timeout=300)
    assert r.returncode == 0, (r.stdout[-2000:], r.stderr[-6000:])
    return r.stdout


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    out = _run(["gcc", "-std=c11", *FLAGS, "-o", exe, os.path.join(SAN, "oracle_driver.c"),
                os.path.join(ROOT, "oracle", "kvq_oracle.c"), "-lm"], tmp_path, exe)
    assert "oracle ok" in out


@pytest.mark.skipif(not os.path.exists(CLANGXX), reason="needs the ROCm clang++")
def test_host_side_under_sanitizers(tmp_path):
    exe = str(tmp_path / "host_driver")
    out = _run([CLANGXX, "-std=c++17", *FLAGS, "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
                "-I" + os.path.join(ROOT, "include"), "-I" + CSRC, "-I" + SAN, "-Wno-unused-command-line-argument",
                "-o", exe, os.path.join(SAN, "host_driver.cpp"), os.path.join(SAN, "hip_stubs.cpp"),
                os.path.join(CSRC, "kvq_host.cpp"), os.path.join(CSRC, "kvq_layout.cpp")], tmp_path, exe)
    assert "host ok" in out
    # the same program with the KVQ_SPLITS override of the automatic split count
    r = subprocess.run([exe], capture_output=True, text=True, env=dict(ENV, KVQ_SPLITS="3"), timeout=300)
    assert r.returncode == 0 and "host ok" in r.stdout, (r.stdout[-2000:], r.stderr[-4000:])
