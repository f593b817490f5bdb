"""The fp64 oracle and the library's host-side layer (argument validation,
overflow guards, workspace sizes) built on the CPU under the address and
undefined-behaviour sanitizers and driven with ordinary and extreme
arguments. The host layer (csrc/host.cpp) holds no HIP code, so it builds with
g++ alone; the kernels are not part of these builds."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
CSRC = os.path.join(ROOT, "vision_mamba_selective_amd", "csrc")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
       "-g", "-O1"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1",
           UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")


def build_and_run(tmp_path, compiler, sources, flags, name):
    if shutil.which(compiler) is None:
        pytest.skip("%s is not installed" % compiler)
    exe = str(tmp_path / name)
    cmd = [compiler, *SAN, *flags, *sources, "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=ENV)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, r.stderr
    return r.stdout


def test_oracle_under_sanitizers(tmp_path):
    out = build_and_run(tmp_path, "gcc",
                        [os.path.join(HERE, "oracle_checks.c"), os.path.join(ROOT, "oracle", "oracle.c")],
                        ["-std=c11", "-lm", "-lpthread"], "oracle_checks")
    assert "oracle checks ok" in out


def test_host_layer_under_sanitizers(tmp_path):
    out = build_and_run(tmp_path, "g++",
                        [os.path.join(HERE, "host_checks.cpp"), os.path.join(CSRC, "host.cpp")],
                        ["-std=c++17", "-I", os.path.join(ROOT, "include"), "-I", CSRC],
                        "host_checks")
    assert "host checks ok" in out
