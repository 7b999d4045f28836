"""The host code under AddressSanitizer and UndefinedBehaviorSanitizer, on
the CPU: the C oracle (every exported function on small grids) and the host
half of the library (layout planning, argument validation, the Hilbert
sequence, the window search), each built with the sanitizers into _build/
and run as its own process.  Device code is not instrumented: the library's
kernel launchers are replaced by stubs in the host driver, and only paths
that fail or finish on the host are exercised."""

import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OUT = os.path.join(ROOT, "_build", "sanitize")
SAN = os.path.join(ROOT, "tests", "sanitize")
CSRC = os.path.join(ROOT, "block_sparse_attention_major_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def _run(exe):
    env = dict(os.environ, ASAN_OPTIONS="abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    res = subprocess.run([exe], capture_output=True, text=True, timeout=600, env=env)
    text = res.stdout + res.stderr
    print(text[-2000:])
    assert res.returncode == 0, text[-4000:]
    assert "AddressSanitizer" not in text and "runtime error" not in text, text[-4000:]
    return text


def test_oracle_under_sanitizers():
    os.makedirs(OUT, exist_ok=True)
    exe = os.path.join(OUT, "oracle_driver")
    subprocess.run(["gcc", "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer", "-fopenmp",
                    "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                    os.path.join(ROOT, "oracle", "oracle.c"), os.path.join(SAN, "oracle_driver.c"),
                    "-o", exe, "-lm"], check=True, timeout=300)
    assert "0 failure(s)" in _run(exe)


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc is not installed")
def test_library_host_code_under_sanitizers():
    os.makedirs(OUT, exist_ok=True)
    exe = os.path.join(OUT, "host_driver")
    # Sanitizers on the host half only (each flag after -Xarch_host); the
    # device half of these files holds only the no-allocation scratch array.
    san = []
    for flag in ("-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=all"):
        san += ["-Xarch_host", flag]
    cmd = [HIPCC, "-x", "hip", "--offload-arch=gfx950", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           *san, "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           os.path.join(CSRC, "sparse_attn.cpp"), os.path.join(CSRC, "search.cpp"),
           os.path.join(SAN, "host_driver.cpp"), "-o", exe]
    res = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert res.returncode == 0, res.stderr[-4000:]
    assert "0 failure(s)" in _run(exe)
