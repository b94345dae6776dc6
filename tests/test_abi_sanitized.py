"""The C-ABI validation layer under the host compiler's address and
undefined-behaviour sanitizers (CPU only): kda_api.cpp is built with g++ and
a host stub for the device side, and the ABI tests plus a random-argument
fuzz of every *_plan entry point run against it in a child process that
preloads the sanitizer runtime."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = [os.path.join(ROOT, "gated_delta_rule_decode_amd", "csrc", "kda_api.cpp"),
       os.path.join(ROOT, "tests", "sanitize", "kda_host_stub.cpp")]


def _runtime(name):
    out = subprocess.run(["g++", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return out if os.path.isabs(out) and os.path.exists(out) else None


def test_validation_layer_under_asan_and_ubsan(tmp_path):
    if shutil.which("g++") is None or _runtime("libasan.so") is None:
        pytest.skip("g++ with libasan is not available")
    so = tmp_path / "libkda_host_asan.so"
    subprocess.run(["g++", "-std=c++17", "-O1", "-g", "-fPIC", "-shared", "-fno-omit-frame-pointer",
                    "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                    "-I", os.path.join(ROOT, "include"), *SRC, "-o", str(so)], check=True)
    env = dict(os.environ)
    env["LD_PRELOAD"] = _runtime("libasan.so")
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    r = subprocess.run([sys.executable, os.path.join(ROOT, "tests", "sanitize", "run_abi_sanitized.py"),
                        str(so)], env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, (r.stdout[-3000:] + r.stderr[-3000:])
    assert "fuzzed plan calls" in r.stdout
