"""The C ABI's host code (argument validation, workspace sizing, the per-device
CU cache and the launch sequence of jagged_attn_fwd) under ThreadSanitizer and
under AddressSanitizer + UBSan, from many threads at once.

ja_api.cpp is built with g++ as plain host code and linked against stub HIP
runtime functions and stub kernel launchers (tests/native/api_host_threads.cpp),
so no GPU and no HIP runtime is involved."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "recsys_jagged_attention_amd", "csrc")
OUT = os.path.join(ROOT, "_build", "host_sanitizers")


def build(kind: str) -> str:
    os.makedirs(OUT, exist_ok=True)
    exe = os.path.join(OUT, f"api_host_threads_{kind}")
    flags = {"tsan": ["-fsanitize=thread"], "asan": ["-fsanitize=address,undefined", "-fno-sanitize-recover=all"]}[kind]
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-pthread", *flags, "-D__HIP_PLATFORM_AMD__",
           "-I/opt/rocm/include", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           os.path.join(CSRC, "ja_api.cpp"), os.path.join(ROOT, "tests", "native", "api_host_threads.cpp"),
           "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return exe


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir("/opt/rocm/include"),
                    reason="needs g++ and the HIP headers")
@pytest.mark.parametrize("kind", ["tsan", "asan"])
def test_api_host_code_under_sanitizer(kind):
    exe = build(kind)
    env = dict(os.environ, TSAN_OPTIONS="halt_on_error=1", ASAN_OPTIONS="detect_leaks=1:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([exe, "8", "300"], capture_output=True, text=True, env=env, timeout=600)
    print(r.stdout, r.stderr[-4000:])
    assert r.returncode == 0, r.stderr[-4000:]
    assert "errors 0" in r.stdout
