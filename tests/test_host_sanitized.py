"""The C ABI's host code (validation, workspace layout, argument marshalling,
in attn_api.cpp) built by the host compiler alone with AddressSanitizer and
UndefinedBehaviorSanitizer, against stand-in launchers that record instead of
launching (tests/native/host_stubs.cpp), and driven through every entry point
with bad and good requests (tests/native/abi_driver.cpp). The driver also
checks the paged cache's address arithmetic (paged_index.h, the helper the
kernels use) at block-table entries where a 32-bit product would wrap. Runs
on the CPU; nothing touches a GPU."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CLANG = "/opt/rocm/llvm/bin/clang++"
OUT = os.path.join(ROOT, "_build", "host_sanitized")


def build_driver():
    os.makedirs(OUT, exist_ok=True)
    exe = os.path.join(OUT, "abi_driver")
    csrc = os.path.join(ROOT, "transformer_attention_tiled_amd", "csrc")
    native = os.path.join(ROOT, "tests", "native")
    cmd = [CLANG, "-std=c++17", "-g", "-O1", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", csrc, "-I", native, "-I", "/opt/rocm/include",
           os.path.join(csrc, "attn_api.cpp"), os.path.join(native, "host_stubs.cpp"),
           os.path.join(native, "abi_driver.cpp"), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return exe


@pytest.mark.skipif(not os.path.exists(CLANG), reason="no host clang++")
def test_abi_host_code_is_sanitizer_clean():
    exe = build_driver()
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0 and "ALL OK" in r.stdout, r.stdout + r.stderr
