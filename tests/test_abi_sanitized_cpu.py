"""The C ABI's host logic under AddressSanitizer and UndefinedBehaviorSanitizer
(no GPU): abi.cpp and host.cpp (argument validation, workspace and storage
size arithmetic, grid and split planning, the codebook tables) built for the
CPU with the kernel launchers replaced by stubs that check every workspace
region a kernel would write lies inside the caller's workspace
(tests/host/launch_stubs.cpp), then driven over the workload shapes, ragged
and extreme sizes and every code type (tests/host/abi_sanitize_main.cpp).
The sanitizers apply to host code only (-Xarch_host)."""

import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "bit_nf4_quantized_quantize_amd", "csrc")
HOST = os.path.join(ROOT, "tests", "host")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def test_abi_host_logic_under_asan_ubsan(tmp_path):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    exe = str(tmp_path / "abi_sanitized")
    cmd = [HIPCC, "-O1", "-g", "-std=c++17", "--offload-arch=gfx950",
           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-I", HOST,
           os.path.join(HOST, "abi_sanitize_main.cpp"), os.path.join(HOST, "launch_stubs.cpp"),
           os.path.join(CSRC, "abi.cpp"), os.path.join(CSRC, "host.cpp"), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
    assert r.stdout.startswith("ok"), r.stdout
