"""Sanitizer builds of the host code (CPU only, no GPU).

- The CPU oracle built with AddressSanitizer and UndefinedBehaviorSanitizer
  (g++), driven through every exported function on small shapes held in
  exactly sized buffers (tests/sanitize/oracle_main.cpp).
- The C ABI's host half (argument validation, workspace layout, block bound,
  packed sizes) built by hipcc with the same sanitizers on the host side only,
  linked against stub launchers, driven through the rejection paths and a
  sweep of dimensions (tests/sanitize/abi_main.hip).
Each driver exits non-zero on a failed check; a sanitizer report aborts it.
"""

from __future__ import annotations

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
OUT = os.path.join(ROOT, "_build", "sanitize")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
           UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")


def _run(exe, env):
    res = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "runtime error" not in res.stderr, res.stderr
    return res.stdout


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
def test_oracle_under_asan_ubsan():
    os.makedirs(OUT, exist_ok=True)
    exe = os.path.join(OUT, "oracle_san")
    subprocess.run(["g++", "-O1", "-g", "-std=c++17", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-pthread", "-o", exe,
                    os.path.join(SAN, "oracle_main.cpp"),
                    os.path.join(ROOT, "oracle", "moe_oracle.cpp")], check=True)
    # leak checking on: the oracle owns no memory past a call
    env = dict(ENV, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1")
    assert "oracle sanitizer driver ok" in _run(exe, env)


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
def test_abi_host_half_under_asan_ubsan():
    os.makedirs(OUT, exist_ok=True)
    exe = os.path.join(OUT, "abi_san")
    csrc = os.path.join(ROOT, "w4_dequant_expert_amd", "csrc")
    # sanitizers on the host side only: each one is handed to the host pass
    cmd = [HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17",
           "-Xarch_host", "-fsanitize=address",
           "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-I", os.path.join(ROOT, "include"), "-I", csrc,
           os.path.join(SAN, "abi_main.hip"), os.path.join(csrc, "api.hip"), "-o", exe]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stdout + res.stderr
    # leaks off: the HIP runtime keeps allocations until exit
    assert "abi sanitizer driver ok" in _run(exe, ENV)
