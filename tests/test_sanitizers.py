"""Host code under the address and undefined-behaviour sanitizers (CPU only).

Two programs are built in a temporary directory and run:

- the CPU oracle (plain C) with a driver that calls every exported function
  on heap blocks of exactly the contracted size, over ordinary and degenerate
  inputs (tests/sanitize/oracle_driver.c);
- the C ABI's host code (argument validation, size helpers, kernel choice),
  compiled host-only and linked against stand-in launchers that touch no
  memory, with a driver that calls every entry point with arguments that fail
  each validation rule, valid arguments and extreme sizes
  (tests/sanitize/abi_driver.cpp, tests/sanitize/launch_stubs.cpp).

No GPU code is built or run: the ABI build passes --offload-host-only and the
sanitizer flags apply to the host compilation only.
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
CSRC = os.path.join(ROOT, "dit_adaptive_layernorm_amd", "csrc")
ENV = dict(os.environ,
           ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
           UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")


def _build_and_run(cmd, exe):
    b = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert b.returncode == 0, b.stderr[-4000:]
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=ENV)
    assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
    assert "0 failures" in r.stdout


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not found")
def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_san")
    cmd = ["gcc", "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer", "-ffp-contract=off",
           "-fsanitize=address,undefined,float-cast-overflow", "-fno-sanitize-recover=all",
           "-Wall", "-Wextra", "-Werror", "-I" + os.path.join(ROOT, "oracle"),
           os.path.join(ROOT, "oracle", "alnp_oracle.c"), os.path.join(SAN, "oracle_driver.c"),
           "-o", exe, "-lm"]
    _build_and_run(cmd, exe)


@pytest.mark.skipif(shutil.which("hipcc") is None, reason="hipcc not found")
def test_abi_host_code_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "abi_san")
    cmd = ["hipcc", "-x", "hip", "--offload-host-only", "-O1", "-g", "-fno-omit-frame-pointer",
           "-Xarch_host", "-fsanitize=address",
           "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all",
           "-I" + os.path.join(ROOT, "include"), "-I" + CSRC,
           os.path.join(CSRC, "abi.hip"), os.path.join(SAN, "launch_stubs.cpp"),
           os.path.join(SAN, "abi_driver.cpp"), "-o", exe]
    _build_and_run(cmd, exe)


def test_abi_driver_calls_every_declared_entry():
    decl = set(re.findall(r"\b(alnp_[a-z0-9_]+)\s*\(", open(os.path.join(ROOT, "include", "alnp.h")).read()))
    called = set(re.findall(r"\b(alnp_[a-z0-9_]+)\(", open(os.path.join(SAN, "abi_driver.cpp")).read()))
    assert decl and decl <= called, sorted(decl - called)
