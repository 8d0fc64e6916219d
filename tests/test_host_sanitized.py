"""The library's host-side logic (eligibility, argument pairing, pool layout,
the write's launch plan and workspace, the producer's K split, validate-mode
row checks) built with the address and undefined-behaviour sanitizers and run
on the CPU, against brute-force and invariant checks (tests/asan)."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "speculative_decoding_draft_stacked_amd", "csrc")


@pytest.mark.skipif(shutil.which("g++") is None, reason="no host C++ compiler")
def test_host_logic_under_asan_and_ubsan(tmp_path):
    exe = tmp_path / "host_logic_check"
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           os.path.join(ROOT, "tests", "asan", "host_logic_check.cpp"),
           os.path.join(CSRC, "host_logic.cpp"), "-o", str(exe)]
    subprocess.run(cmd, check=True, capture_output=True, text=True, timeout=300)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "host logic checks passed" in r.stdout
