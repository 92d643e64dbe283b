"""CPU build of the library's host-side planning (csrc/sffn_host.h) and of the fp64 oracle
(oracle/oracle.c) with AddressSanitizer and UndefinedBehaviorSanitizer, run on randomized
inputs (tests/sanitize/host_check.cpp). Any sanitizer report or failed invariant fails the
test. No GPU, no HIP: plain gcc/g++."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "activation_sparse_decode_rank_amd", "csrc")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
       "-g", "-O1"]


@pytest.mark.skipif(shutil.which("g++") is None or shutil.which("gcc") is None,
                    reason="needs gcc and g++")
def test_host_planning_and_oracle_under_sanitizers(tmp_path):
    oracle_o = tmp_path / "oracle.o"
    exe = tmp_path / "host_check"
    subprocess.run(["gcc", "-std=c11", "-ffp-contract=off", *SAN, "-c",
                    os.path.join(ROOT, "oracle", "oracle.c"), "-o", str(oracle_o)], check=True)
    subprocess.run(["g++", "-std=c++17", *SAN, "-I", CSRC,
                    os.path.join(ROOT, "tests", "sanitize", "host_check.cpp"), str(oracle_o),
                    "-o", str(exe), "-lm"], check=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]
    assert "0 failures" in out
