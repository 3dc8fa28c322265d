"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

The host plan (mla_token_decode_amd/csrc/plan.cpp) and the C oracle
(oracle/mla_oracle.c) are each built with gcc/g++ and
-fsanitize=address,undefined -fno-sanitize-recover=all into a small driver
program (tests/sanitize/) that sweeps shapes and checks invariants; any
sanitizer report fails the test.  No device code is built here."""
import os
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
       "-g", "-O1"]


def _build_and_run(cmd_compiler, sources, extra, out_name):
    if shutil.which(cmd_compiler) is None:
        pytest.skip(f"{cmd_compiler} not found")
    with tempfile.TemporaryDirectory(prefix="mla_san_") as d:
        exe = os.path.join(d, out_name)
        subprocess.run([cmd_compiler, *SAN, *extra, "-o", exe, *sources, "-lm"], check=True)
        env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1:verify_asan_link_order=0",
                   UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
        r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
        assert r.returncode == 0, r.stdout + r.stderr
        assert "runtime error" not in r.stderr and "ERROR: AddressSanitizer" not in r.stderr, r.stderr
        return r.stdout


def test_plan_under_sanitizers():
    csrc = os.path.join(ROOT, "mla_token_decode_amd", "csrc")
    out = _build_and_run("g++", [os.path.join(ROOT, "tests", "sanitize", "plan_driver.cpp"),
                                 os.path.join(csrc, "plan.cpp")],
                         ["-std=c++17", "-I" + csrc, "-I" + os.path.join(ROOT, "include")],
                         "plan_driver")
    assert "plans ok" in out


def test_oracle_under_sanitizers():
    out = _build_and_run("gcc", [os.path.join(ROOT, "tests", "sanitize", "oracle_driver.c"),
                                 os.path.join(ROOT, "oracle", "mla_oracle.c")],
                         ["-std=c99", "-ffp-contract=off", "-Wno-unknown-pragmas"], "oracle_driver")
    assert "cases ok" in out
