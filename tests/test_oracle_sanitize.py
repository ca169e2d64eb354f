"""The CPU oracle under gcc's AddressSanitizer and UndefinedBehaviorSanitizer.

tests/native/oracle_driver.c calls every oracle function (all modes and
distances, selection with pending rows and the budget error, attention and
dense attention) on small seeded inputs; the build stops at the first
report. The same driver built without sanitizers must print the same
checksum, so the instrumented build computes what the plain one does.
"""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = [os.path.join(ROOT, "oracle", "ckv_oracle.c"), os.path.join(HERE, "native", "oracle_driver.c")]
BASE = ["gcc", "-std=c11", "-g", "-O1", "-ffp-contract=off", "-fno-fast-math"]


def _run(tmp_path, name, extra):
    exe = str(tmp_path / name)
    subprocess.run(BASE + extra + ["-o", exe] + SRC + ["-lm"], check=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    env.pop("LD_PRELOAD", None)
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    return r


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_clean_under_asan_and_ubsan(tmp_path):
    plain = _run(tmp_path, "plain", [])
    assert plain.returncode == 0, plain.stderr
    san = _run(tmp_path, "san", ["-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                                 "-fno-omit-frame-pointer"])
    assert san.returncode == 0, san.stdout + san.stderr
    assert "runtime error" not in san.stderr and "AddressSanitizer" not in san.stderr
    assert san.stdout == plain.stdout and san.stdout.startswith("checksum ")
