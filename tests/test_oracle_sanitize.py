"""The CPU oracle under AddressSanitizer and UndefinedBehaviorSanitizer.

tests/oracle_drive.c calls every oracle entry point on small seeded inputs
(ragged shapes, r = 0 and r > 0, zero / subnormal / near-maximum groups,
sampled row lists, optional outputs left out) with every buffer allocated at
exactly the size the oracle's contract states, and prints a hash of each
output.  It is built twice with the oracle's sources: as the oracle is
normally built, and with -fsanitize=address,undefined (no recovery, so any
report ends the run with an error).  Both runs must succeed, the sanitized
one must print no report, and the two must print the same hashes (the
instrumented build computes the same results).  Host code only.
"""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ORACLE = os.path.join(os.path.dirname(HERE), "oracle")
SOURCES = [os.path.join(ORACLE, f) for f in
           ("svdq_oracle.c", "awq_oracle.c", "qkv_oracle.c", "mxfp4_oracle.c")]
DRIVER = os.path.join(HERE, "oracle_drive.c")
BASE = ["-std=c11", "-Wall", "-fopenmp", "-ffp-contract=off", "-fno-fast-math"]
SANITIZE = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
            "-fsanitize=float-cast-overflow", "-fno-sanitize-recover=all"]


def _build(tmp_path, name, flags):
    exe = str(tmp_path / name)
    subprocess.run(["gcc"] + BASE + flags + [DRIVER] + SOURCES + ["-o", exe, "-lm"], check=True,
                   capture_output=True, text=True)
    return exe


def _run(exe):
    env = dict(os.environ, OMP_NUM_THREADS="2",
               ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:exitcode=23",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1:exitcode=24")
    return subprocess.run([exe], env=env, capture_output=True, text=True, timeout=120)


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_clean_under_asan_ubsan(tmp_path):
    plain = _run(_build(tmp_path, "drive_plain", ["-O2"]))
    assert plain.returncode == 0, plain.stderr
    san = _run(_build(tmp_path, "drive_san", SANITIZE))
    assert san.returncode == 0, "sanitizer report:\n" + san.stderr[-4000:]
    assert "runtime error" not in san.stderr and "ERROR:" not in san.stderr, san.stderr[-4000:]
    lines = plain.stdout.splitlines()
    assert len(lines) > 50
    assert san.stdout == plain.stdout
