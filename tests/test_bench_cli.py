"""Host-side contract of bench.py (no GPU): the one-GPU refusal, per-workload defaults, and
the algorithmic byte counts its roofline lines divide by."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


@pytest.mark.parametrize("workload", ["mlp_up", "qkv", "awq_mod", "mx_qkv", "block"])
def test_more_than_one_gpu_is_refused(workload):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2",
                        "--workload", workload], capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def _parse(argv):
    old = sys.argv
    sys.argv = ["bench.py"] + argv
    try:
        return bench.parse()
    finally:
        sys.argv = old


def test_defaults_and_overrides():
    a = _parse([])
    assert (a.workload, a.gpus, a.steps, a.warmup) == ("mlp_up", 1, 50, 300)
    a = _parse(["--workload", "awq_mod"])
    assert a.steps == 2000 and a.warmup == 10000
    a = _parse(["--workload", "awq_mod", "--steps", "7", "--warmup", "3"])
    assert a.steps == 7 and a.warmup == 3


def test_algorithmic_bytes():
    # qkv: every tensor once (codes 4 bits, fp32 scales per 64, bf16 L2 / bias / Y, fp32 xl1)
    M, K, N, r = 4608, 3072, 9216, 32
    G = K // 64
    want = M * K // 2 + 4 * M * G + N * K // 2 + 4 * N * G + 4 * M * r + 2 * r * N + 2 * N + 2 * M * N
    assert bench.k2_bytes(M, N, K, r) == want == 110020608
    assert bench.k1_bytes(M, K, r) == 2 * M * K + 4 * K + 2 * K * r + M * K // 2 + 4 * M * G + 4 * M * r
