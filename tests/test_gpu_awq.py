"""GPU parity of the W4A16 (awq_w4a16) layer against the CPU oracle.

Bit-exact: codes, scales and zero points of the weight quantizer.
Tolerance: the bf16 output within 1 bf16 ulp of |y_oracle| + 1e-3 rms(y_oracle).
All calls go through the C ABI (bit_diffusion_transformer_amd -> libsvdq.so).
"""
import numpy as np
import pytest
import torch

import bit_diffusion_transformer_amd as bdt
import oracle
from synth import AWQ_CONFIGS, AwqSpec, make_awq_layer
from tests.helpers import assert_y_close, bf16_host, to_dev

pytestmark = pytest.mark.gpu

# (M, K, N, bias): 16-row and 16-column tiles, four K quarters, ragged M, N
# and K (odd group counts, N % 16 == 8), one and several row tiles.
SHAPES = [
    (1, 64, 8, False),
    (2, 192, 264, True),
    (5, 320, 136, True),
    (17, 1024, 392, False),
    (33, 3072, 1024, True),
    (2, 3072, 18432, True),
]


@pytest.fixture(scope="module", params=list(enumerate(SHAPES)),
                ids=lambda p: "M%d_K%d_N%d_bias%d" % p[1])
def case(request):
    cid, (M, K, N, bias) = request.param
    L = make_awq_layer(AwqSpec("t%d" % cid, M, K, N, bias, cfg_id=200 + cid))
    q, s, z = oracle.awq_quantize(L.W)
    return dict(L=L, M=M, K=K, N=N, q=q, s=s, z=z)


def test_awq_pack_bit_exact(case):
    qw, sc, zp = bdt.awq_pack_weights(to_dev(case["L"].W))
    assert np.array_equal(qw.cpu().numpy(), case["q"])
    assert np.array_equal(sc.cpu().numpy().view(np.uint32), case["s"].view(np.uint32))
    assert np.array_equal(zp.cpu().numpy(), case["z"])


def test_awq_linear(case):
    L = case["L"]
    Y = bdt.awq_linear(to_dev(L.X), to_dev(case["q"]), to_dev(case["s"]), to_dev(case["z"]),
                       to_dev(L.bias))
    _, y_or = oracle.awq_linear(L.X, case["q"], case["s"], case["z"], L.bias)
    assert_y_close(bf16_host(Y), y_or, "awq")


def test_awq_linear_deterministic(case):
    L = case["L"]
    args = (to_dev(L.X), to_dev(case["q"]), to_dev(case["s"]), to_dev(case["z"]), to_dev(L.bias))
    assert np.array_equal(bf16_host(bdt.awq_linear(*args)), bf16_host(bdt.awq_linear(*args)))


def test_awq_zero_weights_give_bias():
    M, K, N = 3, 128, 64
    W = torch.zeros((N, K), dtype=torch.float32, device="cuda:0")
    qw, sc, zp = bdt.awq_pack_weights(W)
    assert torch.all(sc == 0) and torch.all(zp == 0) and torch.all(qw == 0)
    L = make_awq_layer(AwqSpec("z", M, K, N, True, cfg_id=230))
    Y = bdt.awq_linear(to_dev(L.X), qw, sc, zp, to_dev(L.bias))
    assert np.array_equal(bf16_host(Y), np.broadcast_to(L.bias, (M, N)))


def test_awq_full_size_workload():
    spec = AWQ_CONFIGS["awq_mod"]
    L = make_awq_layer(spec)
    qw, sc, zp = bdt.awq_pack_weights(to_dev(L.W))
    q, s, z = oracle.awq_quantize(L.W)
    assert np.array_equal(qw.cpu().numpy(), q)
    Y = bdt.awq_linear(to_dev(L.X), qw, sc, zp, to_dev(L.bias))
    _, y_or = oracle.awq_linear(L.X, q, s, z, L.bias)
    worst = assert_y_close(bf16_host(Y), y_or, spec.name)
    print("  awq_mod worst |err|/tol = %.3f" % worst, flush=True)
