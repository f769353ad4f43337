"""GPU parity of the W4A16 (awq_w4a16) layer against the CPU oracle.

Bit-exact: the packed records (codes, scales and zero points of the weight
quantizer, placed as documented in svdq.h; expected bytes built on the host
from the oracle's row-major output) and the repacking of row-major weights.
Tolerance: the bf16 output within 1 bf16 ulp of |y_oracle| + 1e-3 rms(y_oracle).
All calls go through the C ABI (bit_diffusion_transformer_amd -> libsvdq.so).
"""
import numpy as np
import pytest
import torch

import bit_diffusion_transformer_amd as bdt
import oracle
from synth import AWQ_CONFIGS, AwqSpec, make_awq_layer
from tests.helpers import assert_y_close, awq_records, bf16_host, to_dev

pytestmark = pytest.mark.gpu

# (M, K, N, bias): column blocks of 16 with N % 16 == 8, K quads of 4 groups
# with ragged group counts (1, 3, 5), fewer quads than waves, several row
# passes, and the full-width modulation shape.
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
    return dict(L=L, M=M, K=K, N=N, q=q, s=s, z=z, rec=awq_records(q, s, z, N, K))


def test_awq_packed_bytes(case):
    N, K = case["N"], case["K"]
    assert bdt.svdq_awq_packed_bytes(N, K) == case["rec"].size
    assert bdt.svdq_awq_packed_bytes(N, K) == ((N + 15) // 16) * ((K // 64 + 3) // 4) * 2368


def test_awq_pack_bit_exact(case):
    packed = bdt.awq_pack_weights(to_dev(case["L"].W))
    assert np.array_equal(packed.cpu().numpy(), case["rec"])


def test_awq_repack_bit_exact(case):
    packed = bdt.awq_repack(to_dev(case["q"]), to_dev(case["s"]), to_dev(case["z"]))
    assert np.array_equal(packed.cpu().numpy(), case["rec"])


def test_awq_linear(case):
    L = case["L"]
    Y = bdt.awq_linear(to_dev(L.X), to_dev(case["rec"]), case["N"], to_dev(L.bias))
    _, y_or = oracle.awq_linear(L.X, case["q"], case["s"], case["z"], L.bias)
    assert_y_close(bf16_host(Y), y_or, "awq")


def test_awq_linear_deterministic(case):
    L = case["L"]
    args = (to_dev(L.X), to_dev(case["rec"]), case["N"], to_dev(L.bias))
    assert np.array_equal(bf16_host(bdt.awq_linear(*args)), bf16_host(bdt.awq_linear(*args)))


def test_awq_zero_weights_give_bias():
    M, K, N = 3, 128, 64
    packed = bdt.awq_pack_weights(torch.zeros((N, K), dtype=torch.float32, device="cuda:0"))
    assert torch.all(packed == 0)
    L = make_awq_layer(AwqSpec("z", M, K, N, True, cfg_id=230))
    Y = bdt.awq_linear(to_dev(L.X), packed, N, to_dev(L.bias))
    assert np.array_equal(bf16_host(Y), np.broadcast_to(L.bias, (M, N)))


def test_awq_full_size_workload():
    spec = AWQ_CONFIGS["awq_mod"]
    L = make_awq_layer(spec)
    q, s, z = oracle.awq_quantize(L.W)
    packed = bdt.awq_pack_weights(to_dev(L.W))
    assert np.array_equal(packed.cpu().numpy(), awq_records(q, s, z, spec.N, spec.K))
    Y = bdt.awq_linear(to_dev(L.X), packed, spec.N, to_dev(L.bias))
    _, y_or = oracle.awq_linear(L.X, q, s, z, L.bias)
    worst = assert_y_close(bf16_host(Y), y_or, spec.name)
    print("  awq_mod worst |err|/tol = %.3f" % worst, flush=True)
