"""GPU parity of every step of the layer against the CPU oracle.

Bit-exact: packed codes, scales, per-group integer sums.  Tolerance: the
bf16 output within 1 bf16 ulp of |y_oracle| + 1e-3 rms(y_oracle); the fp32
down-projection within (2^-15 + K 2^-24) sum|xh L1| of the oracle's fp64.
All calls go through the C ABI (bit_diffusion_transformer_amd -> libsvdq.so).
"""
import numpy as np
import pytest
import torch

import bit_diffusion_transformer_amd as bdt
import oracle
from synth import LayerSpec, make_layer
from tests.helpers import (assert_y_close, bf16_host, from_pairs, from_stage_major, pdev, sdev,
                           to_dev, xl1_bound)

pytestmark = pytest.mark.gpu

# (M, K, N, r, act, bias): tiles of 128 in M and N, stages of 4 groups in K,
# ragged tails in every dimension, the extreme ranks, both activations.
SHAPES = [
    (256, 512, 512, 16, 0, True),
    (77, 192, 264, 32, 1, True),
    (1, 64, 8, 0, 0, False),
    (130, 320, 136, 48, 1, False),
    (300, 256, 256, 128, 0, True),
    (33, 128, 1024, 64, 1, True),
    (517, 1088, 392, 32, 0, True),
]


def _spec(M, K, N, r, act, bias, cid):
    return LayerSpec("t%d" % cid, M, K, N, r, 0.01, 20.0, min(4, r) if r else 2, False,
                     act=act, bias=bias, cfg_id=100 + cid)


@pytest.fixture(scope="module", params=list(enumerate(SHAPES)),
                ids=lambda p: "M%d_K%d_N%d_r%d_act%d_bias%d" % p[1])
def case(request):
    cid, (M, K, N, r, act, bias) = request.param
    L = make_layer(_spec(M, K, N, r, act, bias, cid))
    qa, sa, xh = oracle.quantize_act(L.X, L.lam)
    qw, sw = oracle.pack_weights(L.R)
    xl1 = oracle.down_proj(xh, L.L1) if r > 0 else None
    return dict(L=L, M=M, K=K, N=N, r=r, act=act, qa=qa, sa=sa, xh=xh, qw=qw, sw=sw, xl1=xl1)


def test_pack_weights_bit_exact(case):
    qw, sw = bdt.pack_weights(to_dev(case["L"].R))
    assert np.array_equal(from_pairs(qw, case["N"]), case["qw"])
    G = case["K"] // 64
    assert np.array_equal(from_stage_major(sw, case["N"], G).view(np.uint32),
                          case["sw"].view(np.uint32))


def _twos_complement_bytes(codes):
    """Integer codes [rows, K] -> the common row-major INT4 form: two's-complement nibbles,
    element 2j in the low nibble of byte j."""
    c = np.asarray(codes, np.int64)
    return ((c[:, 0::2] & 0xF) | ((c[:, 1::2] & 0xF) << 4)).astype(np.uint8)


def test_repack_weights_bit_exact(case):
    # codes of the oracle's quantization in the common row-major form -> the stored layout
    N, K = case["N"], case["K"]
    tc = _twos_complement_bytes(oracle.unpack(case["qw"], K))
    qw, sw = bdt.repack_weights(to_dev(tc), to_dev(case["sw"]))
    assert np.array_equal(from_pairs(qw, N), case["qw"])
    assert np.array_equal(from_stage_major(sw, N, K // 64).view(np.uint32),
                          case["sw"].view(np.uint32))


def test_quantize_act_down(case):
    L, r = case["L"], case["r"]
    qa, sa, xl1 = bdt.quantize_act_down(to_dev(L.X), to_dev(L.lam), to_dev(L.L1) if r else None)
    assert np.array_equal(from_pairs(qa, case["M"]), case["qa"])
    assert np.array_equal(from_stage_major(sa, case["M"], case["K"] // 64).view(np.uint32),
                          case["sa"].view(np.uint32))
    if r:
        got = xl1.cpu().numpy().astype(np.float64)
        assert np.all(np.abs(got - case["xl1"]) <= xl1_bound(case["xh"], L.L1))
    else:
        assert xl1 is None


@pytest.fixture(params=[bdt.TILES_FULL, bdt.TILES_QUARTER], ids=["full_tiles", "quarter_tiles"])
def tiles(request):
    bdt.svdq_debug_set_tile_policy(request.param)
    yield request.param
    bdt.svdq_debug_set_tile_policy(bdt.TILES_AUTO)


@pytest.fixture(params=[bdt.TILES_FULL, bdt.TILES_QUARTER, bdt.TILES_KSPLIT,
                        bdt.TILES_KSPLIT_QUARTER],
                ids=["full_tiles", "quarter_tiles", "ksplit_tiles", "ksplit_quarter_tiles"])
def all_tiles(request):
    bdt.svdq_debug_set_tile_policy(request.param)
    yield request.param
    bdt.svdq_debug_set_tile_policy(bdt.TILES_AUTO)


def test_group_sums_bit_exact(case, tiles):
    # the sums come out of the GEMM's own K loop (LDS ring, swizzle, row-pair copies,
    # odd-group tail stage) on 128 x 128 or 64 x 64 tiles
    M, N, K = case["M"], case["N"], case["K"]
    qa, qw = pdev(case["qa"]), pdev(case["qw"])
    sa, sw = sdev(case["sa"]), sdev(case["sw"])
    for (m0, tm, n0, tn) in [(0, M, 0, N), (M // 3, M - M // 3, N // 5, min(37, N - N // 5))]:
        S = bdt.group_sums(qa, sa, qw, sw, M, N, m0, n0, tm, tn).cpu().numpy()
        ref = oracle.group_sums(case["qa"], case["qw"], K, m0, n0, tm, tn)
        assert np.array_equal(S, ref)


def test_gemm_stagewise(case, all_tiles):
    # Same inputs on both sides: the oracle's codes/scales and its xl1 in fp32.
    L, r, K = case["L"], case["r"], case["K"]
    xl1_32 = case["xl1"].astype(np.float32) if r else None
    Y = bdt.w4a4_lr_gemm(pdev(case["qa"]), sdev(case["sa"]), pdev(case["qw"]),
                         sdev(case["sw"]), to_dev(xl1_32), to_dev(L.L2) if r else None,
                         to_dev(L.bias), case["act"])
    _, y_or = oracle.gemm_rows(case["qa"], case["sa"], case["qw"], case["sw"],
                               None if xl1_32 is None else xl1_32.astype(np.float64),
                               L.L2, L.bias, case["act"], K)
    assert_y_close(bf16_host(Y), y_or, "gemm")


def test_linear_end_to_end(case, all_tiles):
    L, r = case["L"], case["r"]
    Y = bdt.linear(to_dev(L.X), to_dev(L.lam), to_dev(L.L1) if r else None, pdev(case["qw"]),
                   sdev(case["sw"]), to_dev(L.L2) if r else None, to_dev(L.bias), case["act"])
    _, y_or = oracle.linear(L.X, L.lam, L.L1 if r else None, case["qw"], case["sw"],
                            L.L2 if r else None, L.bias, case["act"])
    assert_y_close(bf16_host(Y), y_or, "linear")


def test_linear_is_deterministic(case):
    L, r = case["L"], case["r"]
    args = (to_dev(L.X), to_dev(L.lam), to_dev(L.L1) if r else None, pdev(case["qw"]),
            sdev(case["sw"]), to_dev(L.L2) if r else None, to_dev(L.bias), case["act"])
    y1 = bf16_host(bdt.linear(*args))
    y2 = bf16_host(bdt.linear(*args))
    assert np.array_equal(y1, y2)


def test_tile_policies_agree_bit_exact(case):
    # 128 x 128 and 64 x 64 tiles run the same per-output arithmetic in the same order, and
    # so do the two k-split shapes (the same split of K, then acc0 + acc1); the default
    # picks one of the two families
    L, r = case["L"], case["r"]
    args = (to_dev(L.X), to_dev(L.lam), to_dev(L.L1) if r else None, pdev(case["qw"]),
            sdev(case["sw"]), to_dev(L.L2) if r else None, to_dev(L.bias), case["act"])
    out = {}
    try:
        for pol in (bdt.TILES_FULL, bdt.TILES_QUARTER, bdt.TILES_KSPLIT, bdt.TILES_KSPLIT_QUARTER,
                    bdt.TILES_AUTO):
            bdt.svdq_debug_set_tile_policy(pol)
            out[pol] = bf16_host(bdt.linear(*args))
    finally:
        bdt.svdq_debug_set_tile_policy(bdt.TILES_AUTO)
    assert np.array_equal(out[bdt.TILES_FULL], out[bdt.TILES_QUARTER])
    assert np.array_equal(out[bdt.TILES_KSPLIT], out[bdt.TILES_KSPLIT_QUARTER])
    assert (np.array_equal(out[bdt.TILES_AUTO], out[bdt.TILES_FULL])
            or np.array_equal(out[bdt.TILES_AUTO], out[bdt.TILES_KSPLIT]))
