"""GPU parity of the MLP chain fusion: the up-projection GEMM whose epilogue runs the
down layer's activation step (smoothing, INT4 codes and scales, partial X L1 reduced in
column order), and the whole MLP (svdq_mlp).

Bit-exact: the next layer's codes and scales against the oracle's quantizer applied to
the bf16 output the plain GEMM stores (the fused kernel computes that same value in its
epilogue).  xl1 within (2^-15 + K 2^-24) sum|x^ L1| of the oracle's fp64 value.  The
MLP output within 1 bf16 ulp + 1e-3 rms of the oracle's down layer applied to that
same intermediate.  All calls go through the C ABI (libsvdq.so).
"""
import numpy as np
import pytest
import torch

import bit_diffusion_transformer_amd as bdt
import oracle
from synth import DIT_CHAIN, LayerSpec, make_layer
from tests.helpers import (assert_y_close, bf16_host, from_pairs, from_stage_major, pdev, sdev,
                           to_dev, xl1_bound)

pytestmark = pytest.mark.gpu

# (M, K, Nh, r_up, r_down, act, bias): 128-column tiles (Nh % 128 == 0), ragged M,
# odd group counts in K, both activations, next-layer ranks 0 / 16 / 32.
SHAPES = [
    (256, 512, 512, 16, 32, 1, True),
    (77, 192, 384, 32, 16, 1, True),
    (130, 320, 256, 0, 0, 0, False),
    (300, 256, 640, 48, 32, 1, True),
]


def _pair(M, K, Nh, ru, rd, act, bias, cid):
    up = make_layer(LayerSpec("u%d" % cid, M, K, Nh, ru, 0.01, 20.0, min(4, ru) if ru else 2,
                              False, act=act, bias=bias, cfg_id=400 + cid, layer_id=0))
    down = make_layer(LayerSpec("d%d" % cid, M, Nh, K, rd, 0.01, 10.0, min(4, rd) if rd else 2,
                                False, x_gelu=True, bias=bias, cfg_id=400 + cid, layer_id=1))
    return up, down


def _dev_layer(L, r):
    qw, sw = oracle.pack_weights(L.R)
    return dict(lam=to_dev(L.lam), L1=to_dev(L.L1) if r else None, L2=to_dev(L.L2) if r else None,
                bias=to_dev(L.bias), qw=pdev(qw), sw=sdev(sw))


@pytest.fixture(scope="module", params=list(enumerate(SHAPES)),
                ids=lambda p: "M%d_K%d_Nh%d_ru%d_rd%d_act%d_bias%d" % p[1])
def case(request):
    cid, (M, K, Nh, ru, rd, act, bias) = request.param
    up, down = _pair(M, K, Nh, ru, rd, act, bias, cid)
    qa, sa, xh = oracle.quantize_act(up.X, up.lam)
    xl1 = oracle.down_proj(xh, up.L1) if ru else None
    return dict(M=M, K=K, Nh=Nh, ru=ru, rd=rd, act=act, up=up, down=down, qa=qa, sa=sa, xl1=xl1,
                U=_dev_layer(up, ru), D=_dev_layer(down, rd))


def _up_operands(case):
    ru = case["ru"]
    return (pdev(case["qa"]), sdev(case["sa"]), case["U"]["qw"], case["U"]["sw"],
            to_dev(case["xl1"].astype(np.float32)) if ru else None, case["U"]["L2"],
            case["U"]["bias"])


def test_gemm_quant_down_matches_quantizer_of_plain_output(case):
    ops = _up_operands(case)
    D, rd = case["D"], case["rd"]
    # what the plain GEMM stores on whole-K tiles (the fused kernel's tile arithmetic; the
    # k-split tiles the plain GEMM picks for small grids add two partial sums instead)
    bdt.svdq_debug_set_tile_policy(bdt.TILES_FULL)
    try:
        h = bf16_host(bdt.w4a4_lr_gemm(*ops, case["act"]))
    finally:
        bdt.svdq_debug_set_tile_policy(bdt.TILES_AUTO)
    qa_n, sa_n, xl1_n = bdt.w4a4_lr_gemm_quant_down(*ops, case["act"], D["lam"], D["L1"])
    qa_o, sa_o, xh = oracle.quantize_act(h, case["down"].lam)
    assert np.array_equal(from_pairs(qa_n, case["M"]), qa_o)
    assert np.array_equal(from_stage_major(sa_n, sa_o.shape[0], sa_o.shape[1]).view(np.uint32),
                          sa_o.view(np.uint32))
    if rd:
        want = oracle.down_proj(xh, case["down"].L1)
        got = xl1_n.cpu().numpy().astype(np.float64)
        assert np.all(np.abs(got - want) <= xl1_bound(xh, case["down"].L1))
    else:
        assert xl1_n is None


def test_gemm_quant_down_deterministic(case):
    ops = _up_operands(case)
    D = case["D"]
    a = bdt.w4a4_lr_gemm_quant_down(*ops, case["act"], D["lam"], D["L1"])
    b = bdt.w4a4_lr_gemm_quant_down(*ops, case["act"], D["lam"], D["L1"])
    # codes compared as rows: an odd M leaves the last pair's second half unwritten
    assert np.array_equal(from_pairs(a[0], case["M"]), from_pairs(b[0], case["M"]))
    for x, y in zip(a[1:], b[1:]):
        if x is not None:
            assert torch.equal(x, y)


def test_mlp_matches_oracle_down_layer_of_the_intermediate(case):
    U, D, act = case["U"], case["D"], case["act"]
    X = to_dev(case["up"].X)
    Y = bdt.mlp(X, U, D, act)
    # the intermediate svdq_linear stores for the up layer
    h = bf16_host(bdt.linear(X, U["lam"], U["L1"], U["qw"], U["sw"], U["L2"], U["bias"], act))
    dn = case["down"]
    qw_d, sw_d = oracle.pack_weights(dn.R)
    _, y_or = oracle.linear(h, dn.lam, dn.L1 if case["rd"] else None, qw_d, sw_d,
                            dn.L2 if case["rd"] else None, dn.bias, 0)
    worst = assert_y_close(bf16_host(Y), y_or, "mlp")
    # and the unfused GPU chain (svdq_linear twice) agrees to the same band
    Y2 = bdt.linear(to_dev(h), D["lam"], D["L1"], D["qw"], D["sw"], D["L2"], D["bias"], 0)
    assert_y_close(bf16_host(Y2), y_or, "unfused chain")
    print("  mlp worst |err|/tol = %.3f" % worst, flush=True)


def test_mlp_full_size_sampled():
    """One DiT block's MLP (3072 -> 12288 GELU -> 3072, rank 32) at 256 and 4608 tokens,
    checked on sampled rows (all columns) against the oracle's down layer."""
    up_s, dn_s = DIT_CHAIN[2], DIT_CHAIN[3]
    for M, nrows in ((256, 32), (4608, 16)):
        up, dn = make_layer(up_s, M=M), make_layer(dn_s, M=M)
        U, D = _dev_layer(up, up_s.r), _dev_layer(dn, dn_s.r)
        X = to_dev(up.X)
        Y = bf16_host(bdt.mlp(X, U, D, 1))
        h = bf16_host(bdt.linear(X, U["lam"], U["L1"], U["qw"], U["sw"], U["L2"], U["bias"], 1))
        rows = np.sort(np.random.default_rng(9).choice(M, nrows, replace=False))
        qw_d, sw_d = oracle.pack_weights(dn.R)
        _, y_or = oracle.linear(np.ascontiguousarray(h[rows]), dn.lam, dn.L1, qw_d, sw_d, dn.L2,
                                dn.bias, 0)
        worst = assert_y_close(Y[rows], y_or, "mlp M=%d" % M)
        print("  mlp M=%d worst |err|/tol = %.3f" % (M, worst), flush=True)
