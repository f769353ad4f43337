"""GPU parity of the fused QKV epilogue (W4A4 GEMM -> per-head RMS norm + rotary turn
of Q and K, attention layout) against the CPU oracle.

Q and K: within 1 bf16 ulp plus the GEMM tolerance (1e-3 rms of the projection)
propagated through the norm and the turn (tests.helpers.qkv_tolerance).  V: the
GEMM tolerance, and bit-identical to the plain GEMM's V columns re-laid out.
All calls go through the C ABI (bit_diffusion_transformer_amd -> libsvdq.so).
"""
import numpy as np
import pytest
import torch

import bit_diffusion_transformer_amd as bdt
import oracle
from synth import CONFIGS, LayerSpec, make_layer, make_qkv_epilogue
from tests.helpers import assert_y_close, bf16_f64, bf16_host, pdev, qkv_tolerance, sdev, to_dev

pytestmark = pytest.mark.gpu

# (B, S, H, D, K, r, bias): one and two heads per tile (D = 128 / 64), ragged
# token counts (sequences straddling 128-row tiles, a last tile of one row),
# odd group counts, r = 0, and sequences shorter than 8 tokens (positions wrap
# several times within the 8 tokens a lane steps over when it fetches the
# rotary rows; S = 1: every token at position 0).
SHAPES = [
    (1, 96, 2, 64, 256, 16, True),
    (2, 80, 2, 128, 320, 32, True),
    (3, 50, 4, 64, 512, 0, False),
    (1, 257, 1, 128, 192, 48, True),
    (40, 5, 2, 64, 128, 16, True),
    (43, 3, 1, 128, 128, 0, False),
    (130, 1, 2, 64, 192, 32, True),
]


def _layer(B, S, H, D, K, r, bias, cid):
    M, N = B * S, 3 * H * D
    spec = LayerSpec("q%d" % cid, M, K, N, r, 0.01, 20.0, min(4, r) if r else 2, False,
                     act=0, bias=bias, cfg_id=300 + cid)
    return make_layer(spec)


def _oracle(L, epi, rows=None):
    qa, sa, xh = oracle.quantize_act(L.X, L.lam)
    qw, sw = oracle.pack_weights(L.R)
    r = L.L1.shape[1] if L.L1 is not None else 0
    xl1 = oracle.down_proj(xh, L.L1) if r > 0 else None
    acc, y = oracle.gemm_rows(qa, sa, qw, sw, xl1, L.L2 if r else None, L.bias, 0, L.X.shape[1],
                              rows)
    o = oracle.qkv_epilogue(acc, epi.heads, epi.head_dim, epi.seq, epi.gamma_q, epi.gamma_k,
                            epi.eps, epi.cos_t, epi.sin_t, rows)
    return dict(qa=qa, sa=sa, qw=qw, sw=sw, xl1=xl1, acc=acc, y=y, o=o)


def _bhsd_rows(t: torch.Tensor, rows, S):
    """[B, H, S, D] bf16 -> host bits of the given tokens, [R, H, D]."""
    a = bf16_host(t)
    rows = np.asarray(rows)
    return a[rows // S, :, rows % S, :]


def _check(Q, Kt, V, orc, epi, rows, what):
    H, D, S = epi.heads, epi.head_dim, epi.seq
    HD = H * D
    acc = orc["acc"]
    rms = float(np.sqrt(np.mean(acc ** 2)))
    worst = 0.0
    for sec, T, key, gam in ((0, Q, "q", epi.gamma_q), (1, Kt, "k", epi.gamma_k)):
        got = bf16_f64(_bhsd_rows(T, rows, S))
        x = acc[:, sec * HD:(sec + 1) * HD].reshape(-1, H, D)
        ob = dict(o=orc["o"][key], rho=orc["o"]["rho_" + key])
        tol = qkv_tolerance(ob, x, gam, 1e-3 * rms)
        err = np.abs(got - ob["o"])
        bad = err > tol
        assert not bad.any(), "%s %s: %d of %d beyond the bound, worst %.3g (tol %.3g)" % (
            what, key, bad.sum(), bad.size, err[bad].max(), tol[bad][np.argmax(err[bad])])
        worst = max(worst, float((err / tol).max()))
    vb = _bhsd_rows(V, rows, S).reshape(len(rows), HD)
    assert_y_close(vb, orc["o"]["vb"].reshape(len(rows), HD), what + " v", rms=rms)
    return worst


@pytest.fixture(scope="module", params=list(enumerate(SHAPES)),
                ids=lambda p: "B%d_S%d_H%d_D%d_K%d_r%d_bias%d" % p[1])
def case(request):
    cid, (B, S, H, D, K, r, bias) = request.param
    L = _layer(B, S, H, D, K, r, bias, cid)
    epi = make_qkv_epilogue(H, D, S, cfg_id=310 + cid)
    return dict(L=L, epi=epi, B=B, S=S, H=H, D=D, K=K, r=r, orc=_oracle(L, epi))


def _dev_epi(epi):
    return dict(gamma_q=to_dev(epi.gamma_q), gamma_k=to_dev(epi.gamma_k), eps=epi.eps,
                cos_t=to_dev(epi.cos_t), sin_t=to_dev(epi.sin_t))


def _xl1_32(o, r):
    # the oracle's fp64 down-projection handed to the GPU as the fp32 it takes
    return to_dev(o["xl1"].astype(np.float32)) if r else None


def _gemm_qkv(case):
    o, L, epi, r = case["orc"], case["L"], case["epi"], case["r"]
    return bdt.w4a4_lr_gemm_qkv(pdev(o["qa"]), sdev(o["sa"]), pdev(o["qw"]), sdev(o["sw"]),
                                _xl1_32(o, r), to_dev(L.L2) if r else None,
                                to_dev(L.bias), epi.heads, epi.head_dim, epi.seq,
                                **_dev_epi(epi))


def test_gemm_qkv_matches_oracle(case):
    Q, Kt, V = _gemm_qkv(case)
    M = case["B"] * case["S"]
    assert Q.shape == (case["B"], case["H"], case["S"], case["D"])
    worst = _check(Q, Kt, V, case["orc"], case["epi"], np.arange(M), "gemm_qkv")
    print("  worst |err|/bound = %.3f" % worst, flush=True)


def test_linear_qkv_matches_oracle(case):
    L, epi, r = case["L"], case["epi"], case["r"]
    Q, Kt, V = bdt.linear_qkv(to_dev(L.X), to_dev(L.lam), to_dev(L.L1) if r else None,
                              pdev(case["orc"]["qw"]), sdev(case["orc"]["sw"]),
                              to_dev(L.L2) if r else None, to_dev(L.bias), epi.heads,
                              epi.head_dim, epi.seq, **_dev_epi(epi))
    _check(Q, Kt, V, case["orc"], epi, np.arange(case["B"] * case["S"]), "linear_qkv")


def test_v_equals_plain_gemm_columns(case):
    """V comes from the same tile arithmetic as the plain GEMM on whole-K tiles (not the
    k-split tiles the plain GEMM picks for small grids, which add two partial sums):
    bit-identical."""
    o, L, r = case["orc"], case["L"], case["r"]
    _, _, V = _gemm_qkv(case)
    bdt.svdq_debug_set_tile_policy(bdt.TILES_FULL)
    try:
        Y = bdt.w4a4_lr_gemm(pdev(o["qa"]), sdev(o["sa"]), pdev(o["qw"]), sdev(o["sw"]),
                             _xl1_32(o, r), to_dev(L.L2) if r else None, to_dev(L.bias), 0)
    finally:
        bdt.svdq_debug_set_tile_policy(bdt.TILES_AUTO)
    B, S, H, D = case["B"], case["S"], case["H"], case["D"]
    y = bf16_host(Y)[:, 2 * H * D:].reshape(B, S, H, D).transpose(0, 2, 1, 3)
    assert np.array_equal(bf16_host(V), y)


def test_deterministic(case):
    a = [bf16_host(t) for t in _gemm_qkv(case)]
    b = [bf16_host(t) for t in _gemm_qkv(case)]
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def test_qkv_full_size_sampled():
    """The qkv workload (M = 4608 tokens, K = 3072, 24 heads of 128) in the launch
    configuration bench.py times; Q/K/V of 24 sampled tokens against the oracle."""
    spec = CONFIGS["qkv"]
    L = make_layer(spec)
    H, D, S = 24, 128, spec.M
    epi = make_qkv_epilogue(H, D, S, cfg_id=330)
    rng = np.random.default_rng(5)
    rows = np.sort(np.concatenate([[0, 127, 128, S - 1], rng.choice(S, 20, replace=False)]))
    orc = _oracle(L, epi, rows)
    qw, sw = bdt.pack_weights(to_dev(L.R))
    Q, Kt, V = bdt.linear_qkv(to_dev(L.X), to_dev(L.lam), to_dev(L.L1), qw, sw, to_dev(L.L2),
                              to_dev(L.bias), H, D, S, **_dev_epi(epi))
    worst = _check(Q, Kt, V, orc, epi, rows, "qkv full")
    print("  qkv full size worst |err|/bound = %.3f" % worst, flush=True)


def test_tile_policies_agree_bit_exact(case):
    """V tiles as 64 x 64 quarter tiles (the partial-last-round path) give the same bits."""
    out = {}
    for pol in (bdt.TILES_FULL, bdt.TILES_QUARTER):
        bdt.svdq_debug_set_tile_policy(pol)
        try:
            out[pol] = [bf16_host(t) for t in _gemm_qkv(case)]
        finally:
            bdt.svdq_debug_set_tile_policy(bdt.TILES_AUTO)
    for a, b in zip(out[bdt.TILES_FULL], out[bdt.TILES_QUARTER]):
        assert np.array_equal(a, b)
    M = case["B"] * case["S"]
    bdt.svdq_debug_set_tile_policy(bdt.TILES_QUARTER)
    try:
        Q, Kt, V = _gemm_qkv(case)
    finally:
        bdt.svdq_debug_set_tile_policy(bdt.TILES_AUTO)
    _check(Q, Kt, V, case["orc"], case["epi"], np.arange(M), "gemm_qkv quarter V tiles")
