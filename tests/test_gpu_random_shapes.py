"""GPU parity of the whole layer on seeded random shapes, under the automatic tile choice.

The shapes are drawn (seeded) so that the automatic tile policy takes each of its branches:
k-split 64x64 tiles (at most one 64x64 tile per compute unit), all 64x64 tiles (a single
partial round), and 128x128 tiles with or without a 64x64 tail; ragged M and N, odd and even
group counts, every rank the layer takes up to 64, both activations, with and without bias.
Each output is compared element by element with the oracle (1 bf16 ulp + 1e-3 rms over the
whole output), and the automatic choice must equal one of the two tile families bit for bit.
All calls go through the C ABI.
"""
import numpy as np
import pytest

import bit_diffusion_transformer_amd as bdt
import oracle
from synth import LayerSpec, make_layer
from tests.helpers import assert_y_close, bf16_host, pdev, sdev, to_dev

pytestmark = pytest.mark.gpu


def _shapes(n=16, seed=2024):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        # a spread of grid sizes: tiny (k-split), medium (all 64x64) and a few full rounds
        M = int(rng.choice([int(rng.integers(1, 65)), int(rng.integers(65, 700)),
                            int(rng.integers(700, 2200))], p=[0.3, 0.45, 0.25]))
        N = 8 * int(rng.integers(1, 200)) if M < 700 else 8 * int(rng.integers(100, 400))
        K = 64 * int(rng.integers(1, 24))
        r = int(rng.choice([0, 16, 32, 48, 64]))
        act = int(rng.integers(0, 2))
        bias = bool(rng.integers(0, 2))
        out.append((M, K, N, r, act, bias))
    # and the two 128x128 families: a partial round above a quarter of the slots (full
    # tiles only), and a whole round plus a 64-tile tail (run as 64x64 quadrants)
    out += [(2300, 128, 3072, 32, 1, True), (1020, 192, 9216, 16, 0, True)]
    return out


SHAPES = _shapes()


@pytest.mark.parametrize("i,shape", list(enumerate(SHAPES)),
                         ids=["M%d_K%d_N%d_r%d_act%d_bias%d" % s for s in SHAPES])
def test_random_shape_matches_oracle(i, shape):
    M, K, N, r, act, bias = shape
    spec = LayerSpec("rnd%d" % i, M, K, N, r, 0.01, 20.0, min(4, r) if r else 2, False,
                     act=act, bias=bias, cfg_id=700 + i)
    L = make_layer(spec)
    qw_o, sw_o = oracle.pack_weights(L.R)
    args = (to_dev(L.X), to_dev(L.lam), to_dev(L.L1) if r else None, pdev(qw_o), sdev(sw_o),
            to_dev(L.L2) if r else None, to_dev(L.bias), act)
    print("shape M=%d K=%d N=%d r=%d act=%d bias=%d" % shape, flush=True)
    out = {}
    try:
        for pol in (bdt.TILES_AUTO, bdt.TILES_FULL, bdt.TILES_KSPLIT):
            bdt.svdq_debug_set_tile_policy(pol)
            out[pol] = bf16_host(bdt.linear(*args))
    finally:
        bdt.svdq_debug_set_tile_policy(bdt.TILES_AUTO)
    _, y_or = oracle.linear(L.X, L.lam, L.L1 if r else None, qw_o, sw_o, L.L2 if r else None,
                            L.bias, act)
    worst = assert_y_close(out[bdt.TILES_AUTO], y_or, "random shape %d" % i)
    assert (np.array_equal(out[bdt.TILES_AUTO], out[bdt.TILES_FULL])
            or np.array_equal(out[bdt.TILES_AUTO], out[bdt.TILES_KSPLIT]))
    print("  worst |err|/tol = %.3f" % worst, flush=True)
