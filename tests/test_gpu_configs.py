"""Parity at the full workload sizes, through svdq_linear as the benchmark calls it.

Codes and scales are compared in full (bit-exact), the down-projection in
full (error bound), the output Y in full (every element; tolerance 1 bf16 ulp
+ 1e-3 rms with the rms taken over the whole output), and the per-group sums
bit-exact on sampled tiles -- the first, the last (ragged edges) and a random
one -- taken from the GEMM's own K loop on 128 x 128 and on 64 x 64 tiles.
"""
import numpy as np
import pytest

import bit_diffusion_transformer_amd as bdt
import oracle
from synth import CONFIGS, DIT_CHAIN, make_layer
from tests.helpers import assert_y_close, bf16_host, from_pairs, from_stage_major, to_dev, xl1_bound

pytestmark = pytest.mark.gpu

CASES = [("tiny", CONFIGS["tiny"], None), ("qkv", CONFIGS["qkv"], None),
         ("mlp_up", CONFIGS["mlp_up"], None), ("mlp_down", CONFIGS["mlp_down"], None)]
CASES += [("chain%d_%s" % (M, s.name), s, M) for M in (4608, 256) for s in DIT_CHAIN]


def _sample_blocks(M, N, rng):
    """(m0, tm, n0, tn): the first tile, the last (ragged) tile, one random tile."""
    tm, tn = min(128, M), min(128, N)
    out = [(0, tm, 0, tn), (M - tm, tm, N - tn, tn)]
    out.append((int(rng.integers(0, M - tm + 1)), tm, int(rng.integers(0, N - tn + 1)), tn))
    return out


@pytest.mark.parametrize("name,spec,M", CASES, ids=[c[0] for c in CASES])
def test_full_size_config(name, spec, M):
    L = make_layer(spec, seed=0, M=M)
    M, K, N, r, act = L.spec.M, L.spec.K, L.spec.N, L.spec.r, L.spec.act
    print("config %s M=%d K=%d N=%d r=%d act=%d" % (name, M, K, N, r, act), flush=True)

    qw_o, sw_o = oracle.pack_weights(L.R)
    qw, sw = bdt.pack_weights(to_dev(L.R))
    assert np.array_equal(from_pairs(qw, N), qw_o)
    assert np.array_equal(from_stage_major(sw, N, K // 64).view(np.uint32), sw_o.view(np.uint32))

    X, lam, L1, L2, bias = to_dev(L.X), to_dev(L.lam), to_dev(L.L1), to_dev(L.L2), to_dev(L.bias)
    qa_o, sa_o, xh = oracle.quantize_act(L.X, L.lam)
    qa, sa, xl1 = bdt.quantize_act_down(X, lam, L1)
    assert np.array_equal(from_pairs(qa, M), qa_o)
    assert np.array_equal(from_stage_major(sa, M, K // 64).view(np.uint32), sa_o.view(np.uint32))
    xl1_o = oracle.down_proj(xh, L.L1)
    assert np.all(np.abs(xl1.cpu().numpy().astype(np.float64) - xl1_o) <= xl1_bound(xh, L.L1))

    rng = np.random.default_rng(7)
    try:
        for pol in (bdt.TILES_FULL, bdt.TILES_QUARTER):
            bdt.svdq_debug_set_tile_policy(pol)
            for (m0, tm, n0, tn) in _sample_blocks(M, N, rng):
                S = bdt.group_sums(qa, sa, qw, sw, M, N, m0, n0, tm, tn).cpu().numpy()
                assert np.array_equal(S, oracle.group_sums(qa_o, qw_o, K, m0, n0, tm, tn)), \
                    "group sums differ at block (%d, %d) under tile policy %d" % (m0, n0, pol)
    finally:
        bdt.svdq_debug_set_tile_policy(bdt.TILES_AUTO)

    Y = bdt.linear(X, lam, L1, qw, sw, L2, bias, act)
    _, y_or = oracle.linear(L.X, L.lam, L.L1, qw_o, sw_o, L.L2, L.bias, act)
    worst = assert_y_close(bf16_host(Y), y_or, name)
    print("  worst |err|/tol = %.3f over all %d x %d outputs" % (worst, M, N), flush=True)
