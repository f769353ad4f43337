"""svdq_linear_noalloc (the allocation-free entry point, intermediates in the library's
static per-device scratch) against svdq_linear with a caller workspace: bitwise identical
outputs on two calls in a row, the second on a smaller input, so that the second call runs
over the first call's leftovers in the shared scratch."""
import numpy as np
import pytest
import torch

import bit_diffusion_transformer_amd as bdt
from synth import LayerSpec, make_layer
from tests.helpers import bf16_host, to_dev

pytestmark = pytest.mark.gpu


def _layer(M, K, N, r, act, cid):
    spec = LayerSpec("noalloc%d" % cid, M, K, N, r, 0.01, 20.0, 4, False, act=act, cfg_id=300 + cid)
    return make_layer(spec)


def _both(L):
    M, K, N, r, act = L.spec.M, L.spec.K, L.spec.N, L.spec.r, L.spec.act
    X, lam, L1, L2, bias = to_dev(L.X), to_dev(L.lam), to_dev(L.L1), to_dev(L.L2), to_dev(L.bias)
    qw, sw = bdt.pack_weights(to_dev(L.R))
    ref = bdt.linear(X, lam, L1, qw, sw, L2, bias, act)
    Y = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda:0")
    b = bdt._bits
    bdt.svdq_linear_noalloc(b(X), lam, b(L1) if r else None, qw, sw, b(L2) if r else None,
                            b(bias), act, M, N, K, r, b(Y))
    torch.cuda.synchronize()
    return bf16_host(Y), bf16_host(ref)


def test_noalloc_matches_linear_twice_second_smaller():
    # first a layer whose K spans several down-projection chunks (partial sums in the
    # scratch), then a smaller one
    big = _layer(1030, 1600, 776, 32, 1, 1)
    small = _layer(77, 320, 264, 16, 0, 2)
    for L in (big, small):
        got, want = _both(L)
        assert np.array_equal(got, want), "noalloc differs from svdq_linear at M=%d" % L.spec.M


def test_noalloc_rejects_oversized_shape_without_launch():
    M, K, N, r = 1 << 20, 3072, 3072, 32
    assert bdt.svdq_linear_workspace_bytes(M, K, r) > bdt._binding.NOALLOC_SCRATCH_BYTES
    t = torch.zeros(64, dtype=torch.uint8, device="cuda:0")   # never read: refused first
    with pytest.raises(bdt.SVDQError):
        bdt.svdq_linear_noalloc(t, t, t, t, t, t, None, 0, M, N, K, r, t)
