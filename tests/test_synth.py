"""The seeded input generator: reproducible, and built by its stated recipe."""
import numpy as np

from synth import CONFIGS, LayerSpec, bf16_bits_to_f32, make_layer


def test_reproducible_bit_for_bit():
    a = make_layer(CONFIGS["tiny"], seed=0)
    b = make_layer(CONFIGS["tiny"], seed=0)
    for f in ("X", "lam", "L1", "L2", "R", "bias"):
        assert np.array_equal(getattr(a, f), getattr(b, f)), f
    c = make_layer(CONFIGS["tiny"], seed=1)
    assert not np.array_equal(a.X, c.X)


def test_shapes_and_dtypes():
    s = CONFIGS["tiny"]
    L = make_layer(s)
    assert L.X.shape == (s.M, s.K) and L.X.dtype == np.uint16
    assert L.lam.shape == (s.K,) and L.lam.dtype == np.float32
    assert L.L1.shape == (s.K, s.r) and L.L2.shape == (s.r, s.N)
    assert L.R.shape == (s.N, s.K) and L.R.dtype == np.float32
    assert L.bias.shape == (s.N,)


def test_outlier_channels_and_lambda():
    s = CONFIGS["tiny"]
    L = make_layer(s, keep_w=True)
    x = np.abs(bf16_bits_to_f32(L.X)).max(axis=0).astype(np.float64)
    n_out = int(round(s.outlier_frac * s.K))
    # the outlier channels carry the largest column maxima
    big = np.argsort(x)[-n_out:]
    assert x[big].min() > 3 * np.median(x)
    w = np.abs(L.W.astype(np.float64)).max(axis=0)
    np.testing.assert_allclose(L.lam, np.sqrt(x / w).astype(np.float32), rtol=0)


def test_residual_plus_low_rank_is_smoothed_weight():
    s = CONFIGS["tiny"]
    L = make_layer(s, keep_w=True)
    W_hat = L.W.T.astype(np.float64) * L.lam.astype(np.float64)[:, None]
    lr = bf16_bits_to_f32(L.L1).astype(np.float64) @ bf16_bits_to_f32(L.L2).astype(np.float64)
    recon = L.R.T.astype(np.float64) + lr
    assert np.abs(recon - W_hat).max() <= 2.0 ** -23 * np.abs(W_hat).max() * 2
    # Eckart-Young: the residual holds exactly the energy past the top r
    # singular values (up to the bf16 rounding of the factors)
    sv = np.linalg.svd(W_hat, compute_uv=False)
    tail = np.sqrt((sv[s.r:] ** 2).sum())
    assert abs(np.linalg.norm(L.R.astype(np.float64)) - tail) <= 1e-2 * tail
