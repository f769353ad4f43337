"""Pins of the W4A16 (awq_w4a16) part of the CPU oracle against things other than itself.

Hand-derived fixtures, an exactly representable (lossless) grid, the
round-to-nearest error bound, brute-force nearest codes, exact zero, and the
layer product against an independent fp64 matmul.
"""
import os

import numpy as np
import pytest

import oracle
from synth import bf16_bits_to_f32, f32_to_bf16_bits

HERE = os.path.dirname(os.path.abspath(__file__))
G = 64


def _fixtures():
    out = []
    for line in open(os.path.join(HERE, "golden", "awq_fixtures.txt")):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        name, vals, sbits, z, packed = [f.strip() for f in line.split("|")]
        v = np.zeros(G, np.float32)
        vv = [float(t) for t in vals.split()]
        v[:len(vv)] = vv
        out.append((name, v, int(sbits, 16), int(z), bytes.fromhex(packed)))
    return out


@pytest.mark.parametrize("name,v,sbits,z,packed", _fixtures(), ids=lambda x: x if isinstance(x, str) else None)
def test_hand_fixtures(name, v, sbits, z, packed):
    q, s, zz = oracle.awq_quantize(v[None, :])
    assert int(s.view(np.uint32)[0, 0]) == sbits
    assert int(zz[0, 0]) == z
    assert q[0].tobytes() == packed


def _grid_weights(rng, N, K, e):
    """Weights exactly on an asymmetric grid: (q - z) * 2^e with codes 0 and 15 in every group."""
    Gk = K // G
    q = rng.integers(0, 16, size=(N, K))
    q[:, ::G] = 0
    q[:, 1::G] = 15
    z = rng.integers(0, 16, size=(N, Gk))
    s = 2.0 ** e
    W = (q - np.repeat(z, G, axis=1)) * s
    return W.astype(np.float32), q, z, s


def test_lossless_grid_round_trip():
    rng = np.random.default_rng(11)
    N, K = 24, 256
    W, q, z, s = _grid_weights(rng, N, K, -6)
    packed, scales, zeros = oracle.awq_quantize(W)
    assert np.all(scales == np.float32(s))
    assert np.array_equal(zeros.astype(np.int64), z)
    lo = packed & 0xF
    hi = packed >> 4
    codes = np.empty((N, K), np.int64)
    codes[:, 0::2] = lo
    codes[:, 1::2] = hi
    assert np.array_equal(codes, q)
    assert np.array_equal(oracle.awq_dequant(packed, scales, zeros, K), W.astype(np.float64))


def test_linear_equals_fp64_matmul_on_grid():
    rng = np.random.default_rng(12)
    M, N, K = 5, 40, 320
    W, _, _, _ = _grid_weights(rng, N, K, -5)
    packed, scales, zeros = oracle.awq_quantize(W)
    X = f32_to_bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
    bias = f32_to_bf16_bits((0.02 * rng.standard_normal(N)).astype(np.float32))
    acc, y = oracle.awq_linear(X, packed, scales, zeros, bias)
    ref = bf16_bits_to_f32(X).astype(np.float64) @ W.astype(np.float64).T
    ref += bf16_bits_to_f32(bias).astype(np.float64)[None, :]
    assert np.allclose(acc, ref, rtol=1e-12, atol=1e-12)
    assert np.array_equal(y, np.vectorize(oracle.bf16_rne)(acc).astype(np.uint16))


def test_round_to_nearest_bound_and_exact_zero():
    rng = np.random.default_rng(13)
    N, K = 16, 512
    W = (rng.standard_normal((N, K)) * np.exp(rng.uniform(-6, 3, size=(N, 1)))).astype(np.float32)
    W[:, 5] = 0.0
    packed, scales, zeros = oracle.awq_quantize(W)
    Wq = oracle.awq_dequant(packed, scales, zeros, K)
    s = np.repeat(scales.astype(np.float64), G, axis=1)
    err = np.abs(Wq - W.astype(np.float64))
    assert np.all(err <= 0.5 * s * (1 + 1e-5) + 1e-30)
    assert np.all(Wq[:, 5] == 0.0)                # zero is always on the grid


def test_codes_are_brute_force_nearest():
    rng = np.random.default_rng(14)
    N, K = 6, 128
    W = rng.uniform(-3, 5, size=(N, K)).astype(np.float32)
    packed, scales, zeros = oracle.awq_quantize(W)
    Wq = oracle.awq_dequant(packed, scales, zeros, K)
    for n in range(N):
        for g in range(K // G):
            s, z = float(scales[n, g]), int(zeros[n, g])
            grid = (np.arange(16) - z) * s
            for j in range(G):
                k = g * G + j
                best = np.min(np.abs(grid - float(W[n, k])))
                assert abs(Wq[n, k] - float(W[n, k])) <= best + 1e-6 * s


def test_rows_subset_matches_full():
    rng = np.random.default_rng(15)
    M, N, K = 9, 24, 192
    W = rng.standard_normal((N, K)).astype(np.float32)
    packed, scales, zeros = oracle.awq_quantize(W)
    X = f32_to_bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
    acc, y = oracle.awq_linear(X, packed, scales, zeros, None)
    rows = [0, 4, 8]
    acc2, y2 = oracle.awq_linear(X, packed, scales, zeros, None, rows=rows)
    assert np.array_equal(acc2, acc[rows]) and np.array_equal(y2, y[rows])
