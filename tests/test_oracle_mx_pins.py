"""Pins of the MXFP4 (4-bit float variant) part of the CPU oracle against things other than
itself: the specification's value table and scale rule (fixtures), brute-force nearest-even
rounding, closed forms of the scale exponent, a lossless grid, the rounding error bound, and the
layer product against an independent fp64 matmul."""
import os

import numpy as np
import pytest

import oracle
from synth import bf16_bits_to_f32, f32_to_bf16_bits

HERE = os.path.dirname(os.path.abspath(__file__))
MAG = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def _lines(tag):
    for line in open(os.path.join(HERE, "golden", "mx_fixtures.txt")):
        if line.startswith(tag + " "):
            yield [f.strip() for f in line[2:].split("|")]


def test_e2m1_values_and_codes():
    for code, val in _lines("E"):
        assert oracle.mx_e2m1_value(int(code)) == float(val)
        assert oracle.mx_e2m1_code(float(val)) == int(code)
    assert oracle.mx_e2m1_value(8) == 0.0            # -0 decodes to zero
    assert oracle.mx_e2m1_code(-0.0) == 0             # and zero is always stored as +0


def test_scale_bytes():
    for amax, byte in _lines("S"):
        assert oracle.mx_scale_byte(float(amax)) == int(byte)
    for k in range(-120, 120, 7):                     # closed form on either side of 2^k
        assert oracle.mx_scale_byte(2.0 ** k) == k - 2 + 127
        assert oracle.mx_scale_byte(2.0 ** k * 1.999) == k - 2 + 127
        assert oracle.mx_scale_byte(2.0 ** k * 0.999) == k - 3 + 127
    assert oracle.mx_scale_byte(2.0 ** -140) == 0     # clamped at 2^-127
    assert oracle.mx_scale_byte(2.0 ** 135) == 254


def test_block_fixtures():
    for vals, codes, byte in _lines("B"):
        v = np.zeros((1, 32), np.float32)
        vv = [float(t) for t in vals.split()]
        v[0, :len(vv)] = vv
        packed, scales = oracle.mx_quantize(v)
        assert scales[0, 0] == int(byte)
        got = [(packed[0, j // 2] >> (4 * (j % 2))) & 15 for j in range(len(vv))]
        assert got == [int(t) for t in codes.split()]


def test_rounding_is_brute_force_nearest_even():
    ys = np.concatenate([np.linspace(-8, 8, 4001), [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]])
    for y in ys:
        c = oracle.mx_e2m1_code(float(y))
        a = min(abs(y), 6.0)
        dists = [abs(a - m) for m in MAG]
        best = min(dists)
        ties = [i for i, d in enumerate(dists) if d == best]
        want = ties[0] if len(ties) == 1 else [i for i in ties if i % 2 == 0][0]
        assert c & 7 == want, (y, c, want)
        assert (c & 8) == (8 if (y < 0 and want != 0) else 0)


def _grid(rng, rows, K, emin=-6, emax=6):
    """Values exactly on the MXFP4 grid: E2M1 values times 2^e per block, each block holding a
    4 or a 6 so that the scale rule gives back 2^e."""
    codes = rng.integers(0, 16, size=(rows, K))
    codes[:, ::32] = rng.choice([6, 7, 14, 15], size=(rows, K // 32))
    e = rng.integers(emin, emax, size=(rows, K // 32))
    vals = np.array([oracle.mx_e2m1_value(int(c)) for c in codes.ravel()]).reshape(rows, K)
    return (vals * np.repeat(2.0 ** e, 32, axis=1)).astype(np.float32), e


def test_lossless_grid_round_trip():
    rng = np.random.default_rng(41)
    v, e = _grid(rng, 12, 256)
    packed, scales = oracle.mx_quantize(v)
    assert np.array_equal(scales.astype(np.int64), e + 127)
    assert np.array_equal(oracle.mx_dequant(packed, scales, 256), v.astype(np.float64))


def test_rounding_error_bound():
    rng = np.random.default_rng(42)
    v = (rng.standard_normal((16, 512)) * np.exp(rng.uniform(-8, 8, (16, 1)))).astype(np.float32)
    packed, scales = oracle.mx_quantize(v)
    deq = oracle.mx_dequant(packed, scales, 512)
    X = np.repeat(2.0 ** (scales.astype(np.float64) - 127), 32, axis=1)
    y = np.abs(v.astype(np.float64)) / X
    # half the gap of E2M1 at |y| (0.25 below 2, 0.5 below 4, 1 below 6), 2 above 6 (saturation)
    half = np.where(y <= 2, 0.25, np.where(y <= 4, 0.5, np.where(y <= 6, 1.0, 2.0)))
    assert np.all(np.abs(deq - v) <= half * X * (1 + 1e-12))
    assert np.all(np.abs(deq) <= 6 * X)


def test_gemm_equals_fp64_matmul_on_grid():
    rng = np.random.default_rng(43)
    M, N, K, r = 7, 24, 192, 16
    a, _ = _grid(rng, M, K)
    w, _ = _grid(rng, N, K, -8, -2)
    qa, sa = oracle.mx_quantize(a)
    qw, sw = oracle.mx_quantize(w)
    xl1 = rng.standard_normal((M, r))
    L2 = f32_to_bf16_bits((0.1 * rng.standard_normal((r, N))).astype(np.float32))
    bias = f32_to_bf16_bits((0.02 * rng.standard_normal(N)).astype(np.float32))
    acc, y = oracle.mx_gemm_rows(qa, sa, qw, sw, xl1, L2, bias, 0, K)
    ref = a.astype(np.float64) @ w.astype(np.float64).T + xl1 @ bf16_bits_to_f32(L2).astype(np.float64)
    ref += bf16_bits_to_f32(bias).astype(np.float64)[None, :]
    assert np.allclose(acc, ref, rtol=1e-12, atol=1e-9)
    acc_g, _ = oracle.mx_gemm_rows(qa, sa, qw, sw, xl1, L2, bias, 1, K)
    assert np.allclose(acc_g, np.vectorize(oracle.gelu)(acc), rtol=1e-14, atol=1e-14)
    acc_s, y_s = oracle.mx_gemm_rows(qa, sa, qw, sw, xl1, L2, bias, 0, K, rows=[6, 2])
    assert np.array_equal(acc_s, acc[[6, 2]]) and np.array_equal(y_s, y[[6, 2]])
