"""Pins of the CPU oracle against things other than itself.

Each test checks the oracle against a closed form, an invariant, a bound, a
brute-force enumeration or a library routine on a special case, chosen so a
plausible mistake (dropped term, wrong sign or index, transposed operand,
wrong rounding) fails at least one of them.
"""
import math
import os

import numpy as np
import pytest

import oracle
from synth import bf16_bits_to_f32, f32_to_bf16_bits

HERE = os.path.dirname(os.path.abspath(__file__))
G = 64


def _bf16(x):
    return f32_to_bf16_bits(np.asarray(x, np.float32))


# ---------------------------------------------------------------- bf16 rounding

@pytest.mark.parametrize("v,bits", [
    (1.0, 0x3F80),
    (-2.0, 0xC000),
    (0.0, 0x0000),
    (-0.0, 0x8000),
    (1 + 2 ** -8, 0x3F80),              # tie between 1 and 1+2^-7 -> even (1)
    (1 + 3 * 2 ** -8, 0x3F82),          # tie between 0x3f81 and 0x3f82 -> even
    (1 + 2 ** -8 + 2 ** -30, 0x3F81),   # just above the tie (fp32 first would lose it)
    (1 + 2 ** -8 - 2 ** -40, 0x3F80),
    (3.0, 0x4040),
    (2 ** -133, 0x0001),                # smallest bf16 subnormal
    (2 ** -134, 0x0000),                # tie between 0 and 2^-133 -> even (0)
    (3 * 2 ** -134, 0x0002),            # tie between 1 and 2 subnormal ulps -> even
    ((2 - 2 ** -7) * 2 ** 127, 0x7F7F),  # largest finite
    ((2 - 2 ** -8) * 2 ** 127, 0x7F80),  # exactly halfway to 2^128 -> even -> inf
    ((2 - 2 ** -8 - 2 ** -20) * 2 ** 127, 0x7F7F),
    (float("inf"), 0x7F80),
    (-1e300, 0xFF80),
])
def test_bf16_rne_closed_forms(v, bits):
    assert oracle.bf16_rne(v) == bits


def test_bf16_rne_matches_library_on_fp32_values():
    # For a double that is exactly an fp32 value, one RNE rounding to bf16 must
    # agree with the library's fp32 -> bf16 conversion (round to nearest even).
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(1)
    bits = rng.integers(0, 2 ** 32, size=20000, dtype=np.uint64).astype(np.uint32)
    vals = bits.view(np.float32)
    vals = vals[np.isfinite(vals)]
    ref = torch.from_numpy(vals.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([oracle.bf16_rne(float(v)) for v in vals], np.uint16)
    assert np.array_equal(got, ref)


# ---------------------------------------------------------------- GELU

def test_gelu_textbook_values():
    assert oracle.gelu(0.0) == 0.0
    # GELU(x) = x * Phi(x); Phi(1) = 0.841344746068543 (standard normal table)
    assert abs(oracle.gelu(1.0) - 0.8413447460685429) < 1e-15
    assert abs(oracle.gelu(-1.0) - (-(1 - 0.8413447460685429))) < 1e-15
    assert oracle.gelu(40.0) == 40.0
    assert abs(oracle.gelu(-40.0)) < 1e-300
    for x in (0.1, 0.7, 1.3, 2.9, 5.5):
        # odd part of GELU is x/2: GELU(x) - GELU(-x) = x
        assert abs((oracle.gelu(x) - oracle.gelu(-x)) - x) <= 4e-16 * x


# ---------------------------------------------------------------- quantizer fixtures

def _load_fixtures():
    out = []
    with open(os.path.join(HERE, "golden", "quant_fixtures.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            name, lam, vals, scale, packed = [s.strip() for s in line.split("|")]
            v = np.zeros(G)
            first = [float(t) for t in vals.split()]
            v[:len(first)] = first
            out.append((name, float(lam), v, int(scale, 16),
                        bytes(int(b, 16) for b in packed.split())))
    return out


@pytest.mark.parametrize("fx", _load_fixtures(), ids=lambda f: f[0])
def test_quant_fixtures(fx):
    name, lam, v, scale_bits, packed = fx
    X = _bf16(v)[None, :]
    assert np.array_equal(bf16_bits_to_f32(X)[0], v.astype(np.float32)), "fixture not bf16-exact"
    qa, sa, _ = oracle.quantize_act(X, np.full(G, lam, np.float32))
    assert sa.view(np.uint32)[0, 0] == scale_bits
    assert bytes(qa[0]) == packed


# ---------------------------------------------------------------- lossless grid

def _grid_matrix(rng, rows, K, emin, emax):
    """q * 2^e per (row, group) with exactly one |q| = 7 per group."""
    q = rng.integers(-7, 8, size=(rows, K)).astype(np.int64)
    for g in range(K // G):
        pos = rng.integers(0, G, size=rows)
        q[np.arange(rows), g * G + pos] = rng.choice([-7, 7], size=rows)
    e = rng.integers(emin, emax + 1, size=(rows, K // G))
    vals = q * np.exp2(np.repeat(e, G, axis=1))
    return q, e, vals


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_lossless_grid_exact(seed):
    # On-grid inputs with power-of-two scales and lambda are represented
    # exactly, so codes, scales and the 4-bit product are exact.
    rng = np.random.default_rng(seed)
    M, N, K = 7, 9, 256
    qa_true, ea, xh = _grid_matrix(rng, M, K, -12, 4)
    lam = np.exp2(rng.integers(-3, 4, size=K)).astype(np.float32)
    X = _bf16(xh * lam)                       # exact: 3-bit significands
    assert np.array_equal(bf16_bits_to_f32(X).astype(np.float64), xh * lam)
    qw_true, ew, R = _grid_matrix(rng, N, K, -10, 2)

    qa, sa, xh_or = oracle.quantize_act(X, lam)
    assert np.array_equal(xh_or.astype(np.float64), xh)
    assert np.array_equal(oracle.unpack(qa, K), qa_true)
    assert np.array_equal(sa.astype(np.float64), np.exp2(ea))
    qw, sw = oracle.pack_weights(R.astype(np.float32))
    assert np.array_equal(oracle.unpack(qw, K), qw_true)
    assert np.array_equal(sw.astype(np.float64), np.exp2(ew))

    acc, y = oracle.gemm_rows(qa, sa, qw, sw, None, None, None, 0, K)
    ref = xh @ R.T                             # exact in fp64 (small integers x 2^e)
    assert np.array_equal(acc, ref)
    assert all(y[i, j] == oracle.bf16_rne(acc[i, j]) for i in range(M) for j in range(N))


# ---------------------------------------------------------------- low-rank branch

def _lr_inputs(rng, M, K, N, r, pow2_lam):
    X = _bf16(rng.standard_normal((M, K)) * 3)
    if pow2_lam:
        lam = np.exp2(rng.integers(-3, 4, size=K)).astype(np.float32)
    else:
        lam = rng.uniform(0.3, 3.0, size=K).astype(np.float32)
    L1 = _bf16(rng.standard_normal((K, r)))
    L2 = _bf16(rng.standard_normal((r, N)) * 0.1)
    bias = _bf16(rng.standard_normal(N) * 0.02)
    return X, lam, L1, L2, bias


def _f(b):
    return bf16_bits_to_f32(b).astype(np.float64)


@pytest.mark.parametrize("act", [0, 1])
def test_exact_low_rank_weight(act):
    # W exactly rank r (R = 0): the layer reduces to X diag(lam)^-1 L1 L2 + bias,
    # exact in fp64 for power-of-two lambda.
    from scipy.special import erf
    rng = np.random.default_rng(3)
    M, K, N, r = 5, 128, 24, 16
    X, lam, L1, L2, bias = _lr_inputs(rng, M, K, N, r, True)
    qw, sw = oracle.pack_weights(np.zeros((N, K), np.float32))
    assert not qw.any() and not sw.any()
    acc, y = oracle.linear(X, lam, L1, qw, sw, L2, bias, act)
    pre = (_f(X) / lam.astype(np.float64)) @ _f(L1) @ _f(L2) + _f(bias)
    ref = pre if act == 0 else 0.5 * pre * (1 + erf(pre / np.sqrt(2)))
    np.testing.assert_allclose(acc, ref, rtol=1e-12, atol=1e-12)


def test_smoothing_direction_and_invariance():
    # General lambda: xh = X / lam up to one fp32 rounding of 1/lam and of the
    # product, so the low-rank output is X diag(lam)^-1 L1 L2 to ~2^-23.
    rng = np.random.default_rng(4)
    M, K, N, r = 6, 192, 20, 32
    X, lam, L1, L2, _ = _lr_inputs(rng, M, K, N, r, False)
    qw, sw = oracle.pack_weights(np.zeros((N, K), np.float32))
    acc, _ = oracle.linear(X, lam, L1, qw, sw, L2, None, 0)
    t = (_f(X) / lam.astype(np.float64))
    ref = t @ _f(L1) @ _f(L2)
    bound = (np.abs(t) @ np.abs(_f(L1)) @ np.abs(_f(L2))) * 2.5 * 2.0 ** -24
    assert np.all(np.abs(acc - ref) <= bound + 1e-300)
    # and the unquantized identity (X diag(lam)^-1)(diag(lam) W) = X W
    W = rng.standard_normal((N, K))
    xh = oracle.smooth(X, lam).astype(np.float64)
    lhs = xh @ (W.T * lam.astype(np.float64)[:, None])
    rhs = _f(X) @ W.T
    scale = np.abs(_f(X)) @ np.abs(W.T)
    assert np.all(np.abs(lhs - rhs) <= scale * 2.0 ** -22)


def test_down_proj_against_fp64_matmul():
    rng = np.random.default_rng(5)
    M, K, r = 9, 320, 48
    X, lam, L1, _, _ = _lr_inputs(rng, M, K, 8, r, False)
    xh = oracle.smooth(X, lam)
    got = oracle.down_proj(xh, L1)
    ref = xh.astype(np.float64) @ _f(L1)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-10)


# ---------------------------------------------------------------- codes: nearest, ties to even

def _nearest_even(y):
    cands = np.arange(-7, 8, dtype=np.float64)
    d = np.abs(y[:, None] - cands[None, :])
    best = d.min(axis=1, keepdims=True)
    is_best = d == best
    # among tied candidates prefer the even one
    even = (cands % 2 == 0)[None, :]
    pick = np.where(is_best & even, 1, 0) + np.where(is_best, 1, 0)
    return cands[np.argmax(pick, axis=1)]


@pytest.mark.parametrize("seed", range(4))
def test_codes_are_nearest_grid_point_ties_even(seed):
    rng = np.random.default_rng(seed)
    rows, K = 16, 256
    v = rng.standard_normal((rows, K)).astype(np.float32) * rng.uniform(0.01, 50, (rows, 1)).astype(np.float32)
    # plant exact ties: values at k+0.5 times the group scale of 1 (amax 7)
    v[0, :G] = 0
    v[0, 0] = 7
    v[0, 1:15] = np.array([-6.5, -5.5, -4.5, -3.5, -2.5, -1.5, -0.5, 0.5, 1.5, 2.5, 3.5, 4.5, 5.5, 6.5])
    packed, scales = oracle.quantize_groups(v)
    codes = oracle.unpack(packed, K).astype(np.float64)
    for r_ in range(rows):
        for g in range(K // G):
            s = scales[r_, g]
            grp = v[r_, g * G:(g + 1) * G]
            assert s == np.float32(np.abs(grp).max()) / np.float32(7)
            inv = np.float32(1) / s
            y = (grp * inv).astype(np.float64)    # the fp32 product the code rounds
            assert np.array_equal(codes[r_, g * G:(g + 1) * G], _nearest_even(y))
    assert list(codes[0, 1:15]) == [-6, -6, -4, -4, -2, -2, 0, 0, 2, 2, 4, 4, 6, 6]


def test_zero_and_tiny_groups():
    v = np.zeros((3, 128), np.float32)
    v[1, 64] = 1e-45          # smallest subnormal: amax/7 rounds to 0 -> codes 0
    v[2, :64] = 3e-39         # subnormal scale whose reciprocal overflows -> codes 0
    packed, scales = oracle.quantize_groups(v)
    assert not packed.any()
    assert scales[1, 1] == 0.0
    with np.errstate(over="ignore"):                  # the overflow is the point
        assert scales[2, 0] > 0 and not np.isfinite(np.float32(1) / scales[2, 0])


# ---------------------------------------------------------------- group sums

def _decode(packed, K):
    """Codes from the packed layout, written from its definition: in each 8-byte block
    of 16 codes (two little-endian words W0, W1), the 96-bit image of 6-bit fields is
    I0 = W0 without its free bits, I1 = W1 without its free bits, I2 = the free bits of
    both (a free bit is bit 3 or 4 of a field: image position p with p mod 6 in {3, 4});
    code 8h + i is field 2i + h: |c| in bits 0-2, the sign in bit 5."""
    free = [sum(1 << o for o in range(32) if (32 * w + o) % 6 in (3, 4)) for w in (0, 1)]
    words = np.ascontiguousarray(packed, dtype=np.uint8).view("<u4").astype(object)
    W0, W1 = words[:, 0::2], words[:, 1::2]                  # [rows, K / 16], Python ints
    img = ((W0 & (0xFFFFFFFF ^ free[0])) | ((W1 & (0xFFFFFFFF ^ free[1])) << 32)
           | (((W0 & free[0]) | (W1 & free[1])) << 64))
    out = np.empty((packed.shape[0], K), np.int64)
    for e in range(16):
        f = 2 * (e % 8) + e // 8
        v = (img >> (6 * f)) & 63
        mag = (v & 7).astype(np.int64)
        out[:, e::16] = np.where((v & 32).astype(np.int64) != 0, -mag, mag)
    return out


def test_group_sums_closed_form_extreme():
    K = 128
    # every code 7: each 16-code block is the image of sixteen fields 000111, folded
    # (the 8 bytes df f7 7d df 75 5d d7 75); every code -7: all bits set (each field 100111,
    # every free bit filled)
    qa = np.tile(np.array([0xdf, 0xf7, 0x7d, 0xdf, 0x75, 0x5d, 0xd7, 0x75], np.uint8), (2, K // 16))
    qw = np.full((3, K // 2), 0xFF, np.uint8)
    S = oracle.group_sums(qa, qw, K, 0, 0, 2, 3)
    assert S.shape == (2, 3, 2) and np.all(S == -3136)


def test_group_sums_brute_force():
    rng = np.random.default_rng(6)
    M, N, K = 11, 13, 320
    qa = rng.integers(0, 256, size=(M, K // 2), dtype=np.uint8)
    qw = rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    a, w = _decode(qa, K), _decode(qw, K)
    assert np.array_equal(oracle.unpack(qa, K).astype(np.int64), a)
    m0, n0, tm, tn = 2, 3, 7, 8
    S = oracle.group_sums(qa, qw, K, m0, n0, tm, tn)
    ref = np.einsum("mgj,ngj->mng", a[m0:m0 + tm].reshape(tm, -1, G),
                    w[n0:n0 + tn].reshape(tn, -1, G))
    assert np.array_equal(S, ref)


# ---------------------------------------------------------------- quantization error bound

@pytest.mark.parametrize("seed", range(3))
def test_quantized_product_within_analytic_bound(seed):
    # x = sa (qa + da), w = sw (qw + dw), |da|,|dw| <= 1/2 (+ fp32 slack), so
    # |x.w - sa sw qa qw| <= |x| sw/2 + |w| sa/2 + sa sw/4 per element.
    rng = np.random.default_rng(seed)
    M, N, K = 4, 6, 256
    X = _bf16(rng.standard_normal((M, K)) * rng.uniform(0.1, 10, (M, 1)))
    lam = rng.uniform(0.5, 2.0, K).astype(np.float32)
    R = (rng.standard_normal((N, K)) * 0.05).astype(np.float32)
    qa, sa, xh = oracle.quantize_act(X, lam)
    qw, sw = oracle.pack_weights(R)
    acc, _ = oracle.gemm_rows(qa, sa, qw, sw, None, None, None, 0, K)
    x, w = xh.astype(np.float64), R.astype(np.float64)
    exact = x @ w.T
    sa_k = np.repeat(sa.astype(np.float64), G, axis=1)
    sw_k = np.repeat(sw.astype(np.float64), G, axis=1)
    bound = (np.abs(x) @ (sw_k.T / 2) + (sa_k / 2) @ np.abs(w).T + sa_k @ sw_k.T / 4)
    err = np.abs(acc - exact)
    assert np.all(err <= bound * (1 + 1e-5))
    assert err.max() > 0   # the bound is exercised, not trivially met
