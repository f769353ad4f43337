"""Property tests of the oracle's quantizers and rounding, with inputs searched by
hypothesis (derandomized, so every run checks the same examples).

Each property follows from the definition of the operation, not from the
oracle's own formula: the 4-bit group quantizer of the SVDQuant overview
(groups of 64, scale max|v| / 7, codes the nearest of the 15 integers -7..7)
must give codes whose reconstruction code * scale is within half a scale step
of the value, keep signs and order, commute with negation and with scaling by
a power of two; the packed layout must decode back to the codes; bf16 rounding
must pick the nearer of the two neighbouring bf16 values, ties to the even
significand.  Host code only.
"""
from fractions import Fraction

import numpy as np
from hypothesis import given, settings, strategies as st

import oracle

G = 64
SETTINGS = settings(max_examples=200, deadline=None, derandomize=True)

f32 = st.floats(width=32, allow_nan=False, allow_infinity=False)
normal_f32 = st.floats(min_value=2.0 ** -100, max_value=2.0 ** 100, width=32).flatmap(
    lambda a: st.sampled_from([a, -a, 0.0]))
groups = st.lists(f32, min_size=G, max_size=G)
normal_groups = st.lists(normal_f32, min_size=G, max_size=G)


def _quant(vals):
    v = np.array(vals, np.float32).reshape(1, -1)
    packed, scales = oracle.quantize_groups(v)
    return v[0], oracle.unpack(packed, v.shape[1])[0].astype(np.int64), scales[0]


def _decode(packed, K):
    """Codes from the packed layout as its definition states: code k in nibble k of the
    row (low nibble of byte k/2 for even k); in each block of 16, nibble e holds |c_e| in
    bits 0-2 and the sign of c_((e-1) mod 16) in bit 3."""
    nib = np.empty((packed.shape[0], K), np.int64)
    nib[:, 0::2] = packed & 0xF
    nib[:, 1::2] = packed >> 4
    blk = nib.reshape(packed.shape[0], K // 16, 16)
    neg = np.roll(blk >> 3, -1, axis=-1)
    return np.where(neg == 1, -(blk & 7), blk & 7).reshape(packed.shape[0], K)


@SETTINGS
@given(groups)
def test_codes_within_half_step_and_range(vals):
    v, c, s = _quant(vals)
    s = float(s[0])
    assert np.all(np.abs(c) <= 7)
    amax = float(np.abs(v).max())
    with np.errstate(over="ignore", divide="ignore"):
        inv_finite = s != 0.0 and np.isfinite(np.float32(1.0) / np.float32(s))
    if not inv_finite:
        assert not c.any()                       # zero or unusable scale: all codes 0
        return
    # the scale is max|v| / 7, rounded once to fp32
    assert s == float(np.float32(amax) / np.float32(7.0))
    if s >= 2.0 ** -126:                         # a normal scale keeps 24 bits
        err = np.abs(v.astype(np.float64) - c * s)
        assert np.all(err <= s * (0.5 + 2.0 ** -18)), (err.max() / s)
        assert np.abs(c).max() == 7              # the largest value takes the end code


@SETTINGS
@given(groups)
def test_sign_order_and_negation(vals):
    v, c, s = _quant(vals)
    assert np.all((c == 0) | (np.sign(c) == np.sign(v)))
    order = np.argsort(v, kind="stable")
    assert np.all(np.diff(c[order]) >= 0)        # monotone in the value
    vn, cn, sn = _quant([-x for x in vals])
    assert np.array_equal(cn, -c)
    assert sn.view(np.uint32)[0] == s.view(np.uint32)[0]


@SETTINGS
@given(normal_groups, st.integers(-20, 20))
def test_power_of_two_scaling(vals, e):
    v, c, s = _quant(vals)
    v2, c2, s2 = _quant([x * 2.0 ** e for x in vals])
    assert np.array_equal(c2, c)
    assert float(s2[0]) == float(s[0]) * 2.0 ** e


@SETTINGS
@given(st.lists(st.integers(0, 255), min_size=32 * 3, max_size=32 * 3))
def test_packed_layout_decodes_to_unpack(bytes_):
    packed = np.array(bytes_, np.uint8).reshape(1, -1)
    K = packed.shape[1] * 2
    assert np.array_equal(oracle.unpack(packed, K).astype(np.int64), _decode(packed, K))


@SETTINGS
@given(st.lists(st.integers(-7, 7), min_size=G, max_size=G))
def test_integer_groups_round_trip(codes):
    codes = list(codes)
    codes[0] = 7 if codes[0] >= 0 else -7       # max |v| = 7: the scale is exactly 1
    v, c, s = _quant([float(x) for x in codes])
    assert float(s[0]) == 1.0 and np.array_equal(c, codes)
    packed, _ = oracle.quantize_groups(np.array(codes, np.float32).reshape(1, -1))
    assert np.array_equal(_decode(packed, G)[0], codes)


def _bf16_value(bits):
    return np.array([bits << 16], np.uint32).view(np.float32)[0]


@SETTINGS
@given(st.floats(min_value=-3.3e38, max_value=3.3e38, allow_nan=False))
def test_bf16_rounding_is_nearest_even(x):
    b = oracle.bf16_rne(x)
    got = float(_bf16_value(b))
    # the neighbours of the result on the bf16 grid (same sign; magnitudes one step up
    # and down)
    mag = b & 0x7FFF
    cands = [got]
    for m in (mag - 1, mag + 1):
        if 0 <= m < 0x7F80:
            cands.append(float(_bf16_value((b & 0x8000) | m)))
    if mag == 0:
        cands.append(-got if got != 0 else 0.0)
        cands.append(float(_bf16_value(0x0001)) * (1 if x > 0 else -1))
    dx = Fraction(x)
    best = min(abs(Fraction(c) - dx) for c in cands)
    assert abs(Fraction(got) - dx) == best
    ties = [c for c in cands if abs(Fraction(c) - dx) == best and c != got]
    if ties:                                     # an exact tie goes to the even significand
        assert b & 1 == 0
