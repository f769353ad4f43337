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
