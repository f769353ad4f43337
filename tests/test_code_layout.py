"""The packed INT4 code layout (include/svdq.h): within a row the oracle and the
library store the same bytes; the library keeps rows in pairs, which the tests'
converter maps to and from the oracle's row-major bytes.  Also the property the
GEMM relies on: one AND per stored word (two for the third image word) unfolds a
block of 16 codes into its 96-bit FP6 (E2M3) image, each field the E2M3 subnormal
code / 8.  Host-side arithmetic only (no GPU)."""
import numpy as np
import pytest

import oracle
from tests.helpers import from_pairs, from_stage_major, to_pairs, to_stage_major


def _pack(codes):
    """Pack integer codes [rows, K] with the oracle's quantizer: each group of 64 holds
    one +-7, so its scale is exactly 1 and its codes are the values themselves."""
    v = np.asarray(codes, np.float32)
    packed, scales = oracle.quantize_groups(v)
    assert np.all(scales == 1.0)
    return packed


def _codes(rng, rows, K):
    c = rng.integers(-7, 8, size=(rows, K))
    c[:, ::64] = 7
    return c


def test_round_trip_and_zero_has_no_sign():
    rng = np.random.default_rng(3)
    c = _codes(rng, 9, 256)
    p = _pack(c)
    assert np.array_equal(oracle.unpack(p, 256), c)
    z = np.zeros((1, 64), np.float32)
    z[0, 0] = 7.0
    z[0, 1] = -0.25                                   # rounds to -0: stored as plain 0
    p = _pack(z)
    assert p[0, 0] == 0x07 and not p[0, 1:].any()


def _e2m3_subnormal(f):
    """Value of 6-bit E2M3 fields whose exponent bits (3-4) are 0: (-1)^s m / 8."""
    f = np.asarray(f, np.int64)
    assert np.all((f & 0x18) == 0)
    return np.where(f & 0x20, -1.0, 1.0) * (f & 7) / 8.0


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_fp6_operand_form(seed):
    rng = np.random.default_rng(seed)
    c = _codes(rng, 1, 64)[0]
    x = [int(w) for w in _pack(c[None, :])[0, :16].view("<u4")]   # one 16-byte read: codes 0..31
    # the always-zero bits of the image: bits 3-4 of each 6-bit field
    free = [sum(1 << o for o in range(32) if (32 * w + o) % 6 in (3, 4)) for w in (0, 1)]
    keep = [0xFFFFFFFF ^ f for f in free]
    words = []
    for u in range(2):                                  # the two blocks of the read
        w0, w1 = x[2 * u], x[2 * u + 1]
        words += [w0 & keep[0], w1 & keep[1], (w0 & free[0]) | (w1 & free[1])]
    bits = sum(w << (32 * i) for i, w in enumerate(words))
    fields = [(bits >> (6 * f)) & 63 for f in range(32)]
    got = _e2m3_subnormal(fields) * 8.0
    # field f of block u holds code 16 u + 8 (f % 2) + f // 2
    want = np.array([c[16 * (f // 16) + 8 * (f % 2) + (f % 16) // 2] for f in range(32)])
    assert np.array_equal(got, want)


def _pair_offset(i, kb, b):
    """Byte b of row i in the row-pair layout, as include/svdq.h states it."""
    c = b // 64
    w = min(64, kb - 64 * c)
    return (i // 2) * 2 * kb + 128 * c + (i % 2) * w + b % 64


@pytest.mark.parametrize("rows,K", [(1, 64), (2, 128), (5, 192), (4, 256), (7, 1088), (3, 3072)])
def test_row_pair_converter_matches_stated_offsets(rows, K):
    rng = np.random.default_rng(rows * K)
    kb = K // 2
    p = rng.integers(0, 256, size=(rows, kb), dtype=np.uint8)
    d = to_pairs(p)
    assert d.shape == ((rows + 1) // 2, K)
    flat = d.reshape(-1)
    seen = np.zeros(flat.size, bool)
    for i in range(rows):
        for b in range(kb):
            o = _pair_offset(i, kb, b)
            assert flat[o] == p[i, b]
            assert not seen[o]
            seen[o] = True
    # every byte of a full pair is used; an odd count leaves its last half unwritten
    assert seen.sum() == rows * kb
    assert np.array_equal(from_pairs(d, rows), p)


@pytest.mark.parametrize("R,G", [(1, 1), (3, 2), (5, 3), (8, 48), (7, 25)])
def test_stage_major_scale_converter_matches_stated_index(R, G):
    # include/svdq.h: the scale of (row i, group g) is element ((g/2) R + i) 2 + g%2 of a
    # [ceil(G/2), R, 2] array; an odd G's last-stage pad is zero
    rng = np.random.default_rng(R * 100 + G)
    s = rng.standard_normal((R, G)).astype(np.float32)
    d = to_stage_major(s)
    assert d.shape == ((G + 1) // 2, R, 2)
    flat = d.reshape(-1)
    for i in range(R):
        for g in range(G):
            assert flat[((g // 2) * R + i) * 2 + g % 2] == s[i, g]
    if G % 2:
        assert not flat.reshape((G + 1) // 2, R, 2)[-1, :, 1].any()
    assert np.array_equal(from_stage_major(d, R, G), s)
