"""The packed INT4 code layout (include/svdq.h): within a row the oracle and the
library store the same bytes; the library keeps rows in pairs, which the tests'
converter maps to and from the oracle's row-major bytes.  Also the property the
GEMM relies on: one AND gives the E4M3 bytes of the even codes of a block of 16
and a funnel shift plus an AND those of the odd codes, each the E4M3 subnormal
code * 2^-9.  Host-side arithmetic only (no GPU)."""
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


def _e4m3_subnormal(b):
    """Value of E4M3 bytes whose exponent field is 0: (-1)^s m 2^-9."""
    b = np.asarray(b, np.uint32)
    assert np.all((b & 0x78) == 0)
    return np.where(b & 0x80, -1.0, 1.0) * (b & 7) * 2.0 ** -9


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_fp8_operand_form(seed):
    rng = np.random.default_rng(seed)
    c = _codes(rng, 1, 64)[0]
    x = _pack(c[None, :])[0, :16].view("<u4")          # one 16-byte read: codes 0..31
    M = 0x87878787

    def align4(hi, lo):                                # funnel shift of hi:lo right by 4
        return ((int(hi) << 32 | int(lo)) >> 4) & 0xFFFFFFFF

    words = [int(x[0]) & M, align4(x[1], x[0]) & M, int(x[1]) & M, align4(x[0], x[1]) & M,
             int(x[2]) & M, align4(x[3], x[2]) & M, int(x[3]) & M, align4(x[2], x[3]) & M]
    got = _e4m3_subnormal(np.array(words, "<u4").view(np.uint8)) * 2.0 ** 9
    order = [0, 2, 4, 6, 1, 3, 5, 7, 8, 10, 12, 14, 9, 11, 13, 15]
    want = np.concatenate([c[:16][order], c[16:32][order]])
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
