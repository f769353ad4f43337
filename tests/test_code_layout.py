"""The stored layout of the INT4 codes (include/svdq.h, svdq_w4a4 operands): the
test-side converters against a hand-derived block, their round trip, and the
property the GEMM relies on -- one AND gives the E4M3 bytes of the even codes of a
block and a funnel shift plus an AND those of the odd codes."""
import numpy as np
import pytest

from tests.helpers import dev_codes, plain_codes


def _plain(codes):
    n = np.asarray(codes, np.int16) & 15
    return (n[0::2] | (n[1::2] << 4)).astype(np.uint8)


def test_hand_derived_block():
    # nibble e = |c_e| | sign(c_(e-1 mod 16)) << 3, element 2j in the low nibble of byte j:
    # e0: 1 | s(c15=-5) -> 9; e1: 2 | s(c0=-1) -> A; e2: 0 | s(c1) -> 0; e3: 7 | s(c2=0) -> 7;
    # e4: 7 | s(c3=-7) -> F; e5-7: 0; e8: 3; e9: 3 | s(c8=3) -> 3; e10: 0 | s(c9=-3) -> 8;
    # e11-14: 0; e15: 5 | s(c14=0) -> 5
    codes = [-1, 2, 0, -7, 7, 0, 0, 0, 3, -3, 0, 0, 0, 0, 0, -5]
    want = [0xA9, 0x70, 0x0F, 0x00, 0x33, 0x08, 0x00, 0x50]
    assert dev_codes(_plain(codes)).tolist() == want
    assert plain_codes(np.array(want, np.uint8)).tolist() == _plain(codes).tolist()


def test_round_trip_all_codes():
    rng = np.random.default_rng(3)
    c = rng.integers(-7, 8, size=(37, 256))
    p = np.stack([_plain(r) for r in c])
    d = dev_codes(p)
    assert d.shape == p.shape and d.dtype == np.uint8
    assert np.array_equal(plain_codes(d), p)
    # zero codes are stored as +0 and the layout never produces code -8
    assert np.array_equal(dev_codes(np.zeros((2, 8), np.uint8)), np.zeros((2, 8), np.uint8))


def _e4m3_subnormal(b):
    """Value of E4M3 bytes whose exponent field is 0: (-1)^s m 2^-9."""
    b = np.asarray(b, np.uint32)
    assert np.all((b & 0x78) == 0)
    return np.where(b & 0x80, -1.0, 1.0) * (b & 7) * 2.0 ** -9


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_fp8_operand_form(seed):
    rng = np.random.default_rng(seed)
    c = rng.integers(-7, 8, size=32)                   # two blocks: one 16-byte read
    x = dev_codes(_plain(c)).view("<u4").astype(np.uint64)
    M = 0x87878787

    def align4(hi, lo):                                # v_alignbit_b32(hi, lo, 4)
        return int((((int(hi) << 32) | int(lo)) >> 4) & 0xFFFFFFFF)

    words = [int(x[0]) & M, align4(x[1], x[0]) & M, int(x[1]) & M, align4(x[0], x[1]) & M,
             int(x[2]) & M, align4(x[3], x[2]) & M, int(x[3]) & M, align4(x[2], x[3]) & M]
    got = _e4m3_subnormal(np.array(words, "<u4").view(np.uint8)) * 2.0 ** 9
    order = [0, 2, 4, 6, 1, 3, 5, 7, 8, 10, 12, 14, 9, 11, 13, 15]
    want = np.concatenate([c[:16][order], c[16:][order]])
    assert np.array_equal(got, want)
