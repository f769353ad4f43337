"""GPU parity of the MXFP4 (4-bit float) variant against the CPU oracle.

Bit-exact: packed E2M1 codes and E8M0 scale bytes of the weights and of the
smoothed activations.  Tolerance: the down-projection within the INT4
path's bound, the bf16 output within 1 bf16 ulp of |y_oracle| + 1e-3
rms(y_oracle) (the matrix unit sums a group's two scaled blocks in fp32 and
the K loop accumulates in fp32; the oracle is fp64).  Every call goes
through the C ABI (bit_diffusion_transformer_amd -> libsvdq.so).
"""
import numpy as np
import pytest

import bit_diffusion_transformer_amd as bdt
import oracle
from synth import CONFIGS, LayerSpec, make_layer
from tests.helpers import assert_y_close, bf16_host, from_pairs, to_dev, to_pairs, xl1_bound

pytestmark = pytest.mark.gpu


def to_block_major(s: np.ndarray) -> np.ndarray:
    """Oracle scale bytes [rows, K/32] -> the device layout [K/32, P] (padding zero)."""
    rows = s.shape[0]
    out = np.zeros((s.shape[1], bdt.mx_scale_rows(rows)), np.uint8)
    out[:, :rows] = s.T
    return out


def from_block_major(d, rows: int) -> np.ndarray:
    """Device scale bytes [K/32, P] -> [rows, K/32] (the padding dropped)."""
    d = d.cpu().numpy() if hasattr(d, "cpu") else d
    assert d.shape[1] == bdt.mx_scale_rows(rows)
    return np.ascontiguousarray(d[:, :rows].T)

# (M, K, N, r, act, bias): K % 128 == 0; one to nine stages of 128 along K
# (fewer stages than the ring holds, and wrap-around), ragged M and N tails.
SHAPES = [
    (256, 512, 512, 16, 0, True),
    (77, 384, 264, 32, 1, True),
    (1, 128, 8, 0, 0, False),
    (130, 640, 136, 48, 1, False),
    (300, 256, 256, 128, 0, True),
    (517, 1152, 392, 32, 0, True),
]


def _spec(M, K, N, r, act, bias, cid):
    return LayerSpec("mx%d" % cid, M, K, N, r, 0.01, 20.0, min(4, r) if r else 2, False,
                     act=act, bias=bias, cfg_id=200 + cid)


@pytest.fixture(scope="module", params=list(enumerate(SHAPES)),
                ids=lambda p: "M%d_K%d_N%d_r%d_act%d_bias%d" % p[1])
def case(request):
    cid, (M, K, N, r, act, bias) = request.param
    L = make_layer(_spec(M, K, N, r, act, bias, cid))
    print("mx case M=%d K=%d N=%d r=%d act=%d" % (M, K, N, r, act), flush=True)
    qa, sa, xh = oracle.mx_quantize_act(L.X, L.lam)
    qw, sw = oracle.mx_quantize(L.R)
    xl1 = oracle.down_proj(xh, L.L1) if r > 0 else None
    return dict(L=L, M=M, K=K, N=N, r=r, act=act, qa=qa, sa=sa, xh=xh, qw=qw, sw=sw, xl1=xl1)


def test_mx_pack_weights_bit_exact(case):
    qw, sw = bdt.mx_pack_weights(to_dev(case["L"].R))
    assert np.array_equal(from_pairs(qw, case["N"]), case["qw"])
    assert np.array_equal(from_block_major(sw, case["N"]), case["sw"])


def test_mx_quantize_act_down(case):
    L, r = case["L"], case["r"]
    qa, sa, xl1 = bdt.mx_quantize_act_down(to_dev(L.X), to_dev(L.lam),
                                           to_dev(L.L1) if r else None)
    assert np.array_equal(from_pairs(qa, case["M"]), case["qa"])
    assert np.array_equal(from_block_major(sa, case["M"]), case["sa"])
    if r:
        got = xl1.cpu().numpy().astype(np.float64)
        assert np.all(np.abs(got - case["xl1"]) <= xl1_bound(case["xh"], L.L1))
    else:
        assert xl1 is None


@pytest.fixture(params=[bdt.TILES_FULL, bdt.TILES_QUARTER], ids=["full_tiles", "quarter_tiles"])
def tiles(request):
    bdt.svdq_debug_set_tile_policy(request.param)
    yield request.param
    bdt.svdq_debug_set_tile_policy(bdt.TILES_AUTO)


def test_mx_gemm_stagewise(case, tiles):
    # Same inputs on both sides: the oracle's codes, scale bytes and xl1 (fp32).
    L, r, K = case["L"], case["r"], case["K"]
    xl1_32 = case["xl1"].astype(np.float32) if r else None
    Y = bdt.mx_lr_gemm(to_dev(to_pairs(case["qa"])), to_dev(to_block_major(case["sa"])),
                       to_dev(to_pairs(case["qw"])), to_dev(to_block_major(case["sw"])),
                       to_dev(xl1_32), to_dev(L.L2) if r else None, to_dev(L.bias), case["act"],
                       M=case["M"], N=case["N"])
    _, y_or = oracle.mx_gemm_rows(case["qa"], case["sa"], case["qw"], case["sw"],
                                  None if xl1_32 is None else xl1_32.astype(np.float64),
                                  L.L2, L.bias, case["act"], K)
    assert_y_close(bf16_host(Y), y_or, "mx gemm")


def test_mx_linear_end_to_end(case, tiles):
    L, r = case["L"], case["r"]
    Y = bdt.mx_linear(to_dev(L.X), to_dev(L.lam), to_dev(L.L1) if r else None,
                      to_dev(to_pairs(case["qw"])), to_dev(to_block_major(case["sw"])),
                      to_dev(L.L2) if r else None, to_dev(L.bias), case["act"], N=case["N"])
    _, y_or = oracle.mx_linear(L.X, L.lam, L.L1 if r else None, case["qw"], case["sw"],
                               L.L2 if r else None, L.bias, case["act"])
    assert_y_close(bf16_host(Y), y_or, "mx linear")


def test_mx_deterministic_and_tile_shapes_agree(case):
    # Both tile shapes run the same per-output instruction sequence.
    L, r = case["L"], case["r"]
    args = (to_dev(L.X), to_dev(L.lam), to_dev(L.L1) if r else None,
            to_dev(to_pairs(case["qw"])), to_dev(to_block_major(case["sw"])),
            to_dev(L.L2) if r else None, to_dev(L.bias), case["act"])
    out = []
    try:
        for pol in (bdt.TILES_FULL, bdt.TILES_FULL, bdt.TILES_QUARTER, bdt.TILES_AUTO):
            bdt.svdq_debug_set_tile_policy(pol)
            out.append(bf16_host(bdt.mx_linear(*args)))
    finally:
        bdt.svdq_debug_set_tile_policy(bdt.TILES_AUTO)
    for o in out[1:]:
        assert np.array_equal(out[0], o)


def _bf16_bits(v: np.ndarray) -> np.ndarray:
    """Exactly representable values -> bf16 bit patterns."""
    b = np.asarray(v, dtype=np.float32).view(np.uint32)
    assert np.all((b & 0xFFFF) == 0)
    return (b >> 16).astype(np.uint16)


def test_mx_quantizer_special_blocks():
    # lambda = 1, so the quantizer sees X itself; blocks of 32 along K = 256:
    # zero blocks (incl. -0), exact midpoints between E2M1 values (ties go to
    # the even code), values that saturate at 6 after scaling, negative
    # blocks, a block whose exponent is clamped at -127 (max 1.5 2^-126) and
    # one at a large scale.
    rng = np.random.default_rng(5)
    K = 256
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0])
    rows = []
    for e in (-3, 0, 7):
        b = np.concatenate([mids, -mids, mids * 0.5, [7.5, -7.0, 6.5, 0.0, -0.0, 1.0, 4.0, 3.0]])
        rows.append(b * 2.0 ** e)
    blk = [np.zeros(32), -np.zeros(32), rows[0], rows[1], rows[2],
           -np.abs(rows[1]), np.where(np.arange(32) % 2 == 1, 1.5, 1.0) * 2.0 ** -126,
           np.clip(np.round(rng.standard_normal(32) * 64), -255, 255) * 2.0 ** 60]
    X = np.concatenate(blk).reshape(1, K)
    X = np.concatenate([X, X[:, ::-1], -X], axis=0)          # 3 rows
    Xb = _bf16_bits(X)
    lam = np.ones(K, np.float32)
    qa_o, sa_o, _ = oracle.mx_quantize_act(Xb, lam)
    qa, sa, _ = bdt.mx_quantize_act_down(to_dev(Xb), to_dev(lam), None)
    assert np.array_equal(from_pairs(qa, 3), qa_o)
    assert np.array_equal(from_block_major(sa, 3), sa_o)
    assert sa_o[0, 0] == 0 and sa_o[0, 1] == 0        # zero blocks
    qw, sw = bdt.mx_pack_weights(to_dev(X.astype(np.float32)))
    qw_o, sw_o = oracle.mx_quantize(X.astype(np.float32))
    assert np.array_equal(from_pairs(qw, 3), qw_o)
    assert np.array_equal(from_block_major(sw, 3), sw_o)


FULL = [("qkv", CONFIGS["qkv"]), ("mlp_up", CONFIGS["mlp_up"]), ("mlp_down", CONFIGS["mlp_down"])]


@pytest.mark.parametrize("name,spec", FULL, ids=[f[0] for f in FULL])
def test_mx_full_size(name, spec):
    # The benchmark's call (svdq_mx_linear) at the full workload sizes; codes
    # and scales in full, the output on sampled token rows.
    L = make_layer(spec, seed=0)
    M, K, N, r, act = L.spec.M, L.spec.K, L.spec.N, L.spec.r, L.spec.act
    print("mx config %s M=%d K=%d N=%d r=%d act=%d" % (name, M, K, N, r, act), flush=True)
    qw_o, sw_o = oracle.mx_quantize(L.R)
    qw, sw = bdt.mx_pack_weights(to_dev(L.R))
    assert np.array_equal(from_pairs(qw, N), qw_o)
    assert np.array_equal(from_block_major(sw, N), sw_o)
    X, lam, L1, L2, bias = to_dev(L.X), to_dev(L.lam), to_dev(L.L1), to_dev(L.L2), to_dev(L.bias)
    qa_o, sa_o, xh = oracle.mx_quantize_act(L.X, L.lam)
    qa, sa, xl1 = bdt.mx_quantize_act_down(X, lam, L1)
    assert np.array_equal(from_pairs(qa, M), qa_o)
    assert np.array_equal(from_block_major(sa, M), sa_o)
    xl1_o = oracle.down_proj(xh, L.L1)
    assert np.all(np.abs(xl1.cpu().numpy().astype(np.float64) - xl1_o) <= xl1_bound(xh, L.L1))
    Y = bdt.mx_linear(X, lam, L1, qw, sw, L2, bias, act)
    rng = np.random.default_rng(11)
    rows = sorted(set([0, M - 1, M // 2] + list(rng.integers(0, M, size=21))))
    _, y_or = oracle.mx_linear(L.X, L.lam, L.L1, qw_o, sw_o, L.L2, L.bias, act, rows=rows)
    worst = assert_y_close(bf16_host(Y)[rows], y_or, "mx " + name)
    print("  worst |err|/tol = %.3f over %d rows" % (worst, len(rows)), flush=True)
