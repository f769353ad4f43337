"""Edge cases on the GPU: empty inputs, zero and subnormal groups, canaries
around every output, streams, and errors surfacing through the binding."""
import ctypes

import numpy as np
import pytest
import torch

import bit_diffusion_transformer_amd as bdt
import oracle
from bit_diffusion_transformer_amd import _binding
from synth import LayerSpec, f32_to_bf16_bits, make_layer
from tests.helpers import assert_y_close, bf16_host, from_pairs, from_stage_major, pdev, sdev, to_dev

pytestmark = pytest.mark.gpu


def _layer(M=96, K=256, N=136, r=32, act=0, cid=0):
    return make_layer(LayerSpec("e", M, K, N, r, 0.01, 20.0, 4, False, act=act, cfg_id=200 + cid))


def test_empty_batch():
    L = _layer()
    X = to_dev(L.X)[:0]
    qa, sa, xl1 = bdt.quantize_act_down(X, to_dev(L.lam), to_dev(L.L1))
    assert qa.shape == (0, 256) and sa.shape == (2, 0, 2) and xl1.shape == (0, 32)
    qw, sw = bdt.pack_weights(to_dev(L.R))
    Y = bdt.linear(X, to_dev(L.lam), to_dev(L.L1), qw, sw, to_dev(L.L2), to_dev(L.bias))
    assert Y.shape == (0, 136)


def test_zero_and_subnormal_groups_bit_exact():
    rng = np.random.default_rng(11)
    M, K = 48, 512
    x = rng.standard_normal((M, K)).astype(np.float32)
    x[3] = 0.0                                   # an all-zero token
    x[5, 64:128] = 0.0                           # one zero group
    x[7] *= np.float32(1e-37)                    # subnormal after smoothing below
    x[9, :64] = np.float32(2.0 ** -130)          # subnormal inputs themselves
    X = f32_to_bf16_bits(x)
    lam = rng.uniform(0.5, 2.0, K).astype(np.float32)
    lam[200:260] = np.float32(3e38)              # pushes those x / lam into subnormals
    qa_o, sa_o, _ = oracle.quantize_act(X, lam)
    qa, sa, _ = bdt.quantize_act_down(to_dev(X), to_dev(lam), None)
    assert np.array_equal(from_pairs(qa, M), qa_o)
    assert np.array_equal(from_stage_major(sa, sa_o.shape[0], sa_o.shape[1]).view(np.uint32),
                          sa_o.view(np.uint32))
    assert (sa_o == 0).any() and ((sa_o > 0) & (sa_o < 2.0 ** -126)).any()
    R = (rng.standard_normal((64, K)) * 0.05).astype(np.float32)
    R[2] = 0.0
    R[4, :64] = np.float32(1e-40)
    qw_o, sw_o = oracle.pack_weights(R)
    qw, sw = bdt.pack_weights(to_dev(R))
    assert np.array_equal(from_pairs(qw, 64), qw_o)
    assert np.array_equal(from_stage_major(sw, sw_o.shape[0], sw_o.shape[1]).view(np.uint32),
                          sw_o.view(np.uint32))


def test_all_extreme_codes():
    # every group saturated: codes +-7 everywhere, |S| = 3136 per group
    M, K, N = 32, 256, 64
    X = f32_to_bf16_bits(np.where(np.arange(K) % 2 == 0, 3.0, -3.0)[None, :].repeat(M, 0))
    lam = np.ones(K, np.float32)
    R = np.where(np.arange(K) % 2 == 0, -0.5, 0.5)[None, :].repeat(N, 0).astype(np.float32)
    qa_o, sa_o, _ = oracle.quantize_act(X, lam)
    qw_o, sw_o = oracle.pack_weights(R)
    S = bdt.group_sums(pdev(qa_o), sdev(sa_o), pdev(qw_o), sdev(sw_o), M, N, 0, 0, M, N).cpu().numpy()
    assert np.all(S == -3136)
    Y = bdt.w4a4_lr_gemm(pdev(qa_o), sdev(sa_o), pdev(qw_o), sdev(sw_o), None, None, None)
    _, y_or = oracle.gemm_rows(qa_o, sa_o, qw_o, sw_o, None, None, None, 0, K)
    assert_y_close(bf16_host(Y), y_or)


def _padded(n_elem, dtype, fill):
    """A tensor of n_elem inside a buffer with 64 sentinel elements on each side."""
    buf = torch.full((n_elem + 128,), fill, dtype=dtype, device="cuda:0")
    return buf, buf[64:64 + n_elem]


def test_canaries_untouched():
    L = _layer(M=77, K=192, N=264, r=48, act=1, cid=1)
    M, K, N, r = 77, 192, 264, 48
    G = K // 64
    qa_b, qa = _padded(bdt.pair_rows(M) * K, torch.uint8, 0xA5)   # row pairs
    sa_b, sa = _padded((G + 1) // 2 * M * 2, torch.float32, -123.0)   # stage-major pairs
    x_b, x1 = _padded(M * r, torch.float32, -321.0)
    y_b, y = _padded(M * N, torch.int16, 0x5A5A)
    ws_bytes = bdt.svdq_quantize_act_down_workspace_bytes(M, K, r)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device="cuda:0")
    bdt.svdq_quantize_act_down(bdt._bits(to_dev(L.X)), to_dev(L.lam), bdt._bits(to_dev(L.L1)),
                               M, K, r, qa, sa, x1, ws, ws_bytes)
    qw, sw = bdt.pack_weights(to_dev(L.R))
    bdt.svdq_w4a4_lr_gemm(qa, sa, qw, sw, x1, bdt._bits(to_dev(L.L2)), bdt._bits(to_dev(L.bias)),
                          1, M, N, K, r, y)
    torch.cuda.synchronize()
    for b, fill in ((qa_b, 0xA5), (sa_b, -123.0), (x_b, -321.0), (y_b, 0x5A5A)):
        h = b.cpu()
        assert torch.all(h[:64] == fill) and torch.all(h[-64:] == fill)
    qa_o, sa_o, _ = oracle.quantize_act(L.X, L.lam)
    qa_h = qa.cpu().numpy().reshape(bdt.pair_rows(M), K)
    assert np.array_equal(from_pairs(qa_h, M), qa_o)
    # M odd: the second half of the last pair is left unwritten (K / 2 = 96 bytes per
    # row: a 64-byte chunk and a 32-byte last chunk)
    assert np.all(qa_h[-1, 64:128] == 0xA5) and np.all(qa_h[-1, 160:192] == 0xA5)


def test_side_stream_matches_default_stream():
    L = _layer(cid=2)
    args = (to_dev(L.X), to_dev(L.lam), to_dev(L.L1))
    qw, sw = bdt.pack_weights(to_dev(L.R))
    y0 = bf16_host(bdt.linear(*args, qw, sw, to_dev(L.L2), to_dev(L.bias)))
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        y1 = bdt.linear(*args, qw, sw, to_dev(L.L2), to_dev(L.bias))
    s.synchronize()
    assert np.array_equal(y0, bf16_host(y1))


def test_errors_surface_through_binding():
    L = _layer(cid=3)
    with pytest.raises(_binding.SVDQError) as e:
        # K = 200 is not a multiple of 64
        bdt.svdq_quantize_act_down(None, None, None, 4, 200, 0, None, None, None, None, 0)
    assert e.value.status == 2
    assert "multiple of 64" in str(e.value)
    # device check passes on gfx950: a valid call returns OK
    qw, sw = bdt.pack_weights(to_dev(L.R))
    torch.cuda.synchronize()
    assert bdt.svdq_last_error() == ""


def test_repack_minus_eight_is_stored_as_minus_seven():
    # -8 is outside the symmetric code range; the repack stores it as -7
    rng = np.random.default_rng(12)
    N, K = 6, 256
    c = rng.integers(-7, 8, size=(N, K))
    c[:, ::64] = 7                                   # scale 1 per group in the reference packing
    m8 = rng.random((N, K)) < 0.1
    m8[:, ::64] = False
    raw = np.where(m8, -8, c)
    tc = ((raw[:, 0::2] & 0xF) | ((raw[:, 1::2] & 0xF) << 4)).astype(np.uint8)
    want, scales = oracle.quantize_groups(np.where(m8, -7, c).astype(np.float32))
    assert np.all(scales == 1.0)
    qw, sw = bdt.repack_weights(to_dev(tc), to_dev(scales))
    assert np.array_equal(from_pairs(qw, N), want)
    assert np.array_equal(from_stage_major(sw, N, K // 64), scales)


@pytest.mark.parametrize("eta", [0.3, 0.1, 0.03])
def test_rescale_precision_under_cancelling_groups(eta):
    # Per-group terms sa sw S of alternating sign and nearly equal size, so that the
    # output is a small remainder of large terms: with |S_g| ~ 3000 for every group,
    # sa = a (1 + e), sw = b (1 + d), e, d ~ U(-eta, eta), sum_g |term| / rms(Y) is about
    # 17 / eta (57x, 170x, 570x).  The GPU forms sw sa as the fp32 product (rounded
    # once, 2^-24 relative) on the matrix unit and adds each term with one fp32 fma
    # (a rounding of at most 2^-24 of the running sum, itself at most sum_g |term|):
    # over G = 192 groups at most 2^-16 sum_g |term| in all, plus the final bf16
    # rounding.  These cases must stay inside the tolerance and inside that bound.
    rng = np.random.default_rng(int(eta * 1000))
    M, N, K = 64, 64, 12288
    G = K // 64
    a = rng.choice([-7, -6, 6, 7], size=(1, K))                # one code row for every token
    a[:, ::64] = 7
    qa_codes = np.repeat(a, M, axis=0)
    sign = np.where(np.arange(G) % 2 == 0, 1, -1)
    w = np.repeat(a * np.repeat(sign, 64)[None, :], N, axis=0)   # S_g = (-1)^g sum a_g^2
    qa_o, s1 = oracle.quantize_groups(qa_codes.astype(np.float32))
    qw_o, s2 = oracle.quantize_groups(w.astype(np.float32))
    assert np.all(s1 == 1.0) and np.all(s2 == 1.0)
    sa = (rng.uniform(0.5, 2.0, (M, 1)) * (1 + rng.uniform(-eta, eta, (M, G)))).astype(np.float32)
    sw = (rng.uniform(0.5, 2.0, (N, 1)) * (1 + rng.uniform(-eta, eta, (N, G)))).astype(np.float32)
    Y = bdt.w4a4_lr_gemm(pdev(qa_o), sdev(sa), pdev(qw_o), sdev(sw), None, None, None)
    acc, y_or = oracle.gemm_rows(qa_o, sa, qw_o, sw, None, None, None, 0, K)
    S = (qa_codes.reshape(M, G, 64)[0] ** 2).sum(axis=1) * sign          # [G]
    terms = np.abs(sa.astype(np.float64))[:, None, :] * np.abs(sw.astype(np.float64))[None, :, :] \
        * np.abs(S)[None, None, :]
    yg = bf16_host(Y)
    worst = assert_y_close(yg, y_or, "cancelling groups")
    yv = (yg.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    bound = 2.0 ** -16 * terms.sum(axis=2) + np.abs(acc) * 2.0 ** -8 + 1e-30
    assert np.all(np.abs(yv - acc) <= bound)
    ratio = float(terms.sum(axis=2).mean() / np.sqrt(np.mean(acc ** 2)))
    print("eta %.2f: sum|terms| / rms(Y) = %.0f, worst |err|/tol = %.3f" % (eta, ratio, worst))


def test_gelu_epilogue_accuracy():
    # Zero codes and scales leave acc = bias, so Y = bf16(GELU(bias)) elementwise: the
    # epilogue's GELU (a rational erf approximation with |error| <= 1.5e-7, evaluated in
    # fp32) must be within 0.5 bf16 ulp of the output plus 4e-7 |x| of the exact erf-form
    # GELU over a sweep of pre-activations, including the far tails.
    from synth import f32_to_bf16_bits
    M, K, N = 8, 64, 4096
    xs = np.concatenate([np.linspace(-12.0, 12.0, N - 8), [0.0, -0.0, 1e-30, -1e-30, 40.0, -40.0,
                                                             3e-5, -3e-5]])
    bias = f32_to_bf16_bits(xs.astype(np.float32))
    b = (bias.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    qa = torch.zeros((bdt.pair_rows(M), K), dtype=torch.uint8, device="cuda:0")
    sa = torch.zeros(bdt.scale_shape(M, K), dtype=torch.float32, device="cuda:0")
    qw = torch.zeros((bdt.pair_rows(N), K), dtype=torch.uint8, device="cuda:0")
    sw = torch.zeros(bdt.scale_shape(N, K), dtype=torch.float32, device="cuda:0")
    Y = bf16_host(bdt.w4a4_lr_gemm(qa, sa, qw, sw, None, None, to_dev(bias), 1))
    y = (Y.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    exact = np.array([oracle.gelu(v) for v in b])
    bound = 0.5 * oracle.bf16_ulp(exact) + 4e-7 * np.abs(b) + 1e-38
    assert np.all(np.abs(y - exact[None, :]) <= bound[None, :])
    assert np.all(y == y[0:1])                     # every row the same


@pytest.mark.parametrize("K", [65536, 65472])
def test_long_k_whole_layer(K):
    # A long reduction: 1024 (even) and 1023 (odd) groups, so that K1 adds 512 chunks of
    # partial down-projections (two groups each at this token count) and the GEMM's K loop
    # runs 512 stages, the odd count ending in a one-group stage.  Ragged M and N, GELU,
    # r = 32.  Codes and scales bit-exact, every output element within the tolerance.
    M, N, r = 70, 136, 32
    L = make_layer(LayerSpec("longk", M, K, N, r, 0.01, 20.0, 4, False, act=1, cfg_id=260 + K % 7))
    qa_o, sa_o, _ = oracle.quantize_act(L.X, L.lam)
    print("long K: M=%d K=%d N=%d r=%d" % (M, K, N, r), flush=True)
    qa, sa, xl1 = bdt.quantize_act_down(to_dev(L.X), to_dev(L.lam), to_dev(L.L1))
    assert np.array_equal(from_pairs(qa, M), qa_o)
    assert np.array_equal(from_stage_major(sa, M, K // 64).view(np.uint32), sa_o.view(np.uint32))
    qw_o, sw_o = oracle.pack_weights(L.R)
    Y = bf16_host(bdt.linear(to_dev(L.X), to_dev(L.lam), to_dev(L.L1), pdev(qw_o), sdev(sw_o),
                             to_dev(L.L2), to_dev(L.bias), 1))
    _, y_or = oracle.linear(L.X, L.lam, L.L1, qw_o, sw_o, L.L2, L.bias, 1)
    worst = assert_y_close(Y, y_or, "long K %d" % K)
    print("  worst |err|/tol = %.3f" % worst, flush=True)
