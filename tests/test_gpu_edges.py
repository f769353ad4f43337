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
from tests.helpers import assert_y_close, bf16_host, from_pairs, pdev, to_dev

pytestmark = pytest.mark.gpu


def _layer(M=96, K=256, N=136, r=32, act=0, cid=0):
    return make_layer(LayerSpec("e", M, K, N, r, 0.01, 20.0, 4, False, act=act, cfg_id=200 + cid))


def test_empty_batch():
    L = _layer()
    X = to_dev(L.X)[:0]
    qa, sa, xl1 = bdt.quantize_act_down(X, to_dev(L.lam), to_dev(L.L1))
    assert qa.shape == (0, 256) and sa.shape == (0, 4) and xl1.shape == (0, 32)
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
    assert np.array_equal(sa.cpu().numpy().view(np.uint32), sa_o.view(np.uint32))
    assert (sa_o == 0).any() and ((sa_o > 0) & (sa_o < 2.0 ** -126)).any()
    R = (rng.standard_normal((64, K)) * 0.05).astype(np.float32)
    R[2] = 0.0
    R[4, :64] = np.float32(1e-40)
    qw_o, sw_o = oracle.pack_weights(R)
    qw, sw = bdt.pack_weights(to_dev(R))
    assert np.array_equal(from_pairs(qw, 64), qw_o)
    assert np.array_equal(sw.cpu().numpy().view(np.uint32), sw_o.view(np.uint32))


def test_all_extreme_codes():
    # every group saturated: codes +-7 everywhere, |S| = 3136 per group
    M, K, N = 32, 256, 64
    X = f32_to_bf16_bits(np.where(np.arange(K) % 2 == 0, 3.0, -3.0)[None, :].repeat(M, 0))
    lam = np.ones(K, np.float32)
    R = np.where(np.arange(K) % 2 == 0, -0.5, 0.5)[None, :].repeat(N, 0).astype(np.float32)
    qa_o, sa_o, _ = oracle.quantize_act(X, lam)
    qw_o, sw_o = oracle.pack_weights(R)
    S = bdt.group_sums(pdev(qa_o), pdev(qw_o), M, N, 0, 0, M, N).cpu().numpy()
    assert np.all(S == -3136)
    Y = bdt.w4a4_lr_gemm(pdev(qa_o), to_dev(sa_o), pdev(qw_o), to_dev(sw_o), None, None, None)
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
    sa_b, sa = _padded(M * G, torch.float32, -123.0)
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
