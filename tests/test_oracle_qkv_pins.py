"""Pins of the fused-QKV-epilogue part of the CPU oracle against things other than itself.

Hand-derived fixtures, torch's own rms_norm, the rotation written as a
complex product, invariants (unit mean square, scale invariance), turning
back by the opposite angle, position periodicity, and the V layout.
"""
import os

import numpy as np
import pytest
import torch

import oracle
from synth import f32_to_bf16_bits

HERE = os.path.dirname(os.path.abspath(__file__))


def _fixtures():
    out = []
    for line in open(os.path.join(HERE, "golden", "qkv_fixtures.txt")):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        f = [t.strip() for t in line.split("|")]
        vals = [np.array([float(t) for t in x.split()]) for x in f[1:7]]
        out.append((f[0], vals[0], vals[1], float(f[3]), vals[3], vals[4], vals[5], float(f[7])))
    return out


def _one_head(x, gamma, eps, cosv, sinv):
    D = len(x)
    acc = np.zeros((1, 3 * D))
    acc[0, :D] = x
    acc[0, D:2 * D] = x
    g = f32_to_bf16_bits(np.asarray(gamma, np.float32))
    ct = np.asarray(cosv, np.float32).reshape(1, D // 2)
    st = np.asarray(sinv, np.float32).reshape(1, D // 2)
    return oracle.qkv_epilogue(acc, 1, D, 1, g, g, eps, ct, st)


@pytest.mark.parametrize("fx", _fixtures(), ids=lambda f: f[0])
def test_hand_fixtures(fx):
    name, x, gamma, eps, cosv, sinv, want, rho = fx
    o = _one_head(x, gamma, eps, cosv, sinv)
    # fp32 tables: cos/sin such as 0.6 are not exact, so 1e-7 absolute
    assert np.allclose(o["q"][0, 0], want, rtol=0, atol=1e-7), (o["q"], want)
    assert np.allclose(o["k"][0, 0], want, rtol=0, atol=1e-7)
    assert o["rho_q"][0, 0] == pytest.approx(rho, rel=1e-15)


def _random_case(rng, R=7, H=3, D=8, S=5):
    acc = rng.standard_normal((R, 3 * H * D)) * np.exp(rng.uniform(-2, 2, (R, 1)))
    gq = f32_to_bf16_bits(rng.uniform(0.5, 1.5, D).astype(np.float32))
    gk = f32_to_bf16_bits(rng.uniform(0.5, 1.5, D).astype(np.float32))
    ang = rng.uniform(-np.pi, np.pi, (S, D // 2))
    return acc, gq, gk, np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)


def _bf16_f64(b):
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def test_identity_turn_equals_torch_rms_norm():
    rng = np.random.default_rng(31)
    R, H, D, S = 6, 2, 16, 3
    acc, gq, gk, _, _ = _random_case(rng, R, H, D, S)
    ones, zeros = np.ones((S, D // 2), np.float32), np.zeros((S, D // 2), np.float32)
    eps = 1e-6
    o = oracle.qkv_epilogue(acc, H, D, S, gq, gk, eps, ones, zeros)
    x = torch.from_numpy(acc.reshape(R, 3, H, D))
    want_q = torch.nn.functional.rms_norm(x[:, 0], (D,), torch.from_numpy(_bf16_f64(gq)), eps)
    want_k = torch.nn.functional.rms_norm(x[:, 1], (D,), torch.from_numpy(_bf16_f64(gk)), eps)
    assert np.allclose(o["q"], want_q.numpy(), rtol=1e-13, atol=1e-15)
    assert np.allclose(o["k"], want_k.numpy(), rtol=1e-13, atol=1e-15)


def test_turn_is_a_complex_product():
    rng = np.random.default_rng(32)
    R, H, D, S = 9, 2, 8, 4
    acc, gq, gk, ct, st = _random_case(rng, R, H, D, S)
    eps = 1e-5
    o = oracle.qkv_epilogue(acc, H, D, S, gq, gk, eps, ct, st)
    x = acc.reshape(R, 3, H, D)
    for which, g, key in ((0, gq, "q"), (1, gk, "k")):
        v = x[:, which] / np.sqrt((x[:, which] ** 2).mean(-1, keepdims=True) + eps) * _bf16_f64(g)
        z = v[..., 0::2] + 1j * v[..., 1::2]
        pos = np.arange(R) % S
        w = z * (ct[pos].astype(np.float64) + 1j * st[pos].astype(np.float64))[:, None, :]
        got = o[key]
        assert np.allclose(got[..., 0::2], w.real, rtol=1e-13, atol=1e-14)
        assert np.allclose(got[..., 1::2], w.imag, rtol=1e-13, atol=1e-14)


def test_unit_mean_square_and_scale_invariance():
    rng = np.random.default_rng(33)
    R, H, D, S = 5, 4, 32, 5
    acc, _, _, ct, st = _random_case(rng, R, H, D, S)
    one = f32_to_bf16_bits(np.ones(D, np.float32))
    o = oracle.qkv_epilogue(acc, H, D, S, one, one, 0.0, ct, st)
    # |cos|^2 + |sin|^2 = 1 only to fp32 precision
    assert np.allclose((o["q"] ** 2).mean(-1), 1.0, rtol=0, atol=1e-6)
    assert np.allclose((o["k"] ** 2).mean(-1), 1.0, rtol=0, atol=1e-6)
    o2 = oracle.qkv_epilogue(acc * 1024.0, H, D, S, one, one, 0.0, ct, st)
    assert np.allclose(o2["q"], o["q"], rtol=1e-14, atol=1e-15)
    assert np.allclose(o2["rho_q"], 1024.0 * o["rho_q"], rtol=1e-14)


def test_turning_back_recovers_the_normalized_head():
    rng = np.random.default_rng(34)
    R, H, D, S = 4, 2, 8, 4
    acc, _, _, ct, st = _random_case(rng, R, H, D, S)
    one = f32_to_bf16_bits(np.ones(D, np.float32))
    o = oracle.qkv_epilogue(acc, H, D, S, one, one, 0.0, ct, st)
    back = np.zeros_like(acc)
    back[:, :H * D] = o["q"].reshape(R, H * D)
    back[:, H * D:2 * H * D] = o["k"].reshape(R, H * D)
    # cos^2 + sin^2 = 1 + O(2^-24) for the fp32 tables, so rho of the turned head is 1 to 1e-7
    o2 = oracle.qkv_epilogue(back, H, D, S, one, one, 0.0, ct, -st)
    x = acc.reshape(R, 3, H, D)
    vq = x[:, 0] / np.sqrt((x[:, 0] ** 2).mean(-1, keepdims=True))
    assert np.allclose(o2["q"], vq, rtol=0, atol=1e-6)


def test_position_is_token_mod_seq_and_v_layout():
    rng = np.random.default_rng(35)
    H, D, S = 2, 4, 3
    base = rng.standard_normal((1, 3 * H * D))
    acc = np.repeat(base, 7, axis=0)                  # tokens 0..6 carry the same projection
    _, gq, gk, ct, st = _random_case(rng, 7, H, D, S)
    o = oracle.qkv_epilogue(acc, H, D, S, gq, gk, 1e-6, ct, st)
    for m in range(7):
        assert np.array_equal(o["q"][m], o["q"][m % S])
    assert not np.array_equal(o["q"][0], o["q"][1])
    rows = [5, 1]
    o_sub = oracle.qkv_epilogue(acc[rows], H, D, S, gq, gk, 1e-6, ct, st, rows=rows)
    assert np.array_equal(o_sub["q"], o["q"][rows])
    want_v = np.vectorize(oracle.bf16_rne)(acc[:, 2 * H * D:]).astype(np.uint16).reshape(7, H, D)
    assert np.array_equal(o["vb"], want_v)
    assert np.array_equal(o["qb"], np.vectorize(oracle.bf16_rne)(o["q"]).astype(np.uint16))
