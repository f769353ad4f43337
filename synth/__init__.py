"""Seeded synthetic inputs for the SVDQuant W4A4 + low-rank linear layer.

This module is shared by the CPU oracle (``oracle/``) and the HIP path
(``bit_diffusion_transformer_amd``); it holds none of the layer's own
arithmetic (no quantization, packing, integer dot, rescale, low-rank
product, bias or activation of the output).  It only draws the tensors a
layer is called with, and builds the offline weight artefacts that a
quantization toolchain would hand to the layer:

* X   bf16 [M, K]  token activations (returned as uint16 bit patterns),
* lam fp32 [K]     smoothing factors that move activation outliers into
                   the weights ("SVDQuant overview", stage 2, on the
                   svdq-int4-flux.1-canny-dev model card),
* L1  bf16 [K, r], L2 bf16 [r, N]  the 16-bit low-rank branch from a
                   truncated SVD of the smoothed weight (stage 3),
* R   fp32 [N, K]  the residual the 4-bit path quantizes (stage 3),
* bias bf16 [N].

Recipe (all draws from ``numpy.random.Generator(PCG64(SeedSequence(
[seed, cfg_id, layer_id])))`` in this order: X normals, outlier channels,
W noise, planted factors, bias):

1. X = N(0,1) in fp64 (C4 applies the erf-form GELU to it first, as an
   input distribution, via ``scipy.special.erf``); ``n_out = round(p*K)``
   distinct channels chosen without replacement are multiplied by the
   outlier factor; rounded to bf16 via fp32 (RNE at each step).
2. W = N(0, 1/K) noise [N, K] plus a planted term sum_i s_i u_i v_i^T with
   orthonormal u (N) and v (K) from QR of Gaussian matrices;
   s_1 = 4 (1 + sqrt(N/K)) (four times the noise's largest singular value),
   s_i = s_1 / i for a decaying spectrum, s_i = s_1 for a flat one. W is
   stored fp32.
3. lam_j = sqrt(max_m |X_mj| / max_n |W_nj|) in fp64, 1 where either max
   is 0, stored fp32.
4. W_hat = diag(lam) . W^T (K x N, fp64). Its rank-r truncated SVD
   U S V^T gives L1 = U_r S_r, L2 = V_r^T, each rounded to bf16 (via fp32).
   The SVD is exact (LAPACK) when min(K, N) <= 1024, else randomized
   subspace iteration (oversampling 16, 3 power iterations, its own seeded
   stream).  R = (W_hat - L1 L2)^T in fp64, stored fp32: the residual
   absorbs the bf16 rounding of the factors.
5. bias = N(0, 0.02^2) rounded to bf16.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np

__all__ = [
    "LayerSpec", "CONFIGS", "make_layer", "make_config_layers",
    "f32_to_bf16_bits", "bf16_bits_to_f32", "DIT_CHAIN",
    "AwqSpec", "AWQ_CONFIGS", "make_awq_layer", "QkvEpi", "make_qkv_epilogue",
]


def f32_to_bf16_bits(a) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest, ties to even."""
    a = np.ascontiguousarray(np.asarray(a, dtype=np.float32))
    u = a.view(np.uint32).astype(np.uint64)
    nan = np.isnan(a)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    out = rounded.astype(np.uint16)
    out[nan] = 0x7FC0
    return out


def bf16_bits_to_f32(b) -> np.ndarray:
    b = np.asarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def _to_bf16(a64: np.ndarray) -> np.ndarray:
    return f32_to_bf16_bits(np.asarray(a64, dtype=np.float64).astype(np.float32))


@dataclass(frozen=True)
class LayerSpec:
    """One linear layer's shape and input recipe."""
    name: str
    M: int
    K: int
    N: int
    r: int
    outlier_frac: float
    outlier_scale: float
    planted_rank: int
    planted_decay: bool          # True: s_i = s_1 / i, False: flat
    act: int = 0                 # 0 none, 1 GELU (erf form)
    x_gelu: bool = False         # X = GELU(N(0,1)) before outliers
    bias: bool = True
    cfg_id: int = 0
    layer_id: int = 0

    def with_M(self, M: int) -> "LayerSpec":
        d = dict(self.__dict__)
        d["M"] = M
        return LayerSpec(**d)


# The five workloads: a tiny layer, the fused QKV projection of a DiT block
# at 4096 image + 512 text tokens, the MLP up-projection with GELU, the MLP
# down-projection (long K), and one block's chain of four linears.
CONFIGS = {
    "tiny": LayerSpec("tiny", 256, 512, 512, 16, 0.01, 20.0, 4, False, cfg_id=0),
    "qkv": LayerSpec("qkv", 4608, 3072, 9216, 32, 0.005, 30.0, 8, True, cfg_id=1),
    "mlp_up": LayerSpec("mlp_up", 4096, 3072, 12288, 32, 0.01, 20.0, 16, False,
                        act=1, cfg_id=2),
    "mlp_down": LayerSpec("mlp_down", 4096, 12288, 3072, 32, 0.01, 10.0, 16, False,
                          x_gelu=True, cfg_id=3),
}

# One DiT block's linear chain (run back to back); each layer's inputs are
# generated independently from the block seed.
DIT_CHAIN = [
    LayerSpec("chain_qkv", 4608, 3072, 9216, 32, 0.005, 30.0, 8, True, cfg_id=4, layer_id=0),
    LayerSpec("chain_out", 4608, 3072, 3072, 32, 0.005, 30.0, 8, True, cfg_id=4, layer_id=1),
    LayerSpec("chain_up", 4608, 3072, 12288, 32, 0.01, 20.0, 16, False, act=1,
              cfg_id=4, layer_id=2),
    LayerSpec("chain_down", 4608, 12288, 3072, 32, 0.01, 10.0, 16, False, x_gelu=True,
              cfg_id=4, layer_id=3),
]


@dataclass
class Layer:
    spec: LayerSpec
    X: np.ndarray           # uint16 [M, K] bf16 bits
    lam: np.ndarray         # float32 [K]
    L1: np.ndarray          # uint16 [K, r]
    L2: np.ndarray          # uint16 [r, N]
    R: np.ndarray           # float32 [N, K]
    bias: Optional[np.ndarray]  # uint16 [N] or None
    W: np.ndarray = field(repr=False, default=None)  # float32 [N, K] (unquantized)


def _orthonormal(rng: np.random.Generator, n: int, k: int) -> np.ndarray:
    q, _ = np.linalg.qr(rng.standard_normal((n, k)))
    return q


def _truncated_svd(A: np.ndarray, r: int, rng: np.random.Generator):
    """Rank-r truncated SVD of A (fp64). Exact for small matrices."""
    if min(A.shape) <= 1024:
        U, S, Vt = np.linalg.svd(A, full_matrices=False)
        return U[:, :r], S[:r], Vt[:r]
    p = r + 16
    Om = rng.standard_normal((A.shape[1], p))
    Y = A @ Om
    Q, _ = np.linalg.qr(Y)
    for _ in range(3):
        Z, _ = np.linalg.qr(A.T @ Q)
        Q, _ = np.linalg.qr(A @ Z)
    B = Q.T @ A
    Ub, S, Vt = np.linalg.svd(B, full_matrices=False)
    U = Q @ Ub
    return U[:, :r], S[:r], Vt[:r]


def make_layer(spec: LayerSpec, seed: int = 0, M: Optional[int] = None,
               keep_w: bool = False, bias: Optional[bool] = None) -> Layer:
    """Generate one layer's inputs by the recipe in the module docstring."""
    M = spec.M if M is None else int(M)
    K, N, r = spec.K, spec.N, spec.r
    ss = np.random.SeedSequence([seed, spec.cfg_id, spec.layer_id])
    rng = np.random.Generator(np.random.PCG64(ss))

    # 1. activations
    X = rng.standard_normal((M, K))
    if spec.x_gelu:
        from scipy.special import erf
        X = 0.5 * X * (1.0 + erf(X / np.sqrt(2.0)))
    n_out = int(round(spec.outlier_frac * K))
    chans = rng.choice(K, size=n_out, replace=False) if n_out > 0 else np.zeros(0, int)
    X[:, chans] *= spec.outlier_scale
    Xb = _to_bf16(X)

    # 2. weights: noise + planted low-rank term
    W = rng.standard_normal((N, K)) * np.sqrt(1.0 / K)
    if spec.planted_rank > 0:
        pr = spec.planted_rank
        u = _orthonormal(rng, N, pr)
        v = _orthonormal(rng, K, pr)
        s1 = 4.0 * (1.0 + np.sqrt(N / K))
        s = s1 / np.arange(1, pr + 1) if spec.planted_decay else np.full(pr, s1)
        W += (u * s) @ v.T
    W32 = W.astype(np.float32)
    del W

    # 5. bias (drawn before the SVD stream so the draw order stays fixed)
    want_bias = spec.bias if bias is None else bias
    b = rng.standard_normal(N) * 0.02
    bias_bits = _to_bf16(b) if want_bias else None

    # 3. smoothing factors
    xmax = np.abs(bf16_bits_to_f32(Xb).astype(np.float64)).max(axis=0) if M > 0 \
        else np.zeros(K)
    wmax = np.abs(W32.astype(np.float64)).max(axis=0)
    ok = (xmax > 0) & (wmax > 0)
    lam64 = np.ones(K)
    lam64[ok] = np.sqrt(xmax[ok] / wmax[ok])
    lam = lam64.astype(np.float32)

    # 4. smoothed weight, truncated SVD, residual
    W_hat = W32.T.astype(np.float64) * lam.astype(np.float64)[:, None]   # [K, N]
    svd_rng = np.random.Generator(np.random.PCG64(
        np.random.SeedSequence([seed, spec.cfg_id, spec.layer_id, 1])))
    if r > 0:
        U, S, Vt = _truncated_svd(W_hat, r, svd_rng)
        L1 = _to_bf16(U * S)
        L2 = _to_bf16(Vt)
        R = W_hat - bf16_bits_to_f32(L1).astype(np.float64) @ bf16_bits_to_f32(L2).astype(np.float64)
    else:
        L1 = np.zeros((K, 0), np.uint16)
        L2 = np.zeros((0, N), np.uint16)
        R = W_hat
    R32 = np.ascontiguousarray(R.T.astype(np.float32))
    del R, W_hat
    return Layer(spec.with_M(M), np.ascontiguousarray(Xb), lam, np.ascontiguousarray(L1),
                 np.ascontiguousarray(L2), R32, bias_bits, W32 if keep_w else None)


def make_config_layers(name: str, seed: int = 0, M: Optional[int] = None):
    """Layers of a named workload: one for a single-layer config, four for the chain."""
    if name == "chain":
        return [make_layer(s, seed, M=M) for s in DIT_CHAIN]
    return [make_layer(CONFIGS[name], seed, M=M)]


# ---------------------------------------------------------------- W4A16 (awq_w4a16)
# The modulation projection of a DiT block (adaptive layer norm): a few
# conditioning vectors (one per image in the batch; SiLU of a normal, as the
# projection's input is the SiLU of the timestep / text embedding) against a
# 3072 -> 6 x 3072 weight (shift, scale and gate for attention and MLP).

@dataclass
class AwqSpec:
    name: str
    M: int
    K: int
    N: int
    bias: bool = True
    cfg_id: int = 20


AWQ_CONFIGS = {
    "awq_mod": AwqSpec("awq_mod", 2, 3072, 18432, cfg_id=20),
    "awq_mod_single": AwqSpec("awq_mod_single", 2, 3072, 9216, cfg_id=21),
}


@dataclass
class AwqLayer:
    spec: AwqSpec
    X: np.ndarray               # uint16 [M, K] bf16 bits
    W: np.ndarray               # float32 [N, K]
    bias: Optional[np.ndarray]  # uint16 [N] or None


def make_awq_layer(spec: AwqSpec, seed: int = 0, M: Optional[int] = None) -> AwqLayer:
    """Seeded inputs of a W4A16 layer: X = SiLU(N(0,1)) in bf16; W rows N(0, 1/K)
    with a per-row spread of 4x; bias N(0, 0.02)."""
    M = spec.M if M is None else M
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, spec.cfg_id, 0])))
    z = rng.standard_normal((M, spec.K))
    X = _to_bf16(z / (1.0 + np.exp(-z)))
    row = np.exp(rng.uniform(-np.log(2.0), np.log(2.0), size=(spec.N, 1)))
    W = (rng.standard_normal((spec.N, spec.K)) * (row / np.sqrt(spec.K))).astype(np.float32)
    bias = _to_bf16(0.02 * rng.standard_normal(spec.N)) if spec.bias else None
    return AwqLayer(AwqSpec(spec.name, M, spec.K, spec.N, spec.bias, spec.cfg_id),
                    np.ascontiguousarray(X), np.ascontiguousarray(W), bias)


# ---------------------------------------------------------------- fused QKV epilogue inputs

@dataclass
class QkvEpi:
    heads: int
    head_dim: int
    seq: int
    gamma_q: np.ndarray     # uint16 [D] bf16 bits
    gamma_k: np.ndarray     # uint16 [D] bf16 bits
    eps: float
    cos_t: np.ndarray       # float32 [S, D/2]
    sin_t: np.ndarray       # float32 [S, D/2]


def make_qkv_epilogue(heads: int, head_dim: int, seq: int, seed: int = 0, cfg_id: int = 40,
                      theta: float = 10000.0, eps: float = 1e-6) -> QkvEpi:
    """Seeded inputs of the fused QKV epilogue: norm weights bf16(U(0.5, 1.5)) and the
    rotary tables of positions s = 0 .. S-1 with frequencies theta^(-2p/D) (the standard
    one-axis table, standing in for a model's multi-axis one: the tables are caller
    inputs), angles in fp64, cos / sin rounded to fp32."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, cfg_id, 7])))
    gq = _to_bf16(rng.uniform(0.5, 1.5, head_dim))
    gk = _to_bf16(rng.uniform(0.5, 1.5, head_dim))
    freq = theta ** (-2.0 * np.arange(head_dim // 2) / head_dim)
    ang = np.arange(seq, dtype=np.float64)[:, None] * freq[None, :]
    return QkvEpi(heads, head_dim, seq, gq, gk, eps, np.cos(ang).astype(np.float32),
                  np.sin(ang).astype(np.float32))
