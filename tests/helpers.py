"""Shared helpers of the GPU parity tests (host side only)."""
from __future__ import annotations

import numpy as np
import torch

import oracle
from synth import bf16_bits_to_f32

DEV = "cuda:0"


def to_dev(a: np.ndarray | None, dtype=None):
    """numpy -> device tensor; uint16 bf16 bit patterns become torch.bfloat16."""
    if a is None:
        return None
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16).copy()).to(DEV).view(torch.bfloat16)
    t = torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    return t if dtype is None else t.to(dtype)


def to_pairs(p: np.ndarray) -> np.ndarray:
    """Row-major packed codes [rows, kb] (the oracle's) -> the device's row-pair layout
    [ceil(rows/2), 2 kb]: each 64-byte chunk of a row followed by the same chunk of its
    pair partner; a shorter last chunk (kb % 64 == 32) interleaves in 32-byte halves."""
    rows, kb = p.shape
    q = np.zeros(((rows + 1) // 2 * 2, kb), np.uint8)
    q[:rows] = p
    out = np.zeros(((rows + 1) // 2, 2 * kb), np.uint8)
    for c0 in range(0, kb, 64):
        w = min(64, kb - c0)
        out[:, 2 * c0:2 * c0 + w] = q[0::2, c0:c0 + w]
        out[:, 2 * c0 + w:2 * c0 + 2 * w] = q[1::2, c0:c0 + w]
    return out


def from_pairs(d, rows: int) -> np.ndarray:
    """Inverse of to_pairs (the unwritten half of an odd count's last pair dropped)."""
    d = d.cpu().numpy() if hasattr(d, "cpu") else np.asarray(d)
    pairs, K = d.shape
    assert pairs == (rows + 1) // 2, (pairs, rows)
    kb = K // 2
    q = np.zeros((2 * pairs, kb), np.uint8)
    for c0 in range(0, kb, 64):
        w = min(64, kb - c0)
        q[0::2, c0:c0 + w] = d[:, 2 * c0:2 * c0 + w]
        q[1::2, c0:c0 + w] = d[:, 2 * c0 + w:2 * c0 + 2 * w]
    return q[:rows]


def pdev(p: np.ndarray):
    """Oracle codes -> device row-pair codes."""
    return to_dev(to_pairs(p))


def to_stage_major(s: np.ndarray) -> np.ndarray:
    """Row-major group scales [R, G] (the oracle's) -> the device's stage-major pairs
    [ceil(G/2), R, 2]: the scale of (row i, group g) at [g // 2, i, g % 2]; an odd G's
    last-stage pad is zero."""
    R, G = s.shape
    out = np.zeros(((G + 1) // 2, R, 2), np.float32)
    for g in range(G):
        out[g // 2, :, g % 2] = s[:, g]
    return out


def from_stage_major(d, R: int, G: int) -> np.ndarray:
    """Inverse of to_stage_major; also checks that an odd G's pad is zero."""
    d = d.cpu().numpy() if hasattr(d, "cpu") else np.asarray(d)
    d = d.reshape((G + 1) // 2, R, 2)
    if G % 2:
        assert np.all(d[-1, :, 1].view(np.uint32) == 0), "pad of the last stage is not +0"
    out = np.empty((R, G), np.float32)
    for g in range(G):
        out[:, g] = d[g // 2, :, g % 2]
    return out


def sdev(s: np.ndarray):
    """Oracle group scales -> device stage-major scales."""
    return to_dev(to_stage_major(s))


def bf16_host(t: torch.Tensor) -> np.ndarray:
    return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)


def bf16_f64(bits: np.ndarray) -> np.ndarray:
    return bf16_bits_to_f32(bits).astype(np.float64)


def y_tolerance(y_oracle_bits: np.ndarray, rms: float | None = None) -> np.ndarray:
    """1 bf16 ulp of |y_oracle| + 1e-3 * rms(y_oracle)."""
    yo = bf16_f64(y_oracle_bits)
    if rms is None:
        rms = float(np.sqrt(np.mean(yo ** 2))) if yo.size else 0.0
    return oracle.bf16_ulp(yo) + 1e-3 * rms


def assert_y_close(y_gpu_bits: np.ndarray, y_oracle_bits: np.ndarray, what: str = "Y",
                   rms: float | None = None) -> float:
    """Element-wise |y_gpu - y_oracle| <= tol; returns max |err| / tol."""
    assert y_gpu_bits.shape == y_oracle_bits.shape
    yg = bf16_f64(y_gpu_bits)
    yo = bf16_f64(y_oracle_bits)
    assert np.all(np.isfinite(yg)), "%s: non-finite GPU output" % what
    tol = y_tolerance(y_oracle_bits, rms)
    err = np.abs(yg - yo)
    ratio = err / np.where(tol > 0, tol, 1e-300)
    bad = err > tol
    if bad.any():
        i = np.unravel_index(np.argmax(ratio), ratio.shape)
        raise AssertionError("%s: %d of %d outside tolerance; worst at %s: gpu %r oracle %r tol %r"
                             % (what, int(bad.sum()), bad.size, i, yg[i], yo[i], tol[i]))
    return float(ratio.max()) if ratio.size else 0.0


def xl1_bound(xh: np.ndarray, L1_bits: np.ndarray) -> np.ndarray:
    """|xl1_gpu - xl1_oracle| bound: (2^-15 + K 2^-24) * sum_k |xh_k L1_ki|."""
    K = xh.shape[1]
    mag = np.abs(xh.astype(np.float64)) @ np.abs(bf16_f64(L1_bits))
    return (2.0 ** -15 + K * 2.0 ** -24) * mag + 1e-30


def awq_records(codes: np.ndarray, scales: np.ndarray, zeros: np.ndarray, N: int, K: int) -> np.ndarray:
    """The W4A16 records (the byte layout documented with svdq_awq_packed_bytes in svdq.h),
    built on the host from row-major codes [N, K/2] (element 2j in the low nibble of byte j),
    fp32 scales [N, K/64] and u8 zeros [N, K/64].  Written from that description alone."""
    G = K // 64
    GQ, NB = (G + 3) // 4, (N + 15) // 16
    q = np.zeros((NB * 16, GQ * 256), np.uint32)
    q[:N, 0:K:2] = codes & 0xF
    q[:N, 1:K:2] = codes >> 4
    s = np.zeros((NB * 16, GQ * 4), np.float32)
    s[:N, :G] = scales
    z = np.zeros((NB * 16, GQ * 4), np.uint8)
    z[:N, :G] = zeros
    # k = 256 t + 64 j + 16 sl + 8 h + e, column n = 16 b + c
    q7 = q.reshape(NB, 16, GQ, 4, 4, 2, 8)                        # b c t j sl h e
    shift = np.array([4 * (e // 2 + 4 * (e % 2)) for e in range(8)], np.uint32)
    words = (q7 << shift).sum(axis=-1, dtype=np.uint64).astype(np.uint32)   # b c t j sl h
    words = words.reshape(NB, 16, GQ, 2, 2, 4, 2)                 # b c t jhi jlo sl h
    # dword 256 jhi + 64 sl + 4 c + 2 jlo + h of the record
    code_dw = words.transpose(0, 2, 3, 5, 1, 4, 6).reshape(NB, GQ, 512)
    scale_dw = s.reshape(NB, 16, GQ, 4).transpose(0, 2, 1, 3).reshape(NB, GQ, 64).view(np.uint32)
    zero_b = z.reshape(NB, 16, GQ, 4).transpose(0, 2, 1, 3).reshape(NB, GQ, 64)
    rec = np.zeros((NB, GQ, 2368), np.uint8)
    rec[:, :, :2048] = code_dw.astype('<u4').view(np.uint8).reshape(NB, GQ, 2048)
    rec[:, :, 2048:2304] = scale_dw.astype('<u4').view(np.uint8).reshape(NB, GQ, 256)
    rec[:, :, 2304:] = zero_b
    return rec.reshape(-1)


def qkv_tolerance(ob: dict, x: np.ndarray, gamma_bits: np.ndarray, eps_y: float) -> np.ndarray:
    """Per-element bound for Q or K of the fused QKV epilogue, from the oracle's values.

    ob: oracle output for one section (fp64 values "o" [R, H, D] and "rho" [R, H]);
    x: the section's exact pre-norm values [R, H, D]; eps_y: the bound on the GPU's
    fp32 pre-norm error (the GEMM tolerance, 1e-3 rms of the projection).  Perturbing x
    by |e| <= eps_y moves x / rho by at most eps_y / rho (1 + |x_d| / rho) per element;
    gamma scales it and the pair turn mixes two elements (sqrt 2); plus 1 bf16 ulp."""
    rho = ob["rho"][..., None]
    xmax = np.abs(x).max(axis=-1, keepdims=True)
    g = np.abs(bf16_f64(gamma_bits)).max()
    return oracle.bf16_ulp(ob["o"]) + 2.0 * np.sqrt(2.0) * g * eps_y / rho * (1.0 + xmax / rho)
