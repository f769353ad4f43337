"""CPU oracle for the SVDQuant W4A4 + low-rank linear (test infrastructure).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  It wraps ``svdq_oracle.c`` (plain C,
fp64 where the method's pages fix no precision) through ctypes and shares
no code with the HIP implementation.  The C file states the definition it
follows and the readings taken where the pages are silent.

Functions whose result is pinned by a test against something other than
the oracle itself (closed forms, invariants, brute force, library special
cases) are listed in ``tests/test_oracle_pins.py``; every function here has
such a pin.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "svdq_oracle.c")
_SRC_AWQ = os.path.join(_HERE, "awq_oracle.c")
_SRC_QKV = os.path.join(_HERE, "qkv_oracle.c")
_SRC_MX = os.path.join(_HERE, "mxfp4_oracle.c")
# SVDQ_ORACLE_LIB points the binding at another build of the same sources (the
# mutation test builds copies with one planted mistake each).
_LIB = os.environ.get("SVDQ_ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")
_lib = None

GROUP = 64


def build(force: bool = True) -> str:
    """Compile the oracle into ``oracle/liboracle.so`` with gcc."""
    if not force and os.path.exists(_LIB):
        return _LIB
    tmp = _LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
           "-std=c11", "-Wall", "-shared", "-fPIC", _SRC, _SRC_AWQ, _SRC_QKV, _SRC_MX, "-o", tmp,
           "-lm"]
    subprocess.check_call(cmd)
    os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB):
        build()
    lib = ctypes.CDLL(_LIB)
    P = ctypes.c_void_p
    I64 = ctypes.c_int64
    I32 = ctypes.c_int32
    lib.oracle_bf16_rne.argtypes = [ctypes.c_double]
    lib.oracle_bf16_rne.restype = ctypes.c_uint16
    lib.oracle_gelu.argtypes = [ctypes.c_double]
    lib.oracle_gelu.restype = ctypes.c_double
    lib.oracle_smooth.argtypes = [P, P, I64, I64, P]
    lib.oracle_quantize_groups.argtypes = [P, I64, I64, P, P]
    lib.oracle_unpack.argtypes = [P, I64, I64, P]
    lib.oracle_down_proj.argtypes = [P, P, I64, I64, I32, P]
    lib.oracle_group_sums.argtypes = [P, P, I64, I64, I64, I64, I64, I64, I64, P]
    lib.oracle_gemm_rows.argtypes = [P, P, P, P, P, P, P, I32, I64, I64, I64, I32,
                                     P, I64, P, P]
    lib.oracle_awq_quantize.argtypes = [P, I64, I64, P, P, P]
    lib.oracle_awq_dequant.argtypes = [P, P, P, I64, I64, P]
    lib.oracle_awq_linear_rows.argtypes = [P, P, P, P, P, I64, I64, I64, P, I64, P, P]
    lib.oracle_mx_e2m1_code.argtypes = [ctypes.c_double]
    lib.oracle_mx_e2m1_code.restype = ctypes.c_int
    lib.oracle_mx_e2m1_value.argtypes = [ctypes.c_int]
    lib.oracle_mx_e2m1_value.restype = ctypes.c_double
    lib.oracle_mx_scale_byte.argtypes = [ctypes.c_double]
    lib.oracle_mx_scale_byte.restype = ctypes.c_int
    lib.oracle_mx_quantize.argtypes = [P, I64, I64, P, P]
    lib.oracle_mx_dequant.argtypes = [P, P, I64, I64, P]
    lib.oracle_mx_gemm_rows.argtypes = [P, P, P, P, P, P, P, I32, I64, I64, I64, I32, P, I64,
                                        P, P]
    lib.oracle_qkv_epilogue.argtypes = [P, P, I64, I64, I64, I64, P, P, ctypes.c_double, P, P,
                                        P, P, P, P, P, P, P]
    for f in ("oracle_smooth", "oracle_quantize_groups", "oracle_unpack",
              "oracle_down_proj", "oracle_group_sums", "oracle_gemm_rows",
              "oracle_awq_quantize", "oracle_awq_dequant", "oracle_awq_linear_rows",
              "oracle_qkv_epilogue", "oracle_mx_quantize", "oracle_mx_dequant",
              "oracle_mx_gemm_rows"):
        getattr(lib, f).restype = None
    _lib = lib
    return lib


def _ptr(a: Optional[np.ndarray]):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle inputs must be contiguous"
    return a.ctypes.data_as(ctypes.c_void_p)


def set_threads(n: int) -> None:
    """OpenMP thread count used by the oracle (via omp_set_num_threads)."""
    lib = _load()
    try:
        fn = lib.omp_set_num_threads
    except AttributeError:
        fn = ctypes.CDLL("libgomp.so.1").omp_set_num_threads
    fn.argtypes = [ctypes.c_int]
    fn(int(n))


def bf16_rne(v: float) -> int:
    """bf16 bit pattern of the nearest bf16 value to the double v (ties to even)."""
    return int(_load().oracle_bf16_rne(float(v)))


def gelu(x: float) -> float:
    return float(_load().oracle_gelu(float(x)))


def smooth(X: np.ndarray, lam: np.ndarray) -> np.ndarray:
    """xh = fl32(bf16 X * fl32(1 / lam)) -> float32 [M, K]."""
    X = np.ascontiguousarray(X, dtype=np.uint16)
    lam = np.ascontiguousarray(lam, dtype=np.float32)
    M, K = X.shape
    xh = np.empty((M, K), np.float32)
    _load().oracle_smooth(_ptr(X), _ptr(lam), M, K, _ptr(xh))
    return xh


def quantize_groups(v: np.ndarray):
    """Group-64 symmetric INT4 quantization -> (packed uint8 [R, K/2], scales f32 [R, K/64])."""
    v = np.ascontiguousarray(v, dtype=np.float32)
    rows, K = v.shape
    assert K % GROUP == 0
    packed = np.empty((rows, K // 2), np.uint8)
    scales = np.empty((rows, K // GROUP), np.float32)
    _load().oracle_quantize_groups(_ptr(v), rows, K, _ptr(packed), _ptr(scales))
    return packed, scales


def unpack(packed: np.ndarray, K: int) -> np.ndarray:
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    rows = packed.shape[0]
    codes = np.empty((rows, K), np.int8)
    _load().oracle_unpack(_ptr(packed), rows, K, _ptr(codes))
    return codes


def quantize_act(X: np.ndarray, lam: np.ndarray):
    """Smoothing + activation quantization -> (qa, sa, xh)."""
    xh = smooth(X, lam)
    qa, sa = quantize_groups(xh)
    return qa, sa, xh


def pack_weights(R: np.ndarray):
    """Offline residual quantization -> (qw uint8 [N, K/2], sw f32 [N, K/64])."""
    return quantize_groups(R)


def down_proj(xh: np.ndarray, L1: np.ndarray) -> np.ndarray:
    """xl1 = xh @ L1 in fp64 -> float64 [M, r]."""
    xh = np.ascontiguousarray(xh, dtype=np.float32)
    L1 = np.ascontiguousarray(L1, dtype=np.uint16)
    M, K = xh.shape
    r = L1.shape[1] if L1.ndim == 2 else 0
    out = np.zeros((M, r), np.float64)
    if r > 0 and M > 0:
        _load().oracle_down_proj(_ptr(xh), _ptr(L1), M, K, r, _ptr(out))
    return out


def group_sums(qa, qw, K: int, m0: int, n0: int, tm: int, tn: int) -> np.ndarray:
    """Exact int32 per-group dot products for a block -> int32 [tm, tn, K/64]."""
    qa = np.ascontiguousarray(qa, dtype=np.uint8)
    qw = np.ascontiguousarray(qw, dtype=np.uint8)
    M, N = qa.shape[0], qw.shape[0]
    S = np.empty((tm, tn, K // GROUP), np.int32)
    _load().oracle_group_sums(_ptr(qa), _ptr(qw), M, N, K, m0, n0, tm, tn, _ptr(S))
    return S


def gemm_rows(qa, sa, qw, sw, xl1: Optional[np.ndarray], L2: Optional[np.ndarray],
              bias: Optional[np.ndarray], act: int, K: int,
              rows: Optional[Sequence[int]] = None):
    """Layer output for the given rows (all rows if None) -> (acc f64 [R, N], y bf16 bits [R, N])."""
    qa = np.ascontiguousarray(qa, dtype=np.uint8)
    sa = np.ascontiguousarray(sa, dtype=np.float32)
    qw = np.ascontiguousarray(qw, dtype=np.uint8)
    sw = np.ascontiguousarray(sw, dtype=np.float32)
    M, N = qa.shape[0], qw.shape[0]
    r = 0 if xl1 is None else xl1.shape[1]
    if r > 0:
        xl1 = np.ascontiguousarray(xl1, dtype=np.float64)
        L2 = np.ascontiguousarray(L2, dtype=np.uint16)
        assert L2.shape == (r, N)
    else:
        xl1 = None
        L2 = None
    if bias is not None:
        bias = np.ascontiguousarray(bias, dtype=np.uint16)
    if rows is None:
        rows_arr = None
        nrows = M
    else:
        rows_arr = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        nrows = len(rows_arr)
    acc = np.empty((nrows, N), np.float64)
    y = np.empty((nrows, N), np.uint16)
    if nrows > 0:
        _load().oracle_gemm_rows(_ptr(qa), _ptr(sa), _ptr(qw), _ptr(sw), _ptr(xl1), _ptr(L2),
                                 _ptr(bias), int(act), M, N, K, r, _ptr(rows_arr), nrows,
                                 _ptr(acc), _ptr(y))
    return acc, y


def linear(X, lam, L1, qw, sw, L2, bias, act: int, rows=None):
    """The whole layer from its call inputs: quantize + down-proj, then the W4A4 GEMM."""
    K = X.shape[1]
    qa, sa, xh = quantize_act(X, lam)
    r = 0 if L1 is None else L1.shape[1]
    xl1 = down_proj(xh, L1) if r > 0 else None
    return gemm_rows(qa, sa, qw, sw, xl1, L2, bias, act, K, rows)


# ---------------------------------------------------------------- W4A16 (awq_w4a16)

def awq_quantize(W: np.ndarray):
    """Group-64 asymmetric INT4 weights -> (packed uint8 [N, K/2], scales f32 [N, K/64],
    zero points uint8 [N, K/64]).  Readings in awq_oracle.c."""
    W = np.ascontiguousarray(W, dtype=np.float32)
    N, K = W.shape
    assert K % GROUP == 0
    packed = np.empty((N, K // 2), np.uint8)
    scales = np.empty((N, K // GROUP), np.float32)
    zeros = np.empty((N, K // GROUP), np.uint8)
    if N > 0:
        _load().oracle_awq_quantize(_ptr(W), N, K, _ptr(packed), _ptr(scales), _ptr(zeros))
    return packed, scales, zeros


def awq_dequant(packed, scales, zeros, K: int) -> np.ndarray:
    """(q - z) * s in fp64 -> float64 [N, K]."""
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.float32)
    zeros = np.ascontiguousarray(zeros, dtype=np.uint8)
    N = packed.shape[0]
    out = np.empty((N, K), np.float64)
    if N > 0:
        _load().oracle_awq_dequant(_ptr(packed), _ptr(scales), _ptr(zeros), N, K, _ptr(out))
    return out


def awq_linear(X, packed, scales, zeros, bias, rows: Optional[Sequence[int]] = None):
    """Y = X W^T + bias of the W4A16 layer -> (acc f64 [R, N], y bf16 bits [R, N])."""
    X = np.ascontiguousarray(X, dtype=np.uint16)
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.float32)
    zeros = np.ascontiguousarray(zeros, dtype=np.uint8)
    if bias is not None:
        bias = np.ascontiguousarray(bias, dtype=np.uint16)
    M, K = X.shape
    N = packed.shape[0]
    if rows is None:
        rows_arr, nrows = None, M
    else:
        rows_arr = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        nrows = len(rows_arr)
    acc = np.empty((nrows, N), np.float64)
    y = np.empty((nrows, N), np.uint16)
    if nrows > 0 and N > 0:
        _load().oracle_awq_linear_rows(_ptr(X), _ptr(packed), _ptr(scales), _ptr(zeros),
                                       _ptr(bias), M, N, K, _ptr(rows_arr), nrows, _ptr(acc),
                                       _ptr(y))
    return acc, y


def bf16_ulp(v: np.ndarray) -> np.ndarray:
    """ulp of bf16 values: 2^(floor(log2|v|) - 7) for normal v, 2^-133 below 2^-126, 0 for v == 0."""
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    out = np.zeros_like(a)
    nz = a > 0
    e = np.floor(np.log2(a[nz]))
    e = np.maximum(e, -126.0)
    out[nz] = np.exp2(e - 7.0)
    return out


# ---------------------------------------------------------------- fused QKV epilogue

def qkv_epilogue(acc: np.ndarray, H: int, D: int, S: int, gamma_q: np.ndarray,
                 gamma_k: np.ndarray, eps: float, cos_t: np.ndarray, sin_t: np.ndarray,
                 rows: Optional[Sequence[int]] = None):
    """Per-head RMS norm + rotary embedding of Q and K, V re-laid out (readings in
    qkv_oracle.c).  acc: fp64 [R, 3 H D], the exact projection output of tokens
    ``rows`` (token i if None).  Returns dict with q, k (fp64 [R, H, D]), qb, kb, vb
    (bf16 bits [R, H, D]) and rho_q, rho_k (fp64 [R, H])."""
    acc = np.ascontiguousarray(acc, dtype=np.float64)
    R = acc.shape[0]
    assert acc.shape[1] == 3 * H * D and D % 2 == 0
    gq = np.ascontiguousarray(gamma_q, dtype=np.uint16)
    gk = np.ascontiguousarray(gamma_k, dtype=np.uint16)
    ct = np.ascontiguousarray(cos_t, dtype=np.float32)
    st = np.ascontiguousarray(sin_t, dtype=np.float32)
    assert ct.shape == (S, D // 2) and st.shape == (S, D // 2)
    rows_arr = None if rows is None else np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    out = dict(q=np.empty((R, H, D)), k=np.empty((R, H, D)),
               qb=np.empty((R, H, D), np.uint16), kb=np.empty((R, H, D), np.uint16),
               vb=np.empty((R, H, D), np.uint16), rho_q=np.empty((R, H)), rho_k=np.empty((R, H)))
    if R > 0:
        _load().oracle_qkv_epilogue(_ptr(acc), _ptr(rows_arr), R, H, D, S, _ptr(gq), _ptr(gk),
                                    float(eps), _ptr(ct), _ptr(st), _ptr(out["q"]),
                                    _ptr(out["k"]), _ptr(out["qb"]), _ptr(out["kb"]),
                                    _ptr(out["vb"]), _ptr(out["rho_q"]), _ptr(out["rho_k"]))
    return out


# ---------------------------------------------------------------- MXFP4 variant

MX_BLOCK = 32


def mx_e2m1_code(y: float) -> int:
    return int(_load().oracle_mx_e2m1_code(float(y)))


def mx_e2m1_value(code: int) -> float:
    return float(_load().oracle_mx_e2m1_value(int(code)))


def mx_scale_byte(amax: float) -> int:
    return int(_load().oracle_mx_scale_byte(float(amax)))


def mx_quantize(v: np.ndarray):
    """fp32 [rows, K] -> (packed codes uint8 [rows, K/2], E8M0 scale bytes uint8 [rows, K/32]).
    Readings in mxfp4_oracle.c."""
    v = np.ascontiguousarray(v, dtype=np.float32)
    rows, K = v.shape
    assert K % MX_BLOCK == 0
    packed = np.empty((rows, K // 2), np.uint8)
    scales = np.empty((rows, K // MX_BLOCK), np.uint8)
    if rows:
        _load().oracle_mx_quantize(_ptr(v), rows, K, _ptr(packed), _ptr(scales))
    return packed, scales


def mx_dequant(packed: np.ndarray, scales: np.ndarray, K: int) -> np.ndarray:
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    rows = packed.shape[0]
    out = np.empty((rows, K), np.float64)
    if rows:
        _load().oracle_mx_dequant(_ptr(packed), _ptr(scales), rows, K, _ptr(out))
    return out


def mx_quantize_act(X: np.ndarray, lam: np.ndarray):
    """Smoothing (as the INT4 path) then MXFP4 -> (qa, sa bytes, xh fp32)."""
    xh = smooth(X, lam)
    qa, sa = mx_quantize(xh)
    return qa, sa, xh


def mx_gemm_rows(qa, sa, qw, sw, xl1: Optional[np.ndarray], L2: Optional[np.ndarray],
                 bias: Optional[np.ndarray], act: int, K: int,
                 rows: Optional[Sequence[int]] = None):
    """MXFP4 layer output for the given rows -> (acc f64 [R, N], y bf16 bits [R, N])."""
    qa = np.ascontiguousarray(qa, dtype=np.uint8)
    sa = np.ascontiguousarray(sa, dtype=np.uint8)
    qw = np.ascontiguousarray(qw, dtype=np.uint8)
    sw = np.ascontiguousarray(sw, dtype=np.uint8)
    M, N = qa.shape[0], qw.shape[0]
    r = 0 if xl1 is None else xl1.shape[1]
    if r > 0:
        xl1 = np.ascontiguousarray(xl1, dtype=np.float64)
        L2 = np.ascontiguousarray(L2, dtype=np.uint16)
    else:
        xl1, L2 = None, None
    if bias is not None:
        bias = np.ascontiguousarray(bias, dtype=np.uint16)
    rows_arr = None if rows is None else np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    nrows = M if rows is None else len(rows_arr)
    acc = np.empty((nrows, N), np.float64)
    y = np.empty((nrows, N), np.uint16)
    if nrows > 0:
        _load().oracle_mx_gemm_rows(_ptr(qa), _ptr(sa), _ptr(qw), _ptr(sw), _ptr(xl1), _ptr(L2),
                                    _ptr(bias), int(act), M, N, K, r, _ptr(rows_arr), nrows,
                                    _ptr(acc), _ptr(y))
    return acc, y


def mx_linear(X, lam, L1, qw, sw, L2, bias, act: int, rows=None):
    """The whole MXFP4 layer from its call inputs."""
    K = X.shape[1]
    qa, sa, xh = mx_quantize_act(X, lam)
    r = 0 if L1 is None else L1.shape[1]
    xl1 = down_proj(xh, L1) if r > 0 else None
    return mx_gemm_rows(qa, sa, qw, sw, xl1, L2, bias, act, K, rows)
