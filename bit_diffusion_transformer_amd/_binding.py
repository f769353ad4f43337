"""ctypes binding of libsvdq.so (the C ABI in include/svdq.h).

Argument marshalling only: every step of the layer runs in the library's
HIP kernels.  torch supplies device memory and the current HIP stream.
There is no fallback: if the library is missing and cannot be built, or the
device is not gfx950, calls raise.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libsvdq.so")

STATUS = {
    0: "SVDQ_OK", 1: "SVDQ_ERR_INVALID_ARG", 2: "SVDQ_ERR_UNSUPPORTED_SHAPE",
    3: "SVDQ_ERR_MISALIGNED", 4: "SVDQ_ERR_WORKSPACE_TOO_SMALL",
    5: "SVDQ_ERR_UNSUPPORTED_DEVICE", 6: "SVDQ_ERR_HIP",
}
ACT_NONE, ACT_GELU = 0, 1
GROUP = 64

# Every symbol declared in include/svdq.h.
EXPORTS = (
    "svdq_abi_version", "svdq_status_string", "svdq_last_error", "svdq_pack_weights",
    "svdq_repack_weights", "svdq_linear_noalloc",
    "svdq_quantize_act_down_workspace_bytes", "svdq_quantize_act_down", "svdq_w4a4_lr_gemm",
    "svdq_linear_workspace_bytes", "svdq_linear", "svdq_debug_group_sums",
    "svdq_debug_set_tile_policy", "svdq_awq_packed_bytes", "svdq_awq_pack_weights",
    "svdq_awq_repack", "svdq_awq_w4a16_linear", "svdq_w4a4_lr_gemm_qkv", "svdq_linear_qkv",
    "svdq_w4a4_lr_gemm_quant_down_workspace_bytes", "svdq_w4a4_lr_gemm_quant_down",
    "svdq_mlp_workspace_bytes", "svdq_mlp", "svdq_mx_pack_weights", "svdq_mx_quantize_act_down",
    "svdq_mx_lr_gemm", "svdq_mx_linear_workspace_bytes", "svdq_mx_linear",
)


class QkvEpilogue(ctypes.Structure):
    """struct svdq_qkv_epilogue of include/svdq.h (device pointers as integers)."""
    _fields_ = [
        ("heads", ctypes.c_int32), ("head_dim", ctypes.c_int32), ("seq", ctypes.c_int64),
        ("gamma_q", ctypes.c_void_p), ("gamma_k", ctypes.c_void_p), ("eps", ctypes.c_float),
        ("cos_t", ctypes.c_void_p), ("sin_t", ctypes.c_void_p),
        ("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
    ]


def qkv_epilogue(heads, head_dim, seq, gamma_q, gamma_k, eps, cos_t, sin_t, q, k, v):
    """Fill a QkvEpilogue from tensors (kept alive by the caller)."""
    def a(t):
        if t is None:
            return None
        if not t.is_contiguous():
            raise ValueError("tensors passed to libsvdq must be contiguous")
        return t.data_ptr()
    return QkvEpilogue(int(heads), int(head_dim), int(seq), a(gamma_q), a(gamma_k), float(eps),
                       a(cos_t), a(sin_t), a(q), a(k), a(v))


class SVDQError(RuntimeError):
    def __init__(self, status: int, detail: str, fn: str):
        self.status = status
        super().__init__("%s: %s (%s)" % (fn, STATUS.get(status, status), detail))


_lib = None


def load_library(build_if_missing: bool = True) -> ctypes.CDLL:
    """Load libsvdq.so; build it first only if it has never been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        if not build_if_missing:
            raise FileNotFoundError(LIB_PATH)
        from .build import build
        build()
    lib = ctypes.CDLL(LIB_PATH)
    P, I64, I32, SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t
    sig = {
        "svdq_abi_version": ([], I32),
        "svdq_status_string": ([I32], ctypes.c_char_p),
        "svdq_last_error": ([], ctypes.c_char_p),
        "svdq_pack_weights": ([P, I64, I64, P, P, P], I32),
        "svdq_repack_weights": ([P, P, I64, I64, P, P, P], I32),
        "svdq_quantize_act_down_workspace_bytes": ([I64, I64, I32], SZ),
        "svdq_quantize_act_down": ([P, P, P, I64, I64, I32, P, P, P, P, SZ, P], I32),
        "svdq_w4a4_lr_gemm": ([P, P, P, P, P, P, P, I32, I64, I64, I64, I32, P, P], I32),
        "svdq_linear_workspace_bytes": ([I64, I64, I32], SZ),
        "svdq_linear": ([P, P, P, P, P, P, P, I32, I64, I64, I64, I32, P, P, SZ, P], I32),
        "svdq_linear_noalloc": ([P, P, P, P, P, P, P, I32, I64, I64, I64, I32, P, P], I32),
        "svdq_debug_group_sums": ([P, P, P, P, I64, I64, I64, I64, I64, I64, I64, P, P], I32),
        "svdq_debug_set_tile_policy": ([I32], I32),
        "svdq_awq_packed_bytes": ([I64, I64], I64),
        "svdq_awq_pack_weights": ([P, I64, I64, P, P], I32),
        "svdq_awq_repack": ([P, P, P, I64, I64, P, P], I32),
        "svdq_awq_w4a16_linear": ([P, P, P, I64, I64, I64, P, P], I32),
        "svdq_w4a4_lr_gemm_qkv": ([P, P, P, P, P, P, P, I64, I64, I32,
                                   ctypes.POINTER(QkvEpilogue), P], I32),
        "svdq_linear_qkv": ([P, P, P, P, P, P, P, I64, I64, I32, ctypes.POINTER(QkvEpilogue),
                             P, SZ, P], I32),
        "svdq_w4a4_lr_gemm_quant_down_workspace_bytes": ([I64, I64, I32], SZ),
        "svdq_w4a4_lr_gemm_quant_down": ([P, P, P, P, P, P, P, I32, I64, I64, I64, I32, P, P, I32,
                                          P, P, P, P, SZ, P], I32),
        "svdq_mlp_workspace_bytes": ([I64, I64, I64, I32, I32], SZ),
        "svdq_mlp": ([P, P, P, P, P, P, P, P, P, P, P, P, P, I32, I64, I64, I64, I32, I32, P, P,
                      SZ, P], I32),
        "svdq_mx_pack_weights": ([P, I64, I64, P, P, P], I32),
        "svdq_mx_quantize_act_down": ([P, P, P, I64, I64, I32, P, P, P, P, SZ, P], I32),
        "svdq_mx_lr_gemm": ([P, P, P, P, P, P, P, I32, I64, I64, I64, I32, P, P], I32),
        "svdq_mx_linear_workspace_bytes": ([I64, I64, I32], SZ),
        "svdq_mx_linear": ([P, P, P, P, P, P, P, I32, I64, I64, I64, I32, P, P, SZ, P], I32),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    _lib = lib
    return lib


def _p(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to libsvdq must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    if stream is None:
        if not torch.cuda.is_available():
            return None
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _check(status: int, fn: str):
    if status != 0:
        detail = load_library().svdq_last_error().decode(errors="replace")
        raise SVDQError(status, detail, fn)


# ------------------------------------------------------------- raw C-ABI calls
# Same names and argument order as include/svdq.h; tensors in, status checked.

def svdq_abi_version() -> int:
    return int(load_library().svdq_abi_version())


def svdq_status_string(status: int) -> str:
    return load_library().svdq_status_string(int(status)).decode()


def svdq_last_error() -> str:
    return load_library().svdq_last_error().decode(errors="replace")


def svdq_repack_weights(codes, scales, N, K, qw, sw, stream=None):
    _check(load_library().svdq_repack_weights(_p(codes), _p(scales), N, K, _p(qw), _p(sw),
                                              _stream(stream)), "svdq_repack_weights")


def svdq_pack_weights(R, N, K, qw, sw, stream=None):
    _check(load_library().svdq_pack_weights(_p(R), N, K, _p(qw), _p(sw), _stream(stream)),
           "svdq_pack_weights")


def svdq_quantize_act_down_workspace_bytes(M, K, r) -> int:
    return int(load_library().svdq_quantize_act_down_workspace_bytes(M, K, r))


def svdq_quantize_act_down(X, lam, L1, M, K, r, qa, sa, xl1, workspace, ws_bytes, stream=None):
    _check(load_library().svdq_quantize_act_down(
        _p(X), _p(lam), _p(L1), M, K, r, _p(qa), _p(sa), _p(xl1), _p(workspace), ws_bytes,
        _stream(stream)), "svdq_quantize_act_down")


def svdq_w4a4_lr_gemm(qa, sa, qw, sw, xl1, L2, bias, act, M, N, K, r, Y, stream=None):
    _check(load_library().svdq_w4a4_lr_gemm(
        _p(qa), _p(sa), _p(qw), _p(sw), _p(xl1), _p(L2), _p(bias), act, M, N, K, r, _p(Y),
        _stream(stream)), "svdq_w4a4_lr_gemm")


def svdq_linear_workspace_bytes(M, K, r) -> int:
    return int(load_library().svdq_linear_workspace_bytes(M, K, r))


def svdq_linear(X, lam, L1, qw, sw, L2, bias, act, M, N, K, r, Y, workspace, ws_bytes,
                stream=None):
    _check(load_library().svdq_linear(
        _p(X), _p(lam), _p(L1), _p(qw), _p(sw), _p(L2), _p(bias), act, M, N, K, r, _p(Y),
        _p(workspace), ws_bytes, _stream(stream)), "svdq_linear")


def svdq_linear_noalloc(X, lam, L1, qw, sw, L2, bias, act, M, N, K, r, Y, stream=None):
    _check(load_library().svdq_linear_noalloc(
        _p(X), _p(lam), _p(L1), _p(qw), _p(sw), _p(L2), _p(bias), act, M, N, K, r, _p(Y),
        _stream(stream)), "svdq_linear_noalloc")


NOALLOC_SCRATCH_BYTES = 64 << 20


def svdq_debug_group_sums(qa, sa, qw, sw, M, N, K, m0, n0, tm, tn, S, stream=None):
    _check(load_library().svdq_debug_group_sums(
        _p(qa), _p(sa), _p(qw), _p(sw), M, N, K, m0, n0, tm, tn, _p(S), _stream(stream)),
        "svdq_debug_group_sums")


TILES_AUTO, TILES_FULL, TILES_QUARTER, TILES_KSPLIT, TILES_KSPLIT_QUARTER = 0, 1, 2, 3, 4


def svdq_debug_set_tile_policy(policy):
    _check(load_library().svdq_debug_set_tile_policy(policy), "svdq_debug_set_tile_policy")


def svdq_awq_packed_bytes(N, K):
    return int(load_library().svdq_awq_packed_bytes(N, K))


def svdq_awq_pack_weights(W, N, K, packed, stream=None):
    _check(load_library().svdq_awq_pack_weights(_p(W), N, K, _p(packed), _stream(stream)),
           "svdq_awq_pack_weights")


def svdq_awq_repack(codes, scales, zeros, N, K, packed, stream=None):
    _check(load_library().svdq_awq_repack(_p(codes), _p(scales), _p(zeros), N, K, _p(packed),
                                          _stream(stream)), "svdq_awq_repack")


def svdq_awq_w4a16_linear(X, packed, bias, M, N, K, Y, stream=None):
    _check(load_library().svdq_awq_w4a16_linear(_p(X), _p(packed), _p(bias), M, N, K, _p(Y),
                                                _stream(stream)), "svdq_awq_w4a16_linear")


def svdq_w4a4_lr_gemm_qkv(qa, sa, qw, sw, xl1, L2, bias, M, K, r, epi: QkvEpilogue, stream=None):
    _check(load_library().svdq_w4a4_lr_gemm_qkv(_p(qa), _p(sa), _p(qw), _p(sw), _p(xl1), _p(L2),
                                                _p(bias), M, K, r, ctypes.byref(epi),
                                                _stream(stream)), "svdq_w4a4_lr_gemm_qkv")


def svdq_linear_qkv(X, lam, L1, qw, sw, L2, bias, M, K, r, epi: QkvEpilogue, workspace,
                    ws_bytes, stream=None):
    _check(load_library().svdq_linear_qkv(_p(X), _p(lam), _p(L1), _p(qw), _p(sw), _p(L2),
                                          _p(bias), M, K, r, ctypes.byref(epi), _p(workspace),
                                          ws_bytes, _stream(stream)), "svdq_linear_qkv")


def svdq_w4a4_lr_gemm_quant_down_workspace_bytes(M, N, r_next) -> int:
    return int(load_library().svdq_w4a4_lr_gemm_quant_down_workspace_bytes(M, N, r_next))


def svdq_w4a4_lr_gemm_quant_down(qa, sa, qw, sw, xl1, L2, bias, act, M, N, K, r, lambda_next,
                                 L1_next, r_next, qa_next, sa_next, xl1_next, workspace,
                                 ws_bytes, stream=None):
    _check(load_library().svdq_w4a4_lr_gemm_quant_down(
        _p(qa), _p(sa), _p(qw), _p(sw), _p(xl1), _p(L2), _p(bias), act, M, N, K, r,
        _p(lambda_next), _p(L1_next), r_next, _p(qa_next), _p(sa_next), _p(xl1_next),
        _p(workspace), ws_bytes, _stream(stream)), "svdq_w4a4_lr_gemm_quant_down")


def svdq_mlp_workspace_bytes(M, K, N_hidden, r_up, r_down) -> int:
    return int(load_library().svdq_mlp_workspace_bytes(M, K, N_hidden, r_up, r_down))


def svdq_mlp(X, lambda_up, L1_up, qw_up, sw_up, L2_up, bias_up, lambda_down, L1_down, qw_down,
             sw_down, L2_down, bias_down, act, M, K, N_hidden, r_up, r_down, Y, workspace,
             ws_bytes, stream=None):
    _check(load_library().svdq_mlp(
        _p(X), _p(lambda_up), _p(L1_up), _p(qw_up), _p(sw_up), _p(L2_up), _p(bias_up),
        _p(lambda_down), _p(L1_down), _p(qw_down), _p(sw_down), _p(L2_down), _p(bias_down),
        act, M, K, N_hidden, r_up, r_down, _p(Y), _p(workspace), ws_bytes, _stream(stream)),
        "svdq_mlp")


def svdq_mx_pack_weights(R, N, K, qw, sw, stream=None):
    _check(load_library().svdq_mx_pack_weights(_p(R), N, K, _p(qw), _p(sw), _stream(stream)),
           "svdq_mx_pack_weights")


def svdq_mx_quantize_act_down(X, lam, L1, M, K, r, qa, sa, xl1, workspace, ws_bytes,
                              stream=None):
    _check(load_library().svdq_mx_quantize_act_down(
        _p(X), _p(lam), _p(L1), M, K, r, _p(qa), _p(sa), _p(xl1), _p(workspace), ws_bytes,
        _stream(stream)), "svdq_mx_quantize_act_down")


def svdq_mx_lr_gemm(qa, sa, qw, sw, xl1, L2, bias, act, M, N, K, r, Y, stream=None):
    _check(load_library().svdq_mx_lr_gemm(
        _p(qa), _p(sa), _p(qw), _p(sw), _p(xl1), _p(L2), _p(bias), act, M, N, K, r, _p(Y),
        _stream(stream)), "svdq_mx_lr_gemm")


def svdq_mx_linear_workspace_bytes(M, K, r) -> int:
    return int(load_library().svdq_mx_linear_workspace_bytes(M, K, r))


def svdq_mx_linear(X, lam, L1, qw, sw, L2, bias, act, M, N, K, r, Y, workspace, ws_bytes,
                   stream=None):
    _check(load_library().svdq_mx_linear(
        _p(X), _p(lam), _p(L1), _p(qw), _p(sw), _p(L2), _p(bias), act, M, N, K, r, _p(Y),
        _p(workspace), ws_bytes, _stream(stream)), "svdq_mx_linear")
