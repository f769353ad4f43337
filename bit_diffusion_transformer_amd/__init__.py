"""SVDQuant W4A4 + low-rank linear layer for MI355X (gfx950).

The layer computes ``Y = act(Q4(X diag(lam)^-1) Q4(R)^T + (X diag(lam)^-1 L1) L2 + bias)``
with group-64 INT4 activations and weights and a bf16 rank-r branch, in two
HIP kernels behind the C ABI of ``include/svdq.h``.  This package is the
thin Python binding: the ``svdq_*`` functions mirror the C entry points one
to one, and the tensor helpers below only allocate outputs and workspaces.

bf16 tensors may be passed as ``torch.bfloat16`` or as their ``int16``/
``uint16`` bit patterns; they are reinterpreted, never converted.
"""
from __future__ import annotations

from typing import Optional

import torch

from ._binding import (ACT_GELU, ACT_NONE, EXPORTS, GROUP, LIB_PATH, SVDQError,  # noqa: F401
                       QkvEpilogue, TILES_AUTO, TILES_FULL, TILES_QUARTER, TILES_KSPLIT,
                       TILES_KSPLIT_QUARTER, qkv_epilogue,
                       load_library, svdq_abi_version, svdq_awq_pack_weights,
                       svdq_awq_packed_bytes, svdq_awq_repack,
                       svdq_awq_w4a16_linear, svdq_debug_group_sums,
                       svdq_debug_set_tile_policy,
                       svdq_last_error, svdq_linear, svdq_linear_noalloc, svdq_linear_workspace_bytes,
                       svdq_pack_weights, svdq_repack_weights, svdq_quantize_act_down,
                       svdq_quantize_act_down_workspace_bytes, svdq_status_string,
                       svdq_w4a4_lr_gemm, svdq_w4a4_lr_gemm_qkv, svdq_linear_qkv,
                       svdq_w4a4_lr_gemm_quant_down,
                       svdq_w4a4_lr_gemm_quant_down_workspace_bytes, svdq_mlp,
                       svdq_mlp_workspace_bytes, svdq_mx_pack_weights,
                       svdq_mx_quantize_act_down, svdq_mx_lr_gemm,
                       svdq_mx_linear_workspace_bytes, svdq_mx_linear)

MX_BLOCK = 32   # values per E8M0 scale in the MXFP4 variant


def mx_scale_rows(rows: int) -> int:
    """Padded row count P of the block-major MXFP4 scale bytes [K/32, P]."""
    return (int(rows) + 15) // 16 * 16


def _bits(t: Optional[torch.Tensor]) -> Optional[torch.Tensor]:
    """bf16 tensor -> the same storage viewed as int16 (no copy)."""
    if t is None:
        return None
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16)
    if t.dtype in (torch.int16, torch.uint16):
        return t
    raise TypeError("expected bf16 (or its 16-bit pattern), got %s" % t.dtype)


def _rank(L: Optional[torch.Tensor], dim: int) -> int:
    return 0 if L is None or L.numel() == 0 else int(L.shape[dim])


def pair_rows(rows: int) -> int:
    """Leading dimension of packed 4-bit codes stored in row pairs: ceil(rows / 2)."""
    return (rows + 1) // 2


def scale_shape(rows: int, K: int):
    """Shape of INT4 group scales stored stage-major: [ceil(K/128), rows, 2] fp32 (the scale
    of (row i, group g) at [g // 2, i, g % 2]; an odd group count's last pair padded)."""
    return ((K // GROUP + 1) // 2, int(rows), 2)


def scale_rows(s: torch.Tensor) -> int:
    """Row count of stage-major INT4 group scales."""
    return int(s.shape[1])


def _codes_of(q: torch.Tensor, rows: int, K: int, what: str) -> None:
    if tuple(q.shape) != (pair_rows(rows), K) or q.dtype != torch.uint8:
        raise ValueError("%s: expected uint8 row-pair codes of shape %s, got %s %s"
                         % (what, (pair_rows(rows), K), q.dtype, tuple(q.shape)))


def pack_weights(R: torch.Tensor):
    """Residual fp32 [N, K] -> (qw uint8 [ceil(N/2), K] row pairs, sw fp32 stage-major
    [ceil(K/128), N, 2])."""
    N, K = R.shape
    qw = torch.empty((pair_rows(N), K), dtype=torch.uint8, device=R.device)
    sw = torch.empty(scale_shape(N, K), dtype=torch.float32, device=R.device)
    svdq_pack_weights(R, N, K, qw, sw)
    return qw, sw


def repack_weights(codes: torch.Tensor, scales: torch.Tensor):
    """Row-major two's-complement INT4 codes uint8 [N, K/2] and fp32 scales [N, K/64] ->
    (qw uint8 [ceil(N/2), K], sw fp32 stage-major [ceil(K/128), N, 2])."""
    N, K = codes.shape[0], codes.shape[1] * 2
    qw = torch.empty((pair_rows(N), K), dtype=torch.uint8, device=codes.device)
    sw = torch.empty(scale_shape(N, K), dtype=torch.float32, device=codes.device)
    svdq_repack_weights(codes, scales, N, K, qw, sw)
    return qw, sw


def awq_pack_weights(W: torch.Tensor) -> torch.Tensor:
    """fp32 weight [N, K] -> the W4A16 records (uint8, svdq_awq_packed_bytes(N, K) bytes)."""
    N, K = W.shape
    packed = torch.empty(svdq_awq_packed_bytes(N, K), dtype=torch.uint8, device=W.device)
    svdq_awq_pack_weights(W, N, K, packed)
    return packed


def awq_repack(codes: torch.Tensor, scales: torch.Tensor, zeros: torch.Tensor) -> torch.Tensor:
    """Row-major codes uint8 [N, K/2], scales fp32 [N, K/64], zeros uint8 [N, K/64] -> records."""
    N, K = codes.shape[0], codes.shape[1] * 2
    packed = torch.empty(svdq_awq_packed_bytes(N, K), dtype=torch.uint8, device=codes.device)
    svdq_awq_repack(codes, scales, zeros, N, K, packed)
    return packed


def awq_linear(X: torch.Tensor, packed: torch.Tensor, N: int, bias=None) -> torch.Tensor:
    """W4A16 layer: X bf16 [M, K] -> Y bf16 [M, N] (packed from awq_pack_weights / awq_repack)."""
    M, K = X.shape
    Y = torch.empty((M, N), dtype=torch.bfloat16, device=X.device)
    svdq_awq_w4a16_linear(_bits(X), packed, _bits(bias), M, N, K, _bits(Y))
    return Y


def quantize_act_down(X: torch.Tensor, lam: torch.Tensor, L1: Optional[torch.Tensor]):
    """X bf16 [M, K] -> (qa uint8 [ceil(M/2), K] row pairs, sa fp32 stage-major
    [ceil(K/128), M, 2], xl1 fp32 [M, r] or None)."""
    M, K = X.shape
    r = _rank(L1, 1)
    dev = X.device
    qa = torch.empty((pair_rows(M), K), dtype=torch.uint8, device=dev)
    sa = torch.empty(scale_shape(M, K), dtype=torch.float32, device=dev)
    xl1 = torch.empty((M, r), dtype=torch.float32, device=dev) if r > 0 else None
    ws_bytes = svdq_quantize_act_down_workspace_bytes(M, K, r)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    svdq_quantize_act_down(_bits(X), lam, _bits(L1) if r > 0 else None, M, K, r, qa, sa, xl1,
                           ws, ws_bytes)
    return qa, sa, xl1


def w4a4_lr_gemm(qa, sa, qw, sw, xl1, L2, bias, act: int = ACT_NONE) -> torch.Tensor:
    """The W4A4 GEMM with the low-rank up-projection, bias and act -> Y bf16 [M, N]."""
    M, N, K = scale_rows(sa), scale_rows(sw), qa.shape[1]
    _codes_of(qa, M, K, "qa")
    _codes_of(qw, N, K, "qw")
    r = _rank(L2, 0)
    Y = torch.empty((M, N), dtype=torch.bfloat16, device=qa.device)
    svdq_w4a4_lr_gemm(qa, sa, qw, sw, xl1 if r > 0 else None, _bits(L2) if r > 0 else None,
                      _bits(bias), act, M, N, K, r, _bits(Y))
    return Y


def linear(X, lam, L1, qw, sw, L2, bias, act: int = ACT_NONE,
           workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """The whole layer (svdq_linear) -> Y bf16 [M, N]."""
    M, K = X.shape
    N = scale_rows(sw)
    _codes_of(qw, N, K, "qw")
    r = _rank(L1, 1)
    need = svdq_linear_workspace_bytes(M, K, r)
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=X.device)
    Y = torch.empty((M, N), dtype=torch.bfloat16, device=X.device)
    svdq_linear(_bits(X), lam, _bits(L1) if r > 0 else None, qw, sw,
                _bits(L2) if r > 0 else None, _bits(bias), act, M, N, K, r, _bits(Y),
                workspace, need)
    return Y


def _qkv_out(M, heads, head_dim, seq, device):
    shape = (M // seq, heads, seq, head_dim)
    return tuple(torch.empty(shape, dtype=torch.bfloat16, device=device) for _ in range(3))


def w4a4_lr_gemm_qkv(qa, sa, qw, sw, xl1, L2, bias, heads: int, head_dim: int, seq: int,
                     gamma_q, gamma_k, eps: float, cos_t, sin_t):
    """The GEMM with the fused QKV epilogue -> (Q, K, V) bf16 [M/seq, heads, seq, head_dim]."""
    M, K = scale_rows(sa), qa.shape[1]
    _codes_of(qa, M, K, "qa")
    _codes_of(qw, scale_rows(sw), K, "qw")
    r = _rank(L2, 0)
    Q, Kt, V = _qkv_out(M, heads, head_dim, seq, qa.device)
    epi = qkv_epilogue(heads, head_dim, seq, _bits(gamma_q), _bits(gamma_k), eps, cos_t, sin_t,
                       _bits(Q), _bits(Kt), _bits(V))
    svdq_w4a4_lr_gemm_qkv(qa, sa, qw, sw, xl1 if r > 0 else None, _bits(L2) if r > 0 else None,
                          _bits(bias), M, K, r, epi)
    return Q, Kt, V


def linear_qkv(X, lam, L1, qw, sw, L2, bias, heads: int, head_dim: int, seq: int, gamma_q,
               gamma_k, eps: float, cos_t, sin_t, workspace: Optional[torch.Tensor] = None):
    """The whole fused QKV layer (svdq_linear_qkv) -> (Q, K, V) bf16 [M/seq, heads, seq, D]."""
    M, K = X.shape
    _codes_of(qw, scale_rows(sw), K, "qw")
    r = _rank(L1, 1)
    need = svdq_linear_workspace_bytes(M, K, r)
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=X.device)
    Q, Kt, V = _qkv_out(M, heads, head_dim, seq, X.device)
    epi = qkv_epilogue(heads, head_dim, seq, _bits(gamma_q), _bits(gamma_k), eps, cos_t, sin_t,
                       _bits(Q), _bits(Kt), _bits(V))
    svdq_linear_qkv(_bits(X), lam, _bits(L1) if r > 0 else None, qw, sw,
                    _bits(L2) if r > 0 else None, _bits(bias), M, K, r, epi, workspace, need)
    return Q, Kt, V


def w4a4_lr_gemm_quant_down(qa, sa, qw, sw, xl1, L2, bias, act, lambda_next, L1_next):
    """The GEMM whose output feeds the next layer -> that layer's (qa, sa, xl1)."""
    M, N, K = scale_rows(sa), scale_rows(sw), qa.shape[1]
    _codes_of(qa, M, K, "qa")
    _codes_of(qw, N, K, "qw")
    r = _rank(L2, 0)
    rn = _rank(L1_next, 1)
    dev = qa.device
    qa_n = torch.empty((pair_rows(M), N), dtype=torch.uint8, device=dev)
    sa_n = torch.empty(scale_shape(M, N), dtype=torch.float32, device=dev)
    xl1_n = torch.empty((M, rn), dtype=torch.float32, device=dev) if rn > 0 else None
    need = svdq_w4a4_lr_gemm_quant_down_workspace_bytes(M, N, rn)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    svdq_w4a4_lr_gemm_quant_down(qa, sa, qw, sw, xl1 if r > 0 else None,
                                 _bits(L2) if r > 0 else None, _bits(bias), act, M, N, K, r,
                                 lambda_next, _bits(L1_next) if rn > 0 else None, rn, qa_n, sa_n,
                                 xl1_n, ws, need)
    return qa_n, sa_n, xl1_n


def mlp(X, up: dict, down: dict, act: int = ACT_GELU,
        workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Y = down(act(up(X))) through svdq_mlp; up / down: dicts with lam, L1, qw, sw, L2, bias."""
    M, K = X.shape
    Nh = scale_rows(up["sw"])
    _codes_of(up["qw"], Nh, K, "up qw")
    _codes_of(down["qw"], K, Nh, "down qw")
    ru, rd = _rank(up["L1"], 1), _rank(down["L1"], 1)
    need = svdq_mlp_workspace_bytes(M, K, Nh, ru, rd)
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=X.device)
    Y = torch.empty((M, K), dtype=torch.bfloat16, device=X.device)
    svdq_mlp(_bits(X), up["lam"], _bits(up["L1"]) if ru else None, up["qw"], up["sw"],
             _bits(up["L2"]) if ru else None, _bits(up.get("bias")), down["lam"],
             _bits(down["L1"]) if rd else None, down["qw"], down["sw"],
             _bits(down["L2"]) if rd else None, _bits(down.get("bias")), act, M, K, Nh, ru, rd,
             _bits(Y), workspace, need)
    return Y


def group_sums(qa, sa, qw, sw, M: int, N: int, m0: int, n0: int, tm: int,
               tn: int) -> torch.Tensor:
    """Exact per-group int32 sums of a block (test hook, through the GEMM's own tile code)
    -> int32 [tm, tn, K/64]; qa, qw row-pair codes of M and N rows, sa, sw their scales."""
    K = qa.shape[1]
    _codes_of(qa, M, K, "qa")
    _codes_of(qw, N, K, "qw")
    S = torch.empty((tm, tn, K // GROUP), dtype=torch.int32, device=qa.device)
    svdq_debug_group_sums(qa, sa, qw, sw, M, N, K, m0, n0, tm, tn, S)
    return S


class SVDQLinear:
    """A drop-in W4A4 replacement for one linear layer.

    ``from_parts`` takes the offline artefacts of SVDQuant (smoothing
    factors, low-rank factors, fp32 residual, bias), packs the residual on
    the GPU once, and ``__call__`` runs the fused layer.
    """

    def __init__(self, lam, L1, qw, sw, L2, bias, act: int = ACT_NONE):
        self.lam, self.L1, self.qw, self.sw, self.L2, self.bias, self.act = \
            lam, L1, qw, sw, L2, bias, act
        self._ws = None

    @classmethod
    def from_parts(cls, lam, L1, R, L2, bias=None, act: int = ACT_NONE):
        qw, sw = pack_weights(R)
        return cls(lam, L1, qw, sw, L2, bias, act)

    @property
    def in_features(self) -> int:
        return self.qw.shape[1]

    @property
    def out_features(self) -> int:
        return scale_rows(self.sw)

    def __call__(self, X: torch.Tensor) -> torch.Tensor:
        M, K = X.shape
        need = svdq_linear_workspace_bytes(M, K, _rank(self.L1, 1))
        if self._ws is None or self._ws.numel() < need:
            self._ws = torch.empty(max(need, 1), dtype=torch.uint8, device=X.device)
        return linear(X, self.lam, self.L1, self.qw, self.sw, self.L2, self.bias, self.act,
                      workspace=self._ws)


# ----------------------------------------------------------- MXFP4 variant

def mx_pack_weights(R: torch.Tensor):
    """Residual fp32 [N, K] -> (qw uint8 [ceil(N/2), K] in row pairs,
    sw uint8 E8M0 [K/32, mx_scale_rows(N)])."""
    N, K = R.shape
    qw = torch.empty(((N + 1) // 2, K), dtype=torch.uint8, device=R.device)
    sw = torch.empty((K // MX_BLOCK, mx_scale_rows(N)), dtype=torch.uint8, device=R.device)
    svdq_mx_pack_weights(R, N, K, qw, sw)
    return qw, sw


def mx_quantize_act_down(X: torch.Tensor, lam: torch.Tensor, L1: Optional[torch.Tensor]):
    """X bf16 [M, K] -> (qa uint8 [ceil(M/2), K] in row pairs, sa uint8
    [K/32, mx_scale_rows(M)], xl1 fp32 [M, r] or None)."""
    M, K = X.shape
    r = _rank(L1, 1)
    dev = X.device
    qa = torch.empty(((M + 1) // 2, K), dtype=torch.uint8, device=dev)
    sa = torch.empty((K // MX_BLOCK, mx_scale_rows(M)), dtype=torch.uint8, device=dev)
    xl1 = torch.empty((M, r), dtype=torch.float32, device=dev) if r > 0 else None
    ws_bytes = svdq_quantize_act_down_workspace_bytes(M, K, r)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    svdq_mx_quantize_act_down(_bits(X), lam, _bits(L1) if r > 0 else None, M, K, r, qa, sa, xl1,
                              ws, ws_bytes)
    return qa, sa, xl1


def mx_lr_gemm(qa, sa, qw, sw, xl1, L2, bias, act: int = ACT_NONE, M: Optional[int] = None,
               N: Optional[int] = None) -> torch.Tensor:
    """The MXFP4 GEMM with the low-rank up-projection, bias and act -> Y bf16 [M, N].
    qa / qw hold row pairs ([ceil(rows/2), K]); M and N default to twice the pair
    counts and must be given when odd."""
    K = qa.shape[1]
    M = 2 * qa.shape[0] if M is None else M
    N = 2 * qw.shape[0] if N is None else N
    r = _rank(L2, 0)
    Y = torch.empty((M, N), dtype=torch.bfloat16, device=qa.device)
    svdq_mx_lr_gemm(qa, sa, qw, sw, xl1 if r > 0 else None, _bits(L2) if r > 0 else None,
                    _bits(bias), act, M, N, K, r, _bits(Y))
    return Y


def mx_linear(X, lam, L1, qw, sw, L2, bias, act: int = ACT_NONE,
              workspace: Optional[torch.Tensor] = None, N: Optional[int] = None) -> torch.Tensor:
    """The whole MXFP4 layer (svdq_mx_linear) -> Y bf16 [M, N]; N defaults to twice
    qw's pair count and must be given when odd."""
    M, K = X.shape
    N = 2 * qw.shape[0] if N is None else N
    r = _rank(L1, 1)
    need = svdq_mx_linear_workspace_bytes(M, K, r)
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=X.device)
    Y = torch.empty((M, N), dtype=torch.bfloat16, device=X.device)
    svdq_mx_linear(_bits(X), lam, _bits(L1) if r > 0 else None, qw, sw,
                   _bits(L2) if r > 0 else None, _bits(bias), act, M, N, K, r, _bits(Y),
                   workspace, need)
    return Y
