"""The C ABI: the library loads, exports every declared entry point, and
rejects bad arguments before touching a device (no compute calls here).

The fake pointers below are never dereferenced: every call in this file
fails argument validation, which runs before the device check and before
any launch.
"""
import ctypes
import os
import re
import subprocess

import pytest

import bit_diffusion_transformer_amd as bdt
from bit_diffusion_transformer_amd import _binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "svdq.h")

OK, INVALID, SHAPE, MISALIGNED, WS_SMALL, NODEV, HIPERR = range(7)
A = 0x10000      # 16-byte aligned fake address (never dereferenced)
U = 0x10008      # misaligned fake address


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^[a-z_0-9 ]+\**\s*\**(svdq_\w+)\(", text, re.M)))


@pytest.fixture(scope="module")
def lib():
    return _binding.load_library()


def test_every_declared_symbol_is_exported(lib):
    decl = declared_functions()
    assert len(decl) == 28, decl
    assert sorted(_binding.EXPORTS) == decl
    for name in decl:
        assert hasattr(lib, name), name


def test_version_and_status_strings(lib):
    assert bdt.svdq_abi_version() == 4
    assert bdt.svdq_status_string(0) == "ok"
    assert bdt.svdq_status_string(MISALIGNED) == "misaligned pointer"
    assert bdt.svdq_status_string(99) == "unknown status"


def test_workspace_sizes(lib):
    K, r, M = 3072, 32, 4608
    down = lib.svdq_quantize_act_down_workspace_bytes(M, K, r)
    # chunks of 4 groups for r <= 64 at up to 64 groups, 8 beyond, 2 for r > 64 or at most
    # 512 tokens (r <= 32); a single chunk needs no partial sums
    assert down == 12 * M * r * 4                 # twelve chunks of 4 groups; 256-aligned here
    assert lib.svdq_quantize_act_down_workspace_bytes(M, K, 0) == 0
    assert lib.svdq_quantize_act_down_workspace_bytes(M, 256, 32) == 0     # one chunk
    assert lib.svdq_quantize_act_down_workspace_bytes(M, 512, 32) == 2 * M * 32 * 4
    assert lib.svdq_quantize_act_down_workspace_bytes(M, 512, 128) == 4 * M * 128 * 4
    assert lib.svdq_quantize_act_down_workspace_bytes(M, 12288, 32) == 24 * M * 32 * 4
    assert lib.svdq_quantize_act_down_workspace_bytes(M, 12288, 64) == 48 * M * 64 * 4
    assert lib.svdq_quantize_act_down_workspace_bytes(256, K, 32) == 24 * 256 * 32 * 4
    assert lib.svdq_quantize_act_down_workspace_bytes(256, 128, 32) == 0  # one chunk of 2
    assert lib.svdq_quantize_act_down_workspace_bytes(0, K, r) == 0
    lin = lib.svdq_linear_workspace_bytes(M, K, r)
    assert lin == M * K // 2 + M * (K // 64) * 4 + M * r * 4 + down
    assert lib.svdq_linear_workspace_bytes(-1, K, r) == 0


P = ctypes.c_void_p


def _down(lib, X=A, lam=A, L1=A, M=16, K=1024, r=16, qa=A, sa=A, xl1=A, ws=A, ws_bytes=1 << 20):
    return lib.svdq_quantize_act_down(P(X), P(lam), P(L1), M, K, r, P(qa), P(sa), P(xl1),
                                      P(ws), ws_bytes, None)


def _gemm(lib, qa=A, sa=A, qw=A, sw=A, xl1=A, L2=A, bias=A, act=0, M=16, N=64, K=128, r=16, Y=A):
    return lib.svdq_w4a4_lr_gemm(P(qa), P(sa), P(qw), P(sw), P(xl1), P(L2), P(bias), act,
                                 M, N, K, r, P(Y), None)


def _lin(lib, X=A, lam=A, L1=A, qw=A, sw=A, L2=A, bias=A, act=0, M=16, N=64, K=128, r=16, Y=A,
         ws=A, ws_bytes=1 << 30):
    return lib.svdq_linear(P(X), P(lam), P(L1), P(qw), P(sw), P(L2), P(bias), act, M, N, K, r,
                           P(Y), P(ws), ws_bytes, None)


@pytest.mark.parametrize("kw,code", [
    (dict(M=-1), INVALID),
    (dict(K=100), SHAPE), (dict(K=0), SHAPE), (dict(K=32), SHAPE),
    (dict(r=8), SHAPE), (dict(r=-16), SHAPE), (dict(r=144), SHAPE),
    (dict(X=0), INVALID), (dict(lam=0), INVALID), (dict(qa=0), INVALID), (dict(sa=0), INVALID),
    (dict(L1=0), INVALID), (dict(xl1=0), INVALID),
    (dict(r=0), INVALID),                      # L1/xl1 given although r == 0
    (dict(X=U), MISALIGNED), (dict(sa=U), MISALIGNED), (dict(L1=U), MISALIGNED),
    (dict(ws_bytes=16), WS_SMALL), (dict(ws=0), INVALID),
    (dict(K=(1 << 20) + 64), SHAPE), (dict(M=(1 << 28) + 1), SHAPE),   # past the size limits
])
def test_quantize_act_down_rejects(lib, kw, code):
    assert _down(lib, **kw) == code
    assert lib.svdq_last_error()


@pytest.mark.parametrize("kw,code", [
    (dict(M=-2), INVALID), (dict(act=2), INVALID), (dict(act=-1), INVALID),
    (dict(N=60), SHAPE), (dict(N=0), SHAPE), (dict(K=96), SHAPE), (dict(r=24), SHAPE),
    (dict(N=(1 << 28) + 8), SHAPE), (dict(K=(1 << 20) + 64), SHAPE), (dict(M=(1 << 28) + 1), SHAPE),
    (dict(qa=0), INVALID), (dict(sw=0), INVALID), (dict(Y=0), INVALID),
    (dict(xl1=0), INVALID), (dict(L2=0), INVALID), (dict(r=0), INVALID),
    (dict(qw=U), MISALIGNED), (dict(Y=U), MISALIGNED), (dict(bias=U), MISALIGNED),
])
def test_gemm_rejects(lib, kw, code):
    assert _gemm(lib, **kw) == code


@pytest.mark.parametrize("kw,code", [
    (dict(M=-1), INVALID), (dict(act=7), INVALID), (dict(N=12), SHAPE), (dict(K=65), SHAPE),
    (dict(r=17), SHAPE), (dict(X=0), INVALID), (dict(qw=0), INVALID), (dict(L2=0), INVALID),
    (dict(ws_bytes=1000), WS_SMALL), (dict(ws=0), INVALID), (dict(lam=U), MISALIGNED),
])
def test_linear_rejects(lib, kw, code):
    assert _lin(lib, **kw) == code


# Shapes within the row and K limits whose launches would exceed the 2^32 - 1 work-items of a
# dispatch grid: rejected as unsupported before any device call (no GPU needed here).
@pytest.mark.parametrize("call", [
    lambda lib: _down(lib, M=1 << 28, K=1 << 20, r=16),          # the activation step
    lambda lib: _down(lib, M=1 << 28, K=128, r=128),             # its partial-sum reduce
    lambda lib: _gemm(lib, M=1 << 28, N=1 << 16, K=128),         # the GEMM
    lambda lib: _lin(lib, M=1 << 28, N=1 << 16, K=128),
    lambda lib: lib.svdq_repack_weights(P(A), P(A), 1 << 28, 1 << 20, P(A), P(A), None),
    lambda lib: lib.svdq_awq_pack_weights(P(A), 1 << 28, 1 << 20, P(A), None),
])
def test_oversized_launches_rejected(lib, call):
    assert call(lib) == SHAPE
    assert b"work-items" in lib.svdq_last_error()


def test_pack_and_debug_reject(lib):
    assert lib.svdq_pack_weights(P(A), -1, 128, P(A), P(A), None) == INVALID
    assert lib.svdq_pack_weights(P(A), 8, 100, P(A), P(A), None) == SHAPE
    assert lib.svdq_pack_weights(P(0), 8, 128, P(A), P(A), None) == INVALID
    assert lib.svdq_pack_weights(P(A), 8, 128, P(U), P(A), None) == MISALIGNED
    rp = lib.svdq_repack_weights
    assert rp(P(A), P(A), -1, 128, P(A), P(A), None) == INVALID
    assert rp(P(A), P(A), 8, 96, P(A), P(A), None) == SHAPE
    assert rp(P(0), P(A), 8, 128, P(A), P(A), None) == INVALID
    assert rp(P(A), P(0), 8, 128, P(A), P(A), None) == INVALID
    assert rp(P(A), P(A), 8, 128, P(U), P(A), None) == MISALIGNED
    assert rp(P(A), P(A), 8, 128, P(A), P(U), None) == MISALIGNED
    assert lib.svdq_debug_group_sums(P(A), P(A), P(A), P(A), 16, 16, 128, 8, 0, 16, 16, P(A), None) == INVALID
    assert lib.svdq_debug_group_sums(P(A), P(A), P(A), P(A), 16, 16, 100, 0, 0, 16, 16, P(A), None) == SHAPE
    assert lib.svdq_debug_group_sums(P(A), P(0), P(A), P(A), 16, 16, 128, 0, 0, 16, 16, P(A), None) == INVALID
    assert lib.svdq_debug_group_sums(P(A), P(A), P(A), P(U), 16, 16, 128, 0, 0, 16, 16, P(A), None) == MISALIGNED
    ap = lib.svdq_awq_pack_weights
    assert ap(P(A), -1, 128, P(A), None) == INVALID
    assert ap(P(A), 8, 96, P(A), None) == SHAPE
    assert ap(P(A), 12, 128, P(A), None) == SHAPE
    assert ap(P(A), 8, 128, P(0), None) == INVALID
    assert ap(P(U), 8, 128, P(A), None) == MISALIGNED
    ar = lib.svdq_awq_repack
    assert ar(P(A), P(A), P(A), -1, 128, P(A), None) == INVALID
    assert ar(P(A), P(A), P(A), 8, 100, P(A), None) == SHAPE
    assert ar(P(0), P(A), P(A), 8, 128, P(A), None) == INVALID
    assert ar(P(A), P(A), P(0), 8, 128, P(A), None) == INVALID
    assert ar(P(A), P(U), P(A), 8, 128, P(A), None) == MISALIGNED
    aw = lib.svdq_awq_w4a16_linear
    assert aw(P(A), P(A), P(A), -1, 64, 128, P(A), None) == INVALID
    assert aw(P(A), P(A), P(A), 2, 60, 128, P(A), None) == SHAPE
    assert aw(P(A), P(A), P(A), 2, 64, 100, P(A), None) == SHAPE
    assert aw(P(0), P(A), P(A), 2, 64, 128, P(A), None) == INVALID
    assert aw(P(A), P(0), P(A), 2, 64, 128, P(A), None) == INVALID
    assert aw(P(A), P(A), P(U), 2, 64, 128, P(A), None) == MISALIGNED
    assert aw(P(A), P(A), P(A), 2, 64, 128, P(U), None) == MISALIGNED
    assert lib.svdq_debug_set_tile_policy(5) == INVALID
    assert lib.svdq_debug_set_tile_policy(-1) == INVALID


def test_noalloc_rejects(lib):
    nl = lib.svdq_linear_noalloc

    def call(X=A, lam=A, L1=A, qw=A, sw=A, L2=A, bias=0, act=0, M=16, N=16, K=128, r=16, Y=A):
        return nl(P(X), P(lam), P(L1), P(qw), P(sw), P(L2), P(bias), act, M, N, K, r, P(Y), None)

    assert call(M=-1) == INVALID
    assert call(act=3) == INVALID
    assert call(N=12) == SHAPE
    assert call(r=17) == SHAPE
    assert call(X=0) == INVALID
    assert call(L2=0) == INVALID
    assert call(Y=U) == MISALIGNED
    assert call(M=0, X=0, lam=0, L1=0, qw=0, sw=0, L2=0, Y=0) == OK
    # more intermediates than the library's static scratch holds: refused before any launch
    big_m = 1 << 20
    assert lib.svdq_linear_workspace_bytes(big_m, 3072, 32) > _binding.NOALLOC_SCRATCH_BYTES
    assert call(M=big_m, K=3072, r=32, N=3072) == WS_SMALL
    assert b"scratch" in lib.svdq_last_error()


def test_tile_policy_values_accepted(lib):
    # host-side setting only (no launch); restored to the default
    for pol in (bdt.TILES_FULL, bdt.TILES_QUARTER, bdt.TILES_KSPLIT, bdt.TILES_KSPLIT_QUARTER,
                bdt.TILES_AUTO):
        assert lib.svdq_debug_set_tile_policy(pol) == OK


def test_empty_inputs_are_noops(lib):
    # M == 0 (or N == 0 for packing) succeeds without touching any pointer.
    assert _down(lib, X=0, lam=0, L1=0, qa=0, sa=0, xl1=0, ws=0, M=0) == OK
    assert _gemm(lib, qa=0, sa=0, qw=0, sw=0, xl1=0, L2=0, bias=0, Y=0, M=0) == OK
    assert _lin(lib, X=0, lam=0, L1=0, qw=0, sw=0, L2=0, bias=0, Y=0, ws=0, M=0) == OK
    assert lib.svdq_pack_weights(P(0), 0, 128, P(0), P(0), None) == OK
    assert lib.svdq_repack_weights(P(0), P(0), 0, 128, P(0), P(0), None) == OK
    assert lib.svdq_debug_group_sums(P(0), P(0), P(0), P(0), 16, 16, 128, 0, 0, 0, 5, P(0), None) == OK
    assert lib.svdq_awq_pack_weights(P(0), 0, 128, P(0), None) == OK
    assert lib.svdq_awq_repack(P(0), P(0), P(0), 0, 128, P(0), None) == OK
    assert lib.svdq_awq_w4a16_linear(P(0), P(0), P(0), 0, 64, 128, P(0), None) == OK


def test_awq_packed_bytes(lib):
    # (N, K) -> ceil(N/16) * ceil(K/256) records of 2368 bytes; 0 for bad shapes
    assert lib.svdq_awq_packed_bytes(18432, 3072) == 1152 * 12 * 2368
    assert lib.svdq_awq_packed_bytes(8, 64) == 2368
    assert lib.svdq_awq_packed_bytes(264, 320) == 17 * 2 * 2368
    assert lib.svdq_awq_packed_bytes(0, 128) == 0
    assert lib.svdq_awq_packed_bytes(8, 100) == 0
    assert lib.svdq_awq_packed_bytes(-8, 128) == 0


def test_refuses_without_a_gfx950_device(lib):
    torch = pytest.importorskip("torch")
    if torch.cuda.is_available():
        pytest.skip("a GPU is present; the device check is exercised by the GPU tests")
    assert _gemm(lib) == NODEV
    assert "device" in lib.svdq_last_error().decode()


def _epi(**kw):
    e = dict(heads=2, head_dim=128, seq=4, gamma_q=A, gamma_k=A, eps=1e-6, cos_t=A, sin_t=A,
             q=A, k=A, v=A)
    e.update(kw)
    return _binding.QkvEpilogue(**e)


def _gq(lib, epi, M=8, K=128, r=16, **kw):
    a = dict(qa=A, sa=A, qw=A, sw=A, xl1=A, L2=A, bias=A)
    a.update(kw)
    e = None if epi is None else ctypes.byref(epi)
    return lib.svdq_w4a4_lr_gemm_qkv(P(a["qa"]), P(a["sa"]), P(a["qw"]), P(a["sw"]),
                                     P(a["xl1"]), P(a["L2"]), P(a["bias"]), M, K, r, e, None)


def _lq(lib, epi, M=8, K=128, r=16, ws_bytes=1 << 30, **kw):
    a = dict(X=A, lam=A, L1=A, qw=A, sw=A, L2=A, bias=A, ws=A)
    a.update(kw)
    return lib.svdq_linear_qkv(P(a["X"]), P(a["lam"]), P(a["L1"]), P(a["qw"]), P(a["sw"]),
                               P(a["L2"]), P(a["bias"]), M, K, r, ctypes.byref(epi), P(a["ws"]),
                               ws_bytes, None)


@pytest.mark.parametrize("epi_kw,code", [
    (dict(head_dim=96), SHAPE), (dict(heads=1, head_dim=64), SHAPE), (dict(heads=0), INVALID),
    (dict(seq=3), SHAPE), (dict(seq=0), INVALID), (dict(eps=-1.0), INVALID),
    (dict(eps=float("nan")), INVALID), (dict(eps=float("inf")), INVALID),
    (dict(gamma_q=None), INVALID), (dict(cos_t=U), MISALIGNED), (dict(v=U), MISALIGNED),
    (dict(k=None), INVALID),
])
def test_qkv_rejects(lib, epi_kw, code):
    assert _gq(lib, _epi(**epi_kw)) == code
    assert _lq(lib, _epi(**epi_kw)) == code


def test_qkv_rejects_operands(lib):
    assert _gq(lib, None) == INVALID
    assert _gq(lib, _epi(), K=100) == SHAPE
    assert _gq(lib, _epi(), r=17) == SHAPE
    assert _gq(lib, _epi(), qa=0) == INVALID
    assert _gq(lib, _epi(), bias=U) == MISALIGNED
    assert _gq(lib, _epi(), r=0) == INVALID          # xl1 / L2 must be NULL at r == 0
    assert _lq(lib, _epi(), ws_bytes=10) == WS_SMALL
    assert _lq(lib, _epi(), X=0) == INVALID
    # M == 0: no-op; the epilogue's shape rules still apply
    assert _gq(lib, _epi(q=0, k=0, v=0, gamma_q=0, gamma_k=0, cos_t=0, sin_t=0), M=0,
               qa=0, sa=0, qw=0, sw=0, xl1=0, L2=0, bias=0) == OK
    assert _gq(lib, _epi(head_dim=96), M=0) == SHAPE


def test_qkv_struct_layout_matches_header(tmp_path):
    """The ctypes mirror of svdq_qkv_epilogue has the C compiler's size and offsets."""
    src = tmp_path / "layout.c"
    src.write_text('#include <stdio.h>\n#include <stddef.h>\n#include "svdq.h"\n'
                   "int main(void) { printf(\"%zu\", sizeof(svdq_qkv_epilogue));\n"
                   + "".join('printf(" %%zu", offsetof(svdq_qkv_epilogue, %s));\n' % f
                             for f, _ in _binding.QkvEpilogue._fields_)
                   + "return 0; }\n")
    exe = tmp_path / "layout"
    subprocess.check_call(["gcc", "-I", os.path.dirname(HEADER), str(src), "-o", str(exe)])
    got = [int(v) for v in subprocess.check_output([str(exe)]).split()]
    want = [ctypes.sizeof(_binding.QkvEpilogue)] + [getattr(_binding.QkvEpilogue, f).offset
                                                    for f, _ in _binding.QkvEpilogue._fields_]
    assert got == want


def _gqd(lib, M=8, N=256, K=128, r=16, rn=32, ws_bytes=1 << 30, act=1, **kw):
    a = dict(qa=A, sa=A, qw=A, sw=A, xl1=A, L2=A, bias=A, lam=A, L1n=A, qan=A, san=A, xl1n=A, ws=A)
    a.update(kw)
    return lib.svdq_w4a4_lr_gemm_quant_down(
        P(a["qa"]), P(a["sa"]), P(a["qw"]), P(a["sw"]), P(a["xl1"]), P(a["L2"]), P(a["bias"]), act,
        M, N, K, r, P(a["lam"]), P(a["L1n"]), rn, P(a["qan"]), P(a["san"]), P(a["xl1n"]),
        P(a["ws"]), ws_bytes, None)


def _mlp(lib, M=8, K=128, Nh=256, ru=16, rd=32, ws_bytes=1 << 30, act=1, **kw):
    a = dict(X=A, lu=A, L1u=A, qwu=A, swu=A, L2u=A, bu=A, ld=A, L1d=A, qwd=A, swd=A, L2d=A, bd=A,
             Y=A, ws=A)
    a.update(kw)
    return lib.svdq_mlp(P(a["X"]), P(a["lu"]), P(a["L1u"]), P(a["qwu"]), P(a["swu"]), P(a["L2u"]),
                        P(a["bu"]), P(a["ld"]), P(a["L1d"]), P(a["qwd"]), P(a["swd"]), P(a["L2d"]),
                        P(a["bd"]), act, M, K, Nh, ru, rd, P(a["Y"]), P(a["ws"]), ws_bytes, None)


@pytest.mark.parametrize("kw,code", [
    (dict(N=192), SHAPE), (dict(rn=48), SHAPE), (dict(rn=8), SHAPE), (dict(act=7), INVALID),
    (dict(K=100), SHAPE), (dict(lam=0), INVALID), (dict(san=0), INVALID), (dict(qan=U), MISALIGNED),
    (dict(L1n=0), INVALID), (dict(rn=0), INVALID), (dict(xl1n=U), MISALIGNED),
    (dict(ws_bytes=16), WS_SMALL), (dict(ws=0), INVALID), (dict(qa=0), INVALID),
])
def test_gemm_quant_down_rejects(lib, kw, code):
    assert _gqd(lib, **kw) == code


@pytest.mark.parametrize("kw,code", [
    (dict(Nh=192), SHAPE), (dict(rd=48), SHAPE), (dict(ru=17), SHAPE), (dict(K=100), SHAPE),
    (dict(K=64 * 3 + 4), SHAPE), (dict(act=3), INVALID), (dict(X=0), INVALID),
    (dict(ld=0), INVALID), (dict(L1d=0), INVALID), (dict(L2u=0), INVALID), (dict(Y=U), MISALIGNED),
    (dict(bd=U), MISALIGNED), (dict(ws_bytes=16), WS_SMALL), (dict(ws=0), INVALID),
])
def test_mlp_rejects(lib, kw, code):
    assert _mlp(lib, **kw) == code


def test_mlp_empty_and_workspace_sizes(lib):
    assert _gqd(lib, M=0, qa=0, sa=0, qw=0, sw=0, xl1=0, L2=0, bias=0, lam=0, L1n=0, qan=0, san=0,
                xl1n=0, ws=0, ws_bytes=0) == OK
    assert _mlp(lib, M=0, X=0, lu=0, L1u=0, qwu=0, swu=0, L2u=0, bu=0, ld=0, L1d=0, qwd=0, swd=0,
                L2d=0, bd=0, Y=0, ws=0, ws_bytes=0) == OK
    # partial down-projections: [N/128][M][r_next] fp32, 256-byte aligned
    assert lib.svdq_w4a4_lr_gemm_quant_down_workspace_bytes(4608, 12288, 32) == 96 * 4608 * 32 * 4
    assert lib.svdq_w4a4_lr_gemm_quant_down_workspace_bytes(5, 256, 16) == 768
    assert lib.svdq_w4a4_lr_gemm_quant_down_workspace_bytes(5, 256, 0) == 0
    lin = lib.svdq_linear_workspace_bytes(100, 128, 16)
    mlp = lib.svdq_mlp_workspace_bytes(100, 128, 256, 16, 32)
    # up-layer workspace + hidden codes, scales, xl1 and partials
    assert mlp == lin + 12800 + 1792 + 12800 + 25600


# ---------------------------------------------------------------- MXFP4 variant

def _mxd(lib, X=A, lam=A, L1=A, M=16, K=1024, r=16, qa=A, sa=A, xl1=A, ws=A, ws_bytes=1 << 20):
    return lib.svdq_mx_quantize_act_down(P(X), P(lam), P(L1), M, K, r, P(qa), P(sa), P(xl1),
                                         P(ws), ws_bytes, None)


def _mxg(lib, qa=A, sa=A, qw=A, sw=A, xl1=A, L2=A, bias=A, act=0, M=16, N=64, K=128, r=16, Y=A):
    return lib.svdq_mx_lr_gemm(P(qa), P(sa), P(qw), P(sw), P(xl1), P(L2), P(bias), act,
                               M, N, K, r, P(Y), None)


def _mxl(lib, X=A, lam=A, L1=A, qw=A, sw=A, L2=A, bias=A, act=0, M=16, N=64, K=128, r=16, Y=A,
         ws=A, ws_bytes=1 << 30):
    return lib.svdq_mx_linear(P(X), P(lam), P(L1), P(qw), P(sw), P(L2), P(bias), act, M, N, K,
                              r, P(Y), P(ws), ws_bytes, None)


@pytest.mark.parametrize("call,kw,code", [
    # K must be a positive multiple of 128 (whole stages of two 64-value groups)
    (_mxd, dict(K=64), SHAPE), (_mxd, dict(K=192), SHAPE), (_mxd, dict(K=0), SHAPE),
    (_mxg, dict(K=64), SHAPE), (_mxg, dict(K=320), SHAPE), (_mxl, dict(K=64), SHAPE),
    (_mxd, dict(M=-1), INVALID), (_mxd, dict(r=8), SHAPE), (_mxd, dict(sa=0), INVALID),
    (_mxd, dict(sa=U), MISALIGNED), (_mxd, dict(ws_bytes=16), WS_SMALL),
    (_mxd, dict(r=0), INVALID),
    (_mxg, dict(act=2), INVALID), (_mxg, dict(N=60), SHAPE), (_mxg, dict(sw=0), INVALID),
    (_mxg, dict(sa=U), MISALIGNED), (_mxg, dict(L2=0), INVALID), (_mxg, dict(r=0), INVALID),
    (_mxl, dict(M=-1), INVALID), (_mxl, dict(N=12), SHAPE), (_mxl, dict(r=17), SHAPE),
    (_mxl, dict(sw=0), INVALID), (_mxl, dict(ws_bytes=1000), WS_SMALL),
    (_mxl, dict(lam=U), MISALIGNED),
])
def test_mx_rejects(lib, call, kw, code):
    assert call(lib, **kw) == code
    assert lib.svdq_last_error()


def test_mx_pack_rejects_empty_and_sizes(lib):
    mp = lib.svdq_mx_pack_weights
    assert mp(P(A), -1, 128, P(A), P(A), None) == INVALID
    assert mp(P(A), 8, 64, P(A), P(A), None) == SHAPE
    assert mp(P(0), 8, 128, P(A), P(A), None) == INVALID
    assert mp(P(A), 8, 128, P(A), P(U), None) == MISALIGNED
    assert mp(P(0), 0, 128, P(0), P(0), None) == OK
    assert _mxd(lib, X=0, lam=0, L1=0, qa=0, sa=0, xl1=0, ws=0, M=0) == OK
    assert _mxg(lib, qa=0, sa=0, qw=0, sw=0, xl1=0, L2=0, bias=0, Y=0, M=0) == OK
    assert _mxl(lib, X=0, lam=0, L1=0, qw=0, sw=0, L2=0, bias=0, Y=0, ws=0, M=0) == OK
    # codes, E8M0 bytes [M, K/32], xl1, down-projection partials (each 256-aligned)
    M, K, r = 4608, 3072, 32
    down = lib.svdq_quantize_act_down_workspace_bytes(M, K, r)
    assert lib.svdq_mx_linear_workspace_bytes(M, K, r) == M * K // 2 + M * K // 32 + M * r * 4 + down
    assert lib.svdq_mx_linear_workspace_bytes(-1, K, r) == 0
    # block-major scale bytes [K/32][M rounded up to 16]: 4 x 112 -> 512 after alignment
    assert lib.svdq_mx_linear_workspace_bytes(100, 128, 16) == 6400 + 512 + 6400
