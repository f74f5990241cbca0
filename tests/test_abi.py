"""C-ABI contract tests that need no GPU: the library loads, exports every
symbol include/w4a4.h declares, and rejects bad arguments on the host before
anything is launched (fake device pointers are never dereferenced)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "w4a4.h")

OK, INVALID, KMUL, MISALIGNED, DTYPE, WS, HIP = range(7)


@pytest.fixture(scope="module")
def L():
    from hadamard_rotated_w4a4_amd import _lib
    return _lib.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(w4a4_[a-z0-9_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported(L):
    names = declared_functions()
    assert len(names) >= 10
    for name in names:
        assert hasattr(L, name), name


def test_status_strings(L):
    for code, name in enumerate(["W4A4_OK", "W4A4_ERR_INVALID_VALUE", "W4A4_ERR_K_NOT_MULTIPLE_OF_32",
                                 "W4A4_ERR_MISALIGNED", "W4A4_ERR_UNSUPPORTED_DTYPE",
                                 "W4A4_ERR_WORKSPACE_TOO_SMALL", "W4A4_ERR_HIP"]):
        assert L.w4a4_status_string(code).decode() == name
    assert L.w4a4_last_hip_error().decode() == ""


def test_size_queries(L):
    assert L.w4a4_q4_0_bytes(17408, 5120) == 17408 * 160 * 18
    # packed = 32-column tiles x blocks padded to 8 x 1 KB (matrix-core
    # records), then 32-column tiles x groups of 4 blocks x 2304 B (streaming)
    assert L.w4a4_packed_weight_bytes(17408, 5120) == 544 * 160 * 1024 + 544 * 40 * 2304
    assert L.w4a4_packed_weight_bytes(33, 64) == 2 * 8 * 1024 + 2 * 1 * 2304  # n padded to 64
    assert L.w4a4_packed_weight_bytes(10, 33) == 0
    # offsets and tile counts (129 int32 each, 256-byte rounded), perm (8192 int32)
    assert L.w4a4_gemm_id_workspace_bytes(128, 1024, 8) == 2 * 768 + 32768
    assert L.w4a4_gemm_id_workspace_bytes(-1, 1, 1) == 0


A = 0x10000000          # fake, aligned device addresses: never dereferenced
ODD = 0x10000001


def P(x):
    return ctypes.c_void_p(x)


def test_gemm_validation(L):
    g = L.w4a4_gemm
    assert g(P(A), P(A), P(A), P(A), 64, 64, 33, 64, None, 0, None) == KMUL
    assert g(P(A), P(A), P(A), P(A), -1, 64, 64, 64, None, 0, None) == INVALID
    assert g(P(A), P(A), P(A), P(A), 8, -1, 64, 64, None, 0, None) == INVALID
    assert g(P(A), P(A), P(A), P(A), 8, 64, 64, 63, None, 0, None) == INVALID  # ldy < n
    assert g(None, P(A), P(A), P(A), 8, 64, 64, 64, None, 0, None) == INVALID
    assert g(P(A), None, P(A), P(A), 8, 64, 64, 64, None, 0, None) == INVALID
    assert g(P(A), P(A), None, P(A), 8, 64, 64, 64, None, 0, None) == INVALID
    assert g(P(A), P(A), P(A), None, 8, 64, 64, 64, None, 0, None) == INVALID
    assert g(P(A), P(A + 8), P(A), P(A), 8, 64, 64, 64, None, 0, None) == MISALIGNED  # codes need 16 B
    assert g(P(A + 8), P(A), P(A), P(A), 8, 64, 64, 64, None, 0, None) == MISALIGNED  # packed needs 16 B
    assert g(P(A), P(A), P(ODD), P(A), 8, 64, 64, 64, None, 0, None) == MISALIGNED
    assert g(P(A), P(A), P(A), P(A + 2), 8, 64, 64, 64, None, 0, None) == MISALIGNED
    # nothing to do: no launch, no pointer needed
    assert g(None, None, None, None, 0, 64, 64, 64, None, 0, None) == OK
    assert g(None, None, None, None, 8, 0, 64, 0, None, 0, None) == OK
    # m > 16 needs the workspace the size query names, 256-byte aligned
    need = L.w4a4_gemm_workspace_bytes(64, 64, 64)
    assert need == 2 * 8 * 1024  # 32-row tiles x blocks padded to 8 x 1 KB records
    assert L.w4a4_gemm_workspace_bytes(16, 64, 64) == 0
    # m <= 16 with K split (n = 1024: 32 column tiles, K = 5120: 4 splits):
    # one 8-byte arrival word per tile (256 bytes), then the partial sums
    assert L.w4a4_gemm_workspace_bytes(16, 1024, 5120) == 256 + 4 * 16 * 1024 * 4
    assert L.w4a4_gemm_workspace_bytes(3, 1024, 5120) == 256 + 4 * 3 * 1024 * 4
    # n = 5120 (160 tiles), K = 17408 (136 records): 4 splits; 1280 bytes of words
    assert L.w4a4_gemm_workspace_bytes(16, 5120, 17408) == 1280 + 4 * 16 * 5120 * 4
    # K in (5120, 8192] runs 16 waves per workgroup at a quarter of the
    # target: n = 5120 whole K, n = 1024 (32 tiles) in 4 splits
    assert L.w4a4_gemm_workspace_bytes(16, 5120, 6144) == 0
    assert L.w4a4_gemm_workspace_bytes(16, 1024, 6144) == 256 + 4 * 16 * 1024 * 4
    # the fused launch takes the same plan: its own sync words and flags only
    assert L.w4a4_rotate_quantize_gemm_workspace_bytes(16, 5120, 6144) == 256 + 256
    assert L.w4a4_gemm_workspace_bytes(17, 64, 33) == 0
    assert g(P(A), P(A), P(A), P(A), 64, 64, 64, 64, None, need, None) == INVALID
    assert g(P(A), P(A), P(A), P(A), 64, 64, 64, 64, P(A + 16), need, None) == MISALIGNED
    assert g(P(A), P(A), P(A), P(A), 64, 64, 64, 64, P(A), need - 1, None) == WS


def test_a8_validation(L):
    q = L.w4a4_rotate_quantize_act8
    assert q(P(A), 0, 4, 40, 64, P(A), P(A), None) == KMUL
    assert q(P(A), 5, 4, 64, 64, P(A), P(A), None) == DTYPE
    assert q(P(A), 0, 4, 64, 32, P(A), P(A), None) == INVALID  # ldx < k
    assert q(P(A), 0, 4, 64, 64, P(A + 8), P(A), None) == MISALIGNED
    assert q(None, 0, 0, 64, 64, None, None, None) == OK
    g = L.w4a4_gemm_a8
    assert g(P(A), P(A), P(A), P(A), 8, 64, 40, 64, None, 0, None) == KMUL
    assert g(P(A), P(A + 8), P(A), P(A), 8, 64, 64, 64, None, 0, None) == MISALIGNED
    assert g(P(A), P(A), P(A), P(A), 8, 64, 64, 32, None, 0, None) == INVALID  # ldy < n
    assert g(None, None, None, None, 0, 64, 64, 64, None, 0, None) == OK
    # m <= 16 with K split needs the partial-sum workspace; m > 16 the codes'
    # two FP6 planes (row tiles x 2 planes x 160 blocks x 1 KB)
    need = L.w4a4_gemm_a8_workspace_bytes(16, 1024, 5120)
    assert need > 0 and need % 256 == 0
    assert L.w4a4_gemm_a8_workspace_bytes(64, 1024, 5120) == 2 * L.w4a4_act_operand_bytes(64, 5120) == 2 * 2 * 160 * 1024
    assert L.w4a4_gemm_a8_workspace_bytes(65, 1024, 5120) == 2 * 3 * 160 * 1024
    assert L.w4a4_gemm_a8_workspace_bytes(16, 64, 33) == 0
    assert g(P(A), P(A), P(A), P(A), 16, 1024, 5120, 1024, None, 0, None) == INVALID
    assert g(P(A), P(A), P(A), P(A), 16, 1024, 5120, 1024, P(A), need - 1, None) == WS


def test_a8_prepared_validation(L):
    # two planes of the W4A4 operand's shape: (row tiles) x 2 x 160 blocks x 1 KB
    assert L.w4a4_act8_operand_bytes(64, 5120) == 2 * L.w4a4_act_operand_bytes(64, 5120) == 2 * 2 * 160 * 1024
    assert L.w4a4_act8_operand_bytes(1, 64) == 2 * 8 * 1024
    assert L.w4a4_act8_operand_bytes(8, 33) == 0
    pb = L.w4a4_act8_operand_bytes(4, 64)
    q = L.w4a4_rotate_quantize_prepare8
    assert q(P(A), 0, 4, 40, 64, P(A), P(A), P(A), pb, None) == KMUL
    assert q(P(A), 5, 4, 64, 64, P(A), P(A), P(A), pb, None) == DTYPE
    assert q(P(A), 0, 4, 64, 64, P(A), P(A), None, pb, None) == INVALID
    assert q(P(A), 0, 4, 64, 64, P(A), P(A), P(A + 16), pb, None) == MISALIGNED
    assert q(P(A), 0, 4, 64, 64, P(A), P(A), P(A), pb - 1, None) == WS
    # the W4A4 operand's size is too small for the two planes
    assert q(P(A), 0, 4, 64, 64, P(A), P(A), P(A), L.w4a4_act_operand_bytes(4, 64), None) == WS
    assert q(None, 0, 0, 64, 64, None, None, None, 0, None) == OK
    g = L.w4a4_gemm_a8_prepared
    assert g(P(A), P(A), P(A), 8, 64, 40, 64, None) == KMUL
    assert g(P(A), P(A), P(A), 8, 64, 64, 32, None) == INVALID  # ldy < n
    assert g(P(A), None, P(A), 8, 64, 64, 64, None) == INVALID
    assert g(P(A), P(A + 16), P(A), 8, 64, 64, 64, None) == MISALIGNED
    assert g(P(A), P(A), P(A + 2), 8, 64, 64, 64, None) == MISALIGNED
    assert g(None, None, None, 0, 64, 64, 64, None) == OK


def test_prepared_gemm_validation(L):
    pb = L.w4a4_act_operand_bytes(64, 64)
    assert pb == 2 * 8 * 1024
    assert L.w4a4_act_operand_bytes(64, 33) == 0
    prep = L.w4a4_gemm_prepare_act
    assert prep(P(A), P(A), 64, 33, P(A), pb, None) == KMUL
    assert prep(P(A), P(A), -1, 64, P(A), pb, None) == INVALID
    assert prep(None, P(A), 64, 64, P(A), pb, None) == INVALID
    assert prep(P(A), P(A), 64, 64, None, pb, None) == INVALID
    assert prep(P(A + 8), P(A), 64, 64, P(A), pb, None) == MISALIGNED
    assert prep(P(A), P(A), 64, 64, P(A + 16), pb, None) == MISALIGNED
    assert prep(P(A), P(A), 64, 64, P(A), pb - 1, None) == WS
    assert prep(None, None, 0, 64, None, 0, None) == OK
    run = L.w4a4_gemm_prepared
    assert run(P(A), P(A), P(A), 64, 64, 33, 64, None, 0, None) == KMUL
    assert run(P(A), P(A), P(A), 64, 64, 64, 63, None, 0, None) == INVALID  # ldy < n
    assert run(None, P(A), P(A), 64, 64, 64, 64, None, 0, None) == INVALID
    assert run(P(A), None, P(A), 64, 64, 64, 64, None, 0, None) == INVALID
    assert run(P(A), P(A), None, 64, 64, 64, 64, None, 0, None) == INVALID
    assert run(P(A), P(A + 16), P(A), 64, 64, 64, 64, None, 0, None) == MISALIGNED
    assert run(P(A + 8), P(A), P(A), 64, 64, 64, 64, None, 0, None) == MISALIGNED
    assert run(None, None, None, 0, 64, 64, 64, None, 0, None) == OK
    # split K: the FFN-down shape (160 tiles of 128 x 128, 544 blocks) needs
    # 3 x m x n fp32 of partial sums; the FFN-up shape (544 tiles) none
    need = L.w4a4_gemm_prepared_workspace_bytes(512, 5120, 17408)
    assert need == 3 * 512 * 5120 * 4
    assert L.w4a4_gemm_prepared_workspace_bytes(512, 17408, 5120) == 0
    assert L.w4a4_gemm_prepared_workspace_bytes(16, 5120, 17408) == 0   # m <= 16: no matrix-core path
    assert L.w4a4_gemm_prepared_workspace_bytes(512, 1024, 5120) == 0   # K too short to split
    assert run(P(A), P(A), P(A), 512, 5120, 17408, 5120, None, 0, None) == INVALID
    assert run(P(A), P(A), P(A), 512, 5120, 17408, 5120, P(A + 16), need, None) == MISALIGNED
    assert run(P(A), P(A), P(A), 512, 5120, 17408, 5120, P(A), need - 1, None) == WS
    # w4a4_gemm's workspace: the operand (256-rounded), then the partial sums
    assert L.w4a4_gemm_workspace_bytes(512, 5120, 17408) == L.w4a4_act_operand_bytes(512, 17408) + need
    assert L.w4a4_gemm_workspace_bytes(512, 17408, 5120) == L.w4a4_act_operand_bytes(512, 5120)


def test_rotate_quantize_prepare_validation(L):
    f = L.w4a4_rotate_quantize_prepare
    pb = L.w4a4_act_operand_bytes(8, 64)
    assert f(P(A), 1, 8, 64, 64, P(A), P(A), None, pb, None) == INVALID  # act required
    assert f(P(A), 1, 8, 64, 64, P(A), P(A), P(A + 16), pb, None) == MISALIGNED
    assert f(P(A), 1, 8, 64, 64, P(A), P(A), P(A), pb - 1, None) == WS
    assert f(P(A), 7, 8, 64, 64, P(A), P(A), P(A), pb, None) == DTYPE
    assert f(P(A), 1, 8, 48, 64, P(A), P(A), P(A), pb, None) == KMUL
    assert f(None, 1, 0, 64, 64, None, None, None, 0, None) == OK


def test_rotate_quantize_validation(L):
    f = L.w4a4_rotate_quantize_act
    assert f(P(A), 2, 4, 64, 64, P(A), P(A), None) == DTYPE
    assert f(P(A), 1, 4, 48, 64, P(A), P(A), None) == KMUL
    assert f(P(A), 1, 4, 64, 32, P(A), P(A), None) == INVALID  # ldx < k
    assert f(P(A), 1, -4, 64, 64, P(A), P(A), None) == INVALID
    assert f(None, 1, 4, 64, 64, P(A), P(A), None) == INVALID
    assert f(P(ODD), 1, 4, 64, 64, P(A), P(A), None) == MISALIGNED
    assert f(P(A + 2), 0, 4, 64, 64, P(A), P(A), None) == MISALIGNED  # fp32 needs 4 B
    assert f(P(A), 1, 4, 64, 64, P(A + 4), P(A), None) == MISALIGNED
    assert f(None, 1, 0, 64, 64, None, None, None) == OK


def test_ablation_validation(L):
    q = L.w4a4_quantize_act
    assert q(P(A), 2, 4, 64, 64, P(A), P(A), None) == DTYPE
    assert q(P(A), 1, 4, 48, 64, P(A), P(A), None) == KMUL
    assert q(P(A), 1, 4, 64, 32, P(A), P(A), None) == INVALID  # ldx < k
    assert q(P(ODD), 1, 4, 64, 64, P(A), P(A), None) == MISALIGNED
    assert q(P(A), 1, 4, 64, 64, P(A + 4), P(A), None) == MISALIGNED
    assert q(None, 1, 0, 64, 64, None, None, None) == OK
    w = L.w4a4_quantize_q4_0
    assert w(P(A), 4, 40, 40, P(A), None) == KMUL
    assert w(P(A), 4, 64, 32, P(A), None) == INVALID
    assert w(P(ODD), 4, 64, 64, P(A), None) == MISALIGNED
    assert w(None, 0, 64, 64, None, None) == OK


def test_w16_validation(L):
    assert L.w4a4_w16_weight_bytes(17408, 5120) == 17408 * 5120 * 2          # 160 blocks: no K padding
    assert L.w4a4_w16_weight_bytes(33, 64) == 64 * 256 * 2                   # rows to 64, blocks to 8
    assert L.w4a4_w16_act_bytes(1, 5120) == 32 * 5120 * 2
    assert L.w4a4_w16_act_bytes(4, 40) == 0 and L.w4a4_w16_weight_bytes(-1, 64) == 0
    d = L.w4a4_dequantize_w16
    need = L.w4a4_w16_weight_bytes(4, 64)
    assert d(P(A), 4, 40, P(A), need, None) == KMUL
    assert d(P(A), 4, 64, P(A + 8), need, None) == MISALIGNED
    assert d(P(A), 4, 64, P(A), need - 1, None) == WS
    assert d(None, 4, 64, P(A), need, None) == INVALID
    assert d(None, 0, 64, None, 0, None) == OK
    r = L.w4a4_rotate_act16
    need = L.w4a4_w16_act_bytes(4, 64)
    assert r(P(A), 2, 4, 64, 64, P(A), need, None) == DTYPE
    assert r(P(A), 1, 4, 48, 64, P(A), need, None) == KMUL
    assert r(P(A), 1, 4, 64, 32, P(A), need, None) == INVALID  # ldx < k
    assert r(P(ODD), 1, 4, 64, 64, P(A), need, None) == MISALIGNED
    assert r(P(A), 1, 4, 64, 64, P(A + 8), need, None) == MISALIGNED
    assert r(P(A), 1, 4, 64, 64, P(A), need - 2, None) == WS
    assert r(None, 1, 0, 64, 64, None, 0, None) == OK
    g = L.w4a4_gemm_w16
    assert g(P(A), P(A), P(A), 4, 8, 48, 8, None) == KMUL
    assert g(P(A), P(A), P(A), 4, 8, 64, 4, None) == INVALID  # ldy < n
    assert g(P(A + 8), P(A), P(A), 4, 8, 64, 8, None) == MISALIGNED
    assert g(None, P(A), P(A), 4, 8, 64, 8, None) == INVALID
    assert g(P(A), P(A), P(A), 1 << 17, 1 << 17, 64, 1 << 17, None) == INVALID  # 2^20 tiles
    assert g(None, None, None, 0, 8, 64, 8, None) == OK


def test_prep_validation(L):
    q = L.w4a4_quantize_q4_0_h32
    assert q(P(A), 4, 40, 40, P(A), None) == KMUL
    assert q(P(A), 4, 64, 32, P(A), None) == INVALID
    assert q(P(ODD), 4, 64, 64, P(A), None) == MISALIGNED
    assert q(None, 0, 64, 64, None, None) == OK
    r = L.w4a4_repack_q4_0_h32
    assert r(P(A), P(A), 4, 40, None) == KMUL
    assert r(P(A), P(A + 8), 4, 64, None) == MISALIGNED
    assert r(None, P(A), 4, 64, None) == INVALID
    assert r(None, None, 0, 64, None) == OK


def test_gemm_id_validation(L):
    f = L.w4a4_gemm_id
    ws = L.w4a4_gemm_id_workspace_bytes(4, 8, 2)
    args = dict(packed=P(A), E=4, codes=P(A), scales=P(A), arpt=1, ids=P(A), T=8, top_k=2,
                y=P(A), n=64, k=64, ws=P(A), wsb=ws)

    def call(**kw):
        a = dict(args, **kw)
        return f(a["packed"], a["E"], a["codes"], a["scales"], a["arpt"], a["ids"], a["T"], a["top_k"],
                 a["y"], a["n"], a["k"], a["ws"], a["wsb"], None)

    assert call(k=40) == KMUL
    assert call(arpt=3) == INVALID
    assert call(E=0) == INVALID
    assert call(E=9000) == INVALID
    assert call(ids=None) == INVALID
    assert call(ws=None) == INVALID
    assert call(wsb=ws - 1) == WS
    assert call(ws=P(A + 16)) == MISALIGNED
    assert call(ids=P(A + 2)) == MISALIGNED
    assert call(T=0, packed=None, codes=None, scales=None, ids=None, y=None, ws=None) == OK
    r = L.w4a4_gemm_id_route
    assert r(None, 4, 8, 2, P(A), ws, None) == INVALID
    assert r(P(A), 0, 8, 2, P(A), ws, None) == INVALID
    assert r(P(A), 4, 8, 2, None, ws, None) == INVALID
    assert r(P(A + 2), 4, 8, 2, P(A), ws, None) == MISALIGNED
    assert r(P(A), 4, 8, 2, P(A + 16), ws, None) == MISALIGNED
    assert r(P(A), 4, 8, 2, P(A), ws - 1, None) == WS
    assert r(None, 4, 0, 2, None, 0, None) == OK
    g = L.w4a4_gemm_id_routed
    gargs = (P(A), 4, P(A), P(A), 1, 8, 2, P(A), 64, 64)
    assert g(*gargs[:-1], 40, P(A), ws, None) == KMUL
    assert g(*gargs, None, ws, None) == INVALID
    assert g(*gargs, P(A + 16), ws, None) == MISALIGNED
    assert g(*gargs, P(A), ws - 1, None) == WS
    assert g(P(A), 4, P(A), P(A), 3, 8, 2, P(A), 64, 64, P(A), ws, None) == INVALID  # rows per token
    assert g(None, 4, None, None, 1, 0, 2, None, 64, 64, None, 0, None) == OK


MAX_ROWS = 65535 * 32  # row tiles of 32 within the 65535 grid.y of the row-tiled kernels


def test_size_bounds_are_refused_before_any_launch(L):
    """Sizes whose launches would not fit the hardware's grid limits (or the
    kernels' 32-bit offsets) are refused on the host; only refused sizes are
    passed here, so nothing is ever launched on the fake pointers."""
    rq = L.w4a4_rotate_quantize_act
    assert rq(P(A), 1, MAX_ROWS + 1, 64, 64, P(A), P(A), None) == INVALID
    assert rq(P(A), 1, 4, (1 << 24) + 32, (1 << 24) + 32, P(A), P(A), None) == INVALID
    assert L.w4a4_rotate_quantize_act8(P(A), 1, MAX_ROWS + 1, 64, 64, P(A), P(A), None) == INVALID
    assert L.w4a4_rotate_quantize_prepare8(P(A), 1, MAX_ROWS + 1, 64, 64, P(A), P(A), P(A), 1 << 40, None) == INVALID
    assert L.w4a4_rotate_act16(P(A), 1, MAX_ROWS + 1, 64, 64, P(A), 1 << 40, None) == INVALID
    assert L.w4a4_gemm_prepare_act(P(A), P(A), MAX_ROWS + 1, 64, P(A), 1 << 40, None) == INVALID
    g = L.w4a4_gemm
    assert g(P(A), P(A), P(A), P(A), MAX_ROWS + 1, 64, 64, 64, P(A), 1 << 40, None) == INVALID
    assert g(P(A), P(A), P(A), P(A), 8, (1 << 26) + 32, 64, (1 << 26) + 32, P(A), 1 << 40, None) == INVALID
    assert g(P(A), P(A), P(A), P(A), 8, 64, (1 << 24) + 32, 64, P(A), 1 << 40, None) == INVALID
    # 2^20 output tiles of 128 x 128 (1024 x 1024): the dense grid would pass 2^32 threads with pieces
    gp = L.w4a4_gemm_prepared
    assert gp(P(A), P(A), P(A), 1024 * 128, 1024 * 128, 64, 1024 * 128, P(A), 1 << 40, None) == INVALID
    assert gp(P(A), P(A), P(A), MAX_ROWS + 1, 64, 64, 64, P(A), 1 << 40, None) == INVALID
    g8 = L.w4a4_gemm_a8_prepared
    assert g8(P(A), P(A), P(A), 1024 * 128, 1024 * 128, 64, 1024 * 128, None) == INVALID
    assert g8(P(A), P(A), P(A), MAX_ROWS + 1, 64, 64, 64, None) == INVALID
    assert L.w4a4_gemm_a8(P(A), P(A), P(A), P(A), 1024 * 128, 1024 * 128, 64, 1024 * 128, P(A), 1 << 40,
                          None) == INVALID
    # weight preparation: n * k / 32 threads past 2^32
    assert L.w4a4_repack_q4_0_h32(P(A), P(A), 1 << 26, 1 << 24, None) == INVALID
    assert L.w4a4_quantize_q4_0_h32(P(A), 1 << 26, 1 << 24, 1 << 24, P(A), None) == INVALID
    assert L.w4a4_dequantize_w16(P(A), 1 << 26, 1 << 24, P(A), 1 << 60, None) == INVALID
    # routed rows: n_tokens * top_k past the row bound
    gid = L.w4a4_gemm_id
    assert gid(P(A), 8, P(A), P(A), 1, P(A), MAX_ROWS // 4 + 1, 4, P(A), 64, 64, P(A), 1 << 40, None) == INVALID
    assert L.w4a4_gemm_id_route(P(A), 8, MAX_ROWS // 4 + 1, 4, P(A), 1 << 40, None) == INVALID


def test_noalloc_refuses_sizes_past_its_scratch(L):
    """The allocation-free GEMM refuses, before any device call, a product
    whose workspace would not fit its fixed scratch."""
    cap = L.w4a4_gemm_noalloc_scratch_bytes()
    assert cap == 64 << 20
    m, n, k = 16384, 32, 5120
    assert L.w4a4_gemm_workspace_bytes(m, n, k) > cap
    assert L.w4a4_gemm_noalloc(P(A), P(A), P(A), P(A), m, n, k, n, None) == WS
    # invalid sizes are reported as w4a4_gemm reports them
    assert L.w4a4_gemm_noalloc(P(A), P(A), P(A), P(A), 64, 64, 33, 64, None) == KMUL
    assert L.w4a4_gemm_noalloc(None, None, None, None, 0, 64, 64, 64, None) == OK


def test_small_prepared_sizes_and_validation(L):
    # one 1280-byte record (16 rows x 4 blocks of codes, then their scales)
    # per group of 4 blocks; none for m > 16
    assert L.w4a4_small_act_operand_bytes(16, 5120) == 40 * 1280
    assert L.w4a4_small_act_operand_bytes(1, 160) == 2 * 1280   # 5 blocks: 2 groups
    assert L.w4a4_small_act_operand_bytes(17, 5120) == 0
    assert L.w4a4_small_act_operand_bytes(16, 33) == 0
    assert L.w4a4_small_act_operand_bytes(-1, 64) == 0
    q = L.w4a4_rotate_quantize_prepare_small
    ab = L.w4a4_small_act_operand_bytes(8, 5120)
    assert q(P(A), 1, 17, 5120, 5120, P(A), P(A), P(A), 1 << 30, None) == INVALID   # more than 16 rows
    assert q(P(A), 1, 8, 5120, 5120, P(A), P(A), None, ab, None) == INVALID       # act required
    assert q(P(A), 1, 8, 5120, 5120, P(A), P(A), P(A + 16), ab, None) == MISALIGNED
    assert q(P(A), 1, 8, 5120, 5120, P(A), P(A), P(A), ab - 1, None) == WS
    assert q(P(A), 7, 8, 5120, 5120, P(A), P(A), P(A), ab, None) == DTYPE
    assert q(P(A), 1, 8, 48, 64, P(A), P(A), P(A), ab, None) == KMUL
    assert q(None, 1, 0, 64, 64, None, None, None, 0, None) == OK
    g = L.w4a4_gemm_prepared_small
    need = L.w4a4_gemm_workspace_bytes(16, 1024, 5120)   # K splits of a narrow product
    assert need > 0
    assert g(P(A), P(A), P(A), 17, 1024, 5120, 1024, P(A), need, None) == INVALID   # more than 16 rows
    assert g(P(A), P(A), P(A), 16, 1024, 5120, 1000, P(A), need, None) == INVALID   # ldy < n
    assert g(P(A), P(A), P(A), 16, 1024, 48, 1024, P(A), need, None) == KMUL
    assert g(P(A), None, P(A), 16, 1024, 5120, 1024, P(A), need, None) == INVALID
    assert g(P(A), P(A + 16), P(A), 16, 1024, 5120, 1024, P(A), need, None) == MISALIGNED
    assert g(P(ODD), P(A), P(A), 16, 1024, 5120, 1024, P(A), need, None) == MISALIGNED
    assert g(P(A), P(A), P(A), 16, 1024, 5120, 1024, None, need, None) == INVALID    # split sums need it
    assert g(P(A), P(A), P(A), 16, 1024, 5120, 1024, P(A), need - 1, None) == WS
    assert g(P(A), P(A), P(A), 16, 1024, 5120, 1024, P(A + 16), need, None) == MISALIGNED
    assert g(None, None, None, 0, 1024, 5120, 1024, None, 0, None) == OK
