"""The Python binding refuses buffers that do not match the library's size
rules before anything reaches the device (CPU only: the checks run before the
device check, so host tensors reach exactly as far as "must live on the GPU").
"""
import pytest

torch = pytest.importorskip("torch")

from hadamard_rotated_w4a4_amd import _lib as ops  # noqa: E402

W4A4Error = ops.W4A4Error
GPU_ONLY = "must live on the GPU"


def u8(n):
    return torch.zeros(n, dtype=torch.uint8)


def f32(*shape):
    return torch.zeros(shape, dtype=torch.float32)


def raises(match, fn, *a, **kw):
    with pytest.raises(W4A4Error, match=match):
        fn(*a, **kw)


M, N, K = 20, 70, 64


def good_gemm_args():
    return dict(packed=u8(ops.packed_weight_bytes(N, K)), codes=u8(M * K // 2).reshape(M, K // 2),
                scales=f32(M, K // 32))


def test_well_formed_host_tensors_reach_the_device_check():
    a = good_gemm_args()
    raises(GPU_ONLY, ops.gemm, a["packed"], a["codes"], a["scales"], N, K)
    raises(GPU_ONLY, ops.rotate_quantize_act, torch.zeros((M, K), dtype=torch.float16))
    raises(GPU_ONLY, ops.repack_q4_0_h32, u8(ops.q4_0_bytes(N, K)), N, K)
    raises(GPU_ONLY, ops.quantize_q4_0_h32, f32(N, K))


def test_gemm_rejects_short_or_mistyped_buffers():
    a = good_gemm_args()
    raises("packed: .* bytes", ops.gemm, u8(ops.packed_weight_bytes(N, K) - 1), a["codes"], a["scales"], N, K)
    raises("packed: .* bytes", ops.gemm, a["packed"], a["codes"], a["scales"], N + 32, K)  # a wrong n
    raises("codes: dtype", ops.gemm, a["packed"], a["codes"].to(torch.int8), a["scales"], N, K)
    raises("codes: .* bytes", ops.gemm, a["packed"], a["codes"], a["scales"], N, 2 * K)  # a wrong k
    raises("scales: dtype", ops.gemm, a["packed"], a["codes"], a["scales"].double(), N, K)
    raises("scales: .* bytes", ops.gemm, a["packed"], a["codes"], f32(M, 1), N, K)
    raises("y: shape", ops.gemm, a["packed"], a["codes"], a["scales"], N, K, y=f32(M, N - 1))
    raises("y: dtype", ops.gemm, a["packed"], a["codes"], a["scales"], N, K, y=torch.zeros((M, N), dtype=torch.float16))
    raises("y: strides", ops.gemm, a["packed"], a["codes"], a["scales"], N, K, y=f32(N, M).t())


def test_sliced_inputs_are_refused_not_misread():
    a = good_gemm_args()
    wide = u8(M * K).reshape(M, K)[:, ::2]  # right size, not contiguous
    raises("codes must be contiguous", ops.gemm, a["packed"], wide, a["scales"], N, K)
    raises("x: strides", ops.rotate_quantize_act, torch.zeros((K, M), dtype=torch.float16).t())
    raises("unsupported activation dtype", ops.rotate_quantize_act, torch.zeros((M, K), dtype=torch.bfloat16))
    raises("not a multiple of 32", ops.rotate_quantize_act, torch.zeros((M, 48), dtype=torch.float16))


def test_quantiser_outputs_are_checked():
    x = torch.zeros((M, K), dtype=torch.float16)
    raises("codes: .* bytes", ops.rotate_quantize_act, x, codes=u8(M * K // 2 - 1))
    raises("scales: .* bytes", ops.rotate_quantize_act, x, scales=f32(M * K // 32 - 1))
    raises("codes: dtype", ops.rotate_quantize_act8, x, codes=u8(M * K))
    raises("act: .* bytes", ops.rotate_quantize_prepare, x, u8(ops.act_operand_bytes(M, K) - 1))


def test_weight_preparation_checks():
    raises("q4: .* bytes", ops.repack_q4_0_h32, u8(ops.q4_0_bytes(N, K) - 1), N, K)
    raises("out: .* bytes", ops.repack_q4_0_h32, u8(ops.q4_0_bytes(N, K)), N, K, out=u8(10))
    raises("w: dtype", ops.quantize_q4_0_h32, torch.zeros((N, K), dtype=torch.float16))
    raises("out: .* bytes", ops.quantize_q4_0_h32, f32(N, K), out=u8(ops.q4_0_bytes(N, K) - 1))
    raises("out: .* bytes", ops.dequantize_w16, u8(ops.q4_0_bytes(N, K)), N, K,
           out=torch.zeros(4, dtype=torch.float16))


def test_prepared_path_checks():
    raises("act: .* bytes", ops.gemm_prepared, u8(ops.packed_weight_bytes(N, K)),
           u8(ops.act_operand_bytes(M, K) - 1), M, N, K)
    raises("out: .* bytes", ops.prepare_act, u8(M * K // 2).reshape(M, K // 2), f32(M, K // 32), K, out=u8(8))


def test_gemm_id_checks():
    E, T, top_k = 3, 5, 2
    packed = u8(E * ops.packed_weight_bytes(N, K))
    codes, scales = u8(T * K // 2), f32(T, K // 32)
    ids = torch.zeros((T, top_k), dtype=torch.int32)
    raises(GPU_ONLY, ops.gemm_id, packed, E, codes, scales, 1, ids, N, K)
    raises("packed: .* bytes", ops.gemm_id, packed[:-1], E, codes, scales, 1, ids, N, K)
    raises("ids: dtype", ops.gemm_id, packed, E, codes, scales, 1, ids.long(), N, K)
    raises("ids must be contiguous", ops.gemm_id, packed, E, codes, scales, 1, torch.zeros((top_k, T), dtype=torch.int32).t(), N, K)
    raises("act_rows_per_token", ops.gemm_id, packed, E, codes, scales, 3, ids, N, K)
    raises("codes: .* bytes", ops.gemm_id, packed, E, codes, scales, top_k, ids, N, K)  # per-slot rows need T*top_k
    raises("y: .* bytes", ops.gemm_id, packed, E, codes, scales, 1, ids, N, K, y=f32(T, top_k, N - 1))
    raises("workspace: .* bytes", ops.gemm_id_routed, packed, E, codes, scales, 1, T, top_k, N, K, u8(4))


def test_a8_prepared_path_checks():
    x = torch.zeros((M, K), dtype=torch.float16)
    act8 = u8(ops.act8_operand_bytes(M, K))
    assert ops.act8_operand_bytes(M, K) == 2 * ops.act_operand_bytes(M, K)
    raises(GPU_ONLY, ops.rotate_quantize_prepare8, x, act8)
    # the W4A4 operand's size is too small for the two planes of int8 codes
    raises("act: .* bytes", ops.rotate_quantize_prepare8, x, u8(ops.act_operand_bytes(M, K)))
    raises("act: dtype", ops.rotate_quantize_prepare8, x, torch.zeros(act8.numel(), dtype=torch.int8))
    raises("codes: dtype", ops.rotate_quantize_prepare8, x, act8, codes=u8(M * K))
    raises("codes: .* bytes", ops.rotate_quantize_prepare8, x, act8, codes=torch.zeros(M * K - 1, dtype=torch.int8))
    packed = u8(ops.packed_weight_bytes(N, K))
    raises(GPU_ONLY, ops.gemm_a8_prepared, packed, act8, M, N, K)
    raises("act: .* bytes", ops.gemm_a8_prepared, packed, act8[:-1], M, N, K)
    raises("packed: .* bytes", ops.gemm_a8_prepared, packed[:-1], act8, M, N, K)
    raises("y: shape", ops.gemm_a8_prepared, packed, act8, M, N, K, y=f32(M, N - 1))


def test_small_prepared_calls_refuse_short_or_mistyped_buffers():
    m, n, k = 16, 70, 160
    act = u8(ops.small_act_operand_bytes(m, k))
    x = torch.zeros((m, k), dtype=torch.float16)
    raises(GPU_ONLY, ops.rotate_quantize_prepare_small, x, act)
    raises("act: .* bytes", ops.rotate_quantize_prepare_small, x, u8(act.numel() - 1))
    raises("at most 16", ops.rotate_quantize_prepare_small, torch.zeros((17, k), dtype=torch.float16), act)
    packed = u8(ops.packed_weight_bytes(n, k))
    raises(GPU_ONLY, ops.gemm_prepared_small, packed, act, m, n, k)
    raises("act: .* bytes", ops.gemm_prepared_small, packed, u8(act.numel() - 1), m, n, k)
    raises("act: dtype", ops.gemm_prepared_small, packed, act.to(torch.int8), m, n, k)
    raises("packed: .* bytes", ops.gemm_prepared_small, packed, act, m, n + 32, k)
    raises("y: shape", ops.gemm_prepared_small, packed, act, m, n, k, y=f32(m, n - 1))
    raises("at most 16", ops.gemm_prepared_small, packed, act, 17, n, k)
