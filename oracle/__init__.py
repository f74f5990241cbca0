"""CPU oracle for the Hadamard-rotated W4A4 Q4_0 matmul -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product library never does, and the
two share no code: this wraps ``oracle.c`` (plain C, gcc, -ffp-contract=off)
through ctypes and adds nothing of the method's arithmetic of its own.

The method (1bit-MONSTER engine docs, page "The lean option: ROCmFP4, ROCmI4
and Hadamard Q4_0", sections "Hadamard-rotated Q4_0: W4A4 prompt processing"
and "MoE: W4A4 on the experts") and the readings taken where that page is
silent are stated in the header of ``oracle.c``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
QK = 32

_lib = None


def build(force: bool = True) -> str:
    """Compile oracle.c with gcc into liboracle.so (plain C, no contraction)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(
            ["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-std=c11", "-D_GNU_SOURCE",
             "-shared", "-fPIC", "-Wall", "-o", tmp, _SRC, "-lm", "-lpthread"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        lib.oracle_h32.argtypes = [P]
        lib.oracle_c64.restype = ctypes.c_double
        lib.oracle_c32.restype = ctypes.c_float
        lib.oracle_half_to_float.argtypes = [ctypes.c_uint16]
        lib.oracle_half_to_float.restype = ctypes.c_float
        lib.oracle_float_to_half.argtypes = [ctypes.c_float]
        lib.oracle_float_to_half.restype = ctypes.c_uint16
        lib.oracle_rotate_weights.argtypes = [P, I64, I64, P, ctypes.c_int]
        lib.oracle_q4_0_quantize.argtypes = [P, I64, I64, P, ctypes.c_int]
        lib.oracle_q4_0_dequantize.argtypes = [P, I64, I64, P]
        lib.oracle_fwht32_f32.argtypes = [P]
        lib.oracle_rotate_quantize_act.argtypes = [P, ctypes.c_int, I64, I64, I64, P, P, ctypes.c_int]
        lib.oracle_block_sums.argtypes = [P, P, I64, I64, I64, P]
        lib.oracle_gemm.argtypes = [P, P, P, I64, I64, I64, P, I64, ctypes.c_int]
        lib.oracle_gemm_id.argtypes = [P, I64, P, P, I64, P, I64, I64, I64, I64, P, ctypes.c_int]
        lib.oracle_rotate_quantize_act8.argtypes = [P, ctypes.c_int, I64, I64, I64, P, P, ctypes.c_int]
        lib.oracle_block_sums_a8.argtypes = [P, P, I64, I64, I64, P]
        lib.oracle_gemm_a8.argtypes = [P, P, P, I64, I64, I64, P, I64, ctypes.c_int]
        lib.oracle_quantize_act_plain.argtypes = [P, ctypes.c_int, I64, I64, I64, P, P, ctypes.c_int]
        lib.oracle_rotate_act16.argtypes = [P, ctypes.c_int, I64, I64, I64, P, ctypes.c_int]
        lib.oracle_dequantize_w16.argtypes = [P, I64, I64, P]
        lib.oracle_gemm_w16.argtypes = [P, P, I64, I64, I64, P, I64, ctypes.c_int]
        _lib = lib
    return _lib


def _ptr(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data_as(ctypes.c_void_p)


def default_threads() -> int:
    return len(os.sched_getaffinity(0))


# --------------------------------------------------------------------------
# thin wrappers, one per C entry point
# --------------------------------------------------------------------------

def h32() -> np.ndarray:
    H = np.empty((QK, QK), np.int32)
    _load().oracle_h32(_ptr(H))
    return H


def c64() -> float:
    return float(_load().oracle_c64())


def c32() -> np.float32:
    return np.float32(_load().oracle_c32())


def half_to_float(bits: int) -> np.float32:
    return np.float32(_load().oracle_half_to_float(int(bits)))


def float_to_half(x) -> int:
    return int(_load().oracle_float_to_half(float(np.float32(x))))


def rotate_weights(w: np.ndarray, threads: int | None = None) -> np.ndarray:
    """fp32 [n, k] -> fp32 [n, k], each 32-block multiplied by H/sqrt(32) (fp64 sum)."""
    w = np.ascontiguousarray(w, np.float32)
    n, k = w.shape
    assert k % QK == 0
    out = np.empty_like(w)
    _load().oracle_rotate_weights(_ptr(w), n, k, _ptr(out), threads or default_threads())
    return out


def q4_0_quantize(wr: np.ndarray, threads: int | None = None) -> np.ndarray:
    """fp32 [n, k] -> Q4_0 bytes [n, k/32, 18]."""
    wr = np.ascontiguousarray(wr, np.float32)
    n, k = wr.shape
    assert k % QK == 0
    out = np.empty((n, k // QK, 18), np.uint8)
    _load().oracle_q4_0_quantize(_ptr(wr), n, k, _ptr(out), threads or default_threads())
    return out


def q4_0_dequantize(q4: np.ndarray, k: int) -> np.ndarray:
    q4 = np.ascontiguousarray(q4, np.uint8)
    n = q4.shape[0]
    out = np.empty((n, k), np.float32)
    _load().oracle_q4_0_dequantize(_ptr(q4), n, k, _ptr(out))
    return out


def prepare_weights(w: np.ndarray, threads: int | None = None) -> np.ndarray:
    """Offline step: rotate fp32 weights per 32-block, then Q4_0-quantise."""
    return q4_0_quantize(rotate_weights(w, threads), threads)


def fwht32_f32(v: np.ndarray) -> np.ndarray:
    v = np.array(v, np.float32).reshape(QK).copy()
    _load().oracle_fwht32_f32(_ptr(v))
    return v


def rotate_quantize_act(x: np.ndarray, k: int | None = None, threads: int | None = None):
    """x fp32 or fp16 [m, ldx] -> (codes uint8 [m, k/2], scales fp32 [m, k/32])."""
    assert x.dtype in (np.float32, np.float16)
    x = np.ascontiguousarray(x)
    m, ldx = x.shape
    k = ldx if k is None else k
    assert k % QK == 0 and k <= ldx
    codes = np.empty((m, k // 2), np.uint8)
    scales = np.empty((m, k // QK), np.float32)
    dtype = 0 if x.dtype == np.float32 else 1
    _load().oracle_rotate_quantize_act(_ptr(x), dtype, m, k, ldx, _ptr(codes), _ptr(scales),
                                       threads or default_threads())
    return codes, scales


def quantize_act_plain(x: np.ndarray, k: int | None = None, threads: int | None = None):
    """R9 (unrotated ablation): x fp32 or fp16 [m, ldx] -> (codes uint8 [m, k/2],
    scales fp32 [m, k/32]), per-block symmetric int4 without the rotation."""
    assert x.dtype in (np.float32, np.float16)
    x = np.ascontiguousarray(x)
    m, ldx = x.shape
    k = ldx if k is None else k
    assert k % QK == 0 and k <= ldx
    codes = np.empty((m, k // 2), np.uint8)
    scales = np.empty((m, k // QK), np.float32)
    dtype = 0 if x.dtype == np.float32 else 1
    _load().oracle_quantize_act_plain(_ptr(x), dtype, m, k, ldx, _ptr(codes), _ptr(scales),
                                      threads or default_threads())
    return codes, scales


def prepare_weights_plain(w: np.ndarray, threads: int | None = None) -> np.ndarray:
    """R9 (unrotated ablation): plain Q4_0 of the unrotated weights."""
    return q4_0_quantize(w, threads)


def rotate_act16(x: np.ndarray, k: int | None = None, threads: int | None = None) -> np.ndarray:
    """R10: x fp32 or fp16 [m, ldx] -> rotated activations as fp16 [m, k]."""
    assert x.dtype in (np.float32, np.float16)
    x = np.ascontiguousarray(x)
    m, ldx = x.shape
    k = ldx if k is None else k
    assert k % QK == 0 and k <= ldx
    out = np.empty((m, k), np.uint16)
    _load().oracle_rotate_act16(_ptr(x), 0 if x.dtype == np.float32 else 1, m, k, ldx, _ptr(out),
                                threads or default_threads())
    return out.view(np.float16)


def dequantize_w16(q4: np.ndarray, k: int) -> np.ndarray:
    """R10: Q4_0 bytes [n, k/32, 18] -> dequantised weights as fp16 [n, k]."""
    q4 = np.ascontiguousarray(q4, np.uint8)
    n = q4.shape[0]
    out = np.empty((n, k), np.uint16)
    _load().oracle_dequantize_w16(_ptr(q4), n, k, _ptr(out))
    return out.view(np.float16)


def gemm_w16(w16: np.ndarray, x16: np.ndarray, threads: int | None = None) -> np.ndarray:
    """R10: fp32 [m, n] = fp64 sums of the fp16 operands' products, rounded once."""
    w16 = np.ascontiguousarray(w16, np.float16)
    x16 = np.ascontiguousarray(x16, np.float16)
    n, k = w16.shape
    m = x16.shape[0]
    assert x16.shape[1] == k
    y = np.empty((m, n), np.float32)
    _load().oracle_gemm_w16(_ptr(w16), _ptr(x16), m, n, k, _ptr(y), n, threads or default_threads())
    return y


def block_sums(q4: np.ndarray, codes: np.ndarray, k: int) -> np.ndarray:
    """int32 [m, n, k/32]: exact per-block integer dots."""
    q4 = np.ascontiguousarray(q4, np.uint8)
    codes = np.ascontiguousarray(codes, np.uint8)
    m, n = codes.shape[0], q4.shape[0]
    S = np.empty((m, n, k // QK), np.int32)
    _load().oracle_block_sums(_ptr(q4), _ptr(codes), m, n, k, _ptr(S))
    return S


def gemm(q4: np.ndarray, codes: np.ndarray, scales: np.ndarray, k: int,
         threads: int | None = None) -> np.ndarray:
    """fp32 [m, n] = sum_b dw*s*S, each term and the sum in fp64, rounded once."""
    q4 = np.ascontiguousarray(q4, np.uint8)
    codes = np.ascontiguousarray(codes, np.uint8)
    scales = np.ascontiguousarray(scales, np.float32)
    m, n = codes.shape[0], q4.shape[0]
    y = np.empty((m, n), np.float32)
    _load().oracle_gemm(_ptr(q4), _ptr(codes), _ptr(scales), m, n, k, _ptr(y), n,
                        threads or default_threads())
    return y


def gemm_id(q4_experts: np.ndarray, codes: np.ndarray, scales: np.ndarray,
            act_rows_per_token: int, ids: np.ndarray, n: int, k: int,
            threads: int | None = None) -> np.ndarray:
    """fp32 [n_tokens, top_k, n]; q4_experts is [E, n, k/32, 18]."""
    q4_experts = np.ascontiguousarray(q4_experts, np.uint8)
    codes = np.ascontiguousarray(codes, np.uint8)
    scales = np.ascontiguousarray(scales, np.float32)
    ids = np.ascontiguousarray(ids, np.int32)
    n_expert = q4_experts.shape[0]
    n_tokens, top_k = ids.shape
    y = np.empty((n_tokens, top_k, n), np.float32)
    _load().oracle_gemm_id(_ptr(q4_experts), n_expert, _ptr(codes), _ptr(scales),
                           act_rows_per_token, _ptr(ids), n_tokens, top_k, n, k, _ptr(y),
                           threads or default_threads())
    return y


# --------------------------------------------------------------------------
# W4A8-H32 (reading R8 in oracle.c): int8 activation codes, same rotation
# --------------------------------------------------------------------------

def rotate_quantize_act8(x: np.ndarray, k: int | None = None, threads: int | None = None):
    """x fp32 or fp16 [m, ldx] -> (codes int8 [m, k], scales fp32 [m, k/32])."""
    assert x.dtype in (np.float32, np.float16)
    x = np.ascontiguousarray(x)
    m, ldx = x.shape
    k = ldx if k is None else k
    assert k % QK == 0 and k <= ldx
    codes = np.empty((m, k), np.int8)
    scales = np.empty((m, k // QK), np.float32)
    dtype = 0 if x.dtype == np.float32 else 1
    _load().oracle_rotate_quantize_act8(_ptr(x), dtype, m, k, ldx, _ptr(codes), _ptr(scales),
                                        threads or default_threads())
    return codes, scales


def block_sums_a8(q4: np.ndarray, codes: np.ndarray, k: int) -> np.ndarray:
    """int32 [m, n, k/32]: exact per-block dots of int8 codes with Q4_0 codes."""
    q4 = np.ascontiguousarray(q4, np.uint8)
    codes = np.ascontiguousarray(codes, np.int8)
    m, n = codes.shape[0], q4.shape[0]
    S = np.empty((m, n, k // QK), np.int32)
    _load().oracle_block_sums_a8(_ptr(q4), _ptr(codes), m, n, k, _ptr(S))
    return S


def gemm_a8(q4: np.ndarray, codes: np.ndarray, scales: np.ndarray, k: int,
            threads: int | None = None) -> np.ndarray:
    """fp32 [m, n] = sum_b dw*s*S with int8 codes, each term and the sum in fp64."""
    q4 = np.ascontiguousarray(q4, np.uint8)
    codes = np.ascontiguousarray(codes, np.int8)
    scales = np.ascontiguousarray(scales, np.float32)
    m, n = codes.shape[0], q4.shape[0]
    y = np.empty((m, n), np.float32)
    _load().oracle_gemm_a8(_ptr(q4), _ptr(codes), _ptr(scales), m, n, k, _ptr(y), n,
                           threads or default_threads())
    return y
