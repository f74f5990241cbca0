"""ctypes binding of libw4a4.so (include/w4a4.h): argument marshalling only.

Every step of the hot path runs in the library's HIP kernels.  PyTorch supplies
device memory (tensor data pointers) and the current stream.  There is no
fallback: if the library is missing or a call fails, this raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libw4a4.so")

DTYPE_F32 = 0
DTYPE_F16 = 1


class W4A4Error(RuntimeError):
    """A libw4a4 call returned a status other than W4A4_OK."""


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise W4A4Error(f"{LIB_PATH} is not built; run `python -m hadamard_rotated_w4a4_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P, I64, SZ, ST = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t, ctypes.c_int
        sigs = {
            "w4a4_status_string": ([ST], ctypes.c_char_p),
            "w4a4_last_hip_error": ([], ctypes.c_char_p),
            "w4a4_q4_0_bytes": ([I64, I64], SZ),
            "w4a4_quantize_q4_0_h32": ([P, I64, I64, I64, P, P], ST),
            "w4a4_packed_weight_bytes": ([I64, I64], SZ),
            "w4a4_repack_q4_0_h32": ([P, P, I64, I64, P], ST),
            "w4a4_rotate_quantize_act": ([P, ST, I64, I64, I64, P, P, P], ST),
            "w4a4_rotate_quantize_prepare": ([P, ST, I64, I64, I64, P, P, P, SZ, P], ST),
            "w4a4_gemm_workspace_bytes": ([I64, I64, I64], SZ),
            "w4a4_act_operand_bytes": ([I64, I64], SZ),
            "w4a4_gemm_prepare_act": ([P, P, I64, I64, P, SZ, P], ST),
            "w4a4_gemm_prepared": ([P, P, P, I64, I64, I64, I64, P, SZ, P], ST),
            "w4a4_small_act_operand_bytes": ([I64, I64], SZ),
            "w4a4_rotate_quantize_prepare_small": ([P, ST, I64, I64, I64, P, P, P, SZ, P], ST),
            "w4a4_gemm_prepared_small": ([P, P, P, I64, I64, I64, I64, P, SZ, P], ST),
            "w4a4_gemm_prepared_workspace_bytes": ([I64, I64, I64], SZ),
            "w4a4_gemm": ([P, P, P, P, I64, I64, I64, I64, P, SZ, P], ST),
            "w4a4_gemm_noalloc_scratch_bytes": ([], SZ),
            "w4a4_rotate_quantize_gemm_workspace_bytes": ([I64, I64, I64], SZ),
            "w4a4_rotate_quantize_gemm": ([P, ST, I64, I64, I64, P, I64, P, I64, P, P, P, SZ, P], ST),
            "w4a4_gemm_noalloc": ([P, P, P, P, I64, I64, I64, I64, P], ST),
            "w4a4_gemm_id_workspace_bytes": ([I64, I64, I64], SZ),
            "w4a4_rotate_quantize_act8": ([P, ST, I64, I64, I64, P, P, P], ST),
            "w4a4_quantize_q4_0": ([P, I64, I64, I64, P, P], ST),
            "w4a4_quantize_act": ([P, ST, I64, I64, I64, P, P, P], ST),
            "w4a4_gemm_a8_workspace_bytes": ([I64, I64, I64], SZ),
            "w4a4_gemm_a8": ([P, P, P, P, I64, I64, I64, I64, P, SZ, P], ST),
            "w4a4_act8_operand_bytes": ([I64, I64], SZ),
            "w4a4_rotate_quantize_prepare8": ([P, ST, I64, I64, I64, P, P, P, SZ, P], ST),
            "w4a4_gemm_a8_prepared": ([P, P, P, I64, I64, I64, I64, P], ST),
            "w4a4_gemm_id": ([P, I64, P, P, I64, P, I64, I64, P, I64, I64, P, SZ, P], ST),
            "w4a4_gemm_id_route": ([P, I64, I64, I64, P, SZ, P], ST),
            "w4a4_gemm_id_routed": ([P, I64, P, P, I64, I64, I64, P, I64, I64, P, SZ, P], ST),
            "w4a4_w16_weight_bytes": ([I64, I64], SZ),
            "w4a4_w16_act_bytes": ([I64, I64], SZ),
            "w4a4_dequantize_w16": ([P, I64, I64, P, SZ, P], ST),
            "w4a4_rotate_act16": ([P, ST, I64, I64, I64, P, SZ, P], ST),
            "w4a4_gemm_w16": ([P, P, P, I64, I64, I64, I64, P], ST),
        }
        for name, (args, res) in sigs.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = res
        _lib = L
    return _lib


def _check(status: int, what: str):
    if status != 0:
        msg = lib().w4a4_status_string(status).decode()
        detail = lib().w4a4_last_hip_error().decode()
        raise W4A4Error(f"{what}: {msg}" + (f" ({detail})" if detail else ""))


def _ptr(t):
    return ctypes.c_void_p(0 if t is None else t.data_ptr())


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _require_cuda(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise W4A4Error("tensors must live on the GPU")


# --------------------------------------------------------------------------
# argument checks: the kernels trust the sizes they are given, so every
# buffer is checked against the library's own size rules before a call
# --------------------------------------------------------------------------

def _span_bytes(t: torch.Tensor) -> int:
    """Bytes from t's first element to the end of its last one."""
    if t.numel() == 0:
        return 0
    return (sum((size - 1) * stride for size, stride in zip(t.shape, t.stride())) + 1) * t.element_size()


def _need(t, name: str, dtype=None, nbytes: int = 0, dense: bool = True):
    """t exists, has the dtype, is contiguous (when the kernel reads it as a
    flat buffer) and spans at least nbytes."""
    if t is None:
        raise W4A4Error(f"{name} is required")
    if dtype is not None and t.dtype != dtype:
        raise W4A4Error(f"{name}: dtype {t.dtype}, expected {dtype}")
    if dense and not t.is_contiguous():
        raise W4A4Error(f"{name} must be contiguous")
    if _span_bytes(t) < nbytes:
        raise W4A4Error(f"{name}: {_span_bytes(t)} bytes, at least {nbytes} needed")


def _need_rows(t, name: str, dtype, rows: int, cols: int):
    """t is a 2-D matrix of at least rows x cols with unit column stride and
    a row stride of at least cols (the kernels take the row stride)."""
    if t is None:
        raise W4A4Error(f"{name} is required")
    if dtype is not None and t.dtype != dtype:
        raise W4A4Error(f"{name}: dtype {t.dtype}, expected {dtype}")
    if t.dim() != 2 or t.shape[0] < rows or t.shape[1] < cols:
        raise W4A4Error(f"{name}: shape {tuple(t.shape)}, expected at least ({rows}, {cols})")
    if rows > 1 and cols > 0 and (t.stride(1) != 1 or t.stride(0) < cols):
        raise W4A4Error(f"{name}: strides {t.stride()}, expected unit column stride and row stride >= {cols}")


def _act_dtype(x) -> int:
    dt = {torch.float32: DTYPE_F32, torch.float16: DTYPE_F16}.get(x.dtype)
    if dt is None:
        raise W4A4Error(f"unsupported activation dtype {x.dtype}")
    return dt


def _k_of(x, k):
    k = x.shape[1] if k is None else k
    if k < 0 or k % 32:
        raise W4A4Error(f"k = {k} is not a multiple of 32")
    return k


# --------------------------------------------------------------------------
# sizes
# --------------------------------------------------------------------------

def q4_0_bytes(n: int, k: int) -> int:
    return int(lib().w4a4_q4_0_bytes(n, k))


def packed_weight_bytes(n: int, k: int) -> int:
    return int(lib().w4a4_packed_weight_bytes(n, k))


def gemm_workspace_bytes(m: int, n: int, k: int) -> int:
    return int(lib().w4a4_gemm_workspace_bytes(m, n, k))


def act_operand_bytes(m: int, k: int) -> int:
    return int(lib().w4a4_act_operand_bytes(m, k))


def gemm_id_workspace_bytes(n_expert: int, n_tokens: int, top_k: int) -> int:
    return int(lib().w4a4_gemm_id_workspace_bytes(n_expert, n_tokens, top_k))


# --------------------------------------------------------------------------
# entry points
# --------------------------------------------------------------------------

def quantize_q4_0_h32(w: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """fp32 [n, k] (row stride w.stride(0)) -> rotated Q4_0 bytes uint8 [n, k/32, 18]."""
    if w is None or w.dim() != 2:
        raise W4A4Error("w must be a 2-D fp32 matrix")
    n, k = w.shape
    _need_rows(w, "w", torch.float32, n, k)
    if out is not None:
        _need(out, "out", torch.uint8, q4_0_bytes(n, k))
    _require_cuda(w, out)
    if out is None:
        out = torch.empty((n, k // 32, 18), dtype=torch.uint8, device=w.device)
    _check(lib().w4a4_quantize_q4_0_h32(_ptr(w), n, k, w.stride(0), _ptr(out), _stream(w.device)),
           "w4a4_quantize_q4_0_h32")
    return out


def repack_q4_0_h32(q4: torch.Tensor, n: int, k: int, out: torch.Tensor | None = None) -> torch.Tensor:
    """Rotated Q4_0 bytes -> packed weight buffer (uint8, private layout)."""
    _need(q4, "q4", torch.uint8, q4_0_bytes(n, k))
    if out is not None:
        _need(out, "out", torch.uint8, packed_weight_bytes(n, k))
    _require_cuda(q4, out)
    if out is None:
        out = torch.empty(packed_weight_bytes(n, k), dtype=torch.uint8, device=q4.device)
    _check(lib().w4a4_repack_q4_0_h32(_ptr(q4), _ptr(out), n, k, _stream(q4.device)),
           "w4a4_repack_q4_0_h32")
    return out


def _quantiser_outputs(x, k, codes, scales, code_bytes_per_row, code_dtype):
    m = x.shape[0]
    _need_rows(x, "x", None, m, k)
    if codes is not None:
        _need(codes, "codes", code_dtype, m * code_bytes_per_row)
    if scales is not None:
        _need(scales, "scales", torch.float32, m * (k // 32) * 4)
    _require_cuda(x, codes, scales)
    if codes is None:
        codes = torch.empty((m, code_bytes_per_row), dtype=code_dtype, device=x.device)
    if scales is None:
        scales = torch.empty((m, k // 32), dtype=torch.float32, device=x.device)
    return m, codes, scales


def rotate_quantize_act(x: torch.Tensor, k: int | None = None, codes: torch.Tensor | None = None,
                        scales: torch.Tensor | None = None):
    """x fp16/fp32 [m, >=k] (row stride x.stride(0)) -> (codes uint8 [m, k/2], scales fp32 [m, k/32])."""
    dt, k = _act_dtype(x), _k_of(x, k)
    m, codes, scales = _quantiser_outputs(x, k, codes, scales, k // 2, torch.uint8)
    _check(lib().w4a4_rotate_quantize_act(_ptr(x), dt, m, k, x.stride(0), _ptr(codes), _ptr(scales),
                                          _stream(x.device)), "w4a4_rotate_quantize_act")
    return codes, scales


def rotate_quantize_prepare(x: torch.Tensor, act: torch.Tensor, k: int | None = None,
                            codes: torch.Tensor | None = None, scales: torch.Tensor | None = None):
    """rotate_quantize_act that also writes the matrix-core operand into `act`."""
    dt, k = _act_dtype(x), _k_of(x, k)
    _need(act, "act", torch.uint8, act_operand_bytes(x.shape[0], k))
    m, codes, scales = _quantiser_outputs(x, k, codes, scales, k // 2, torch.uint8)
    _require_cuda(act)
    _check(lib().w4a4_rotate_quantize_prepare(_ptr(x), dt, m, k, x.stride(0), _ptr(codes), _ptr(scales), _ptr(act),
                                              act.numel(), _stream(x.device)), "w4a4_rotate_quantize_prepare")
    return codes, scales


def _check_out(y, ws, m, n, need):
    if y is not None:
        _need_rows(y, "y", torch.float32, m, n)
    if ws is not None:
        _need(ws, "workspace", torch.uint8, need)


def _output(y, m, n, device):
    return torch.empty((m, n), dtype=torch.float32, device=device) if y is None else y


def _workspace(ws, need, device):
    if ws is not None:
        _need(ws, "workspace", torch.uint8, need)
        return ws
    return torch.empty(need, dtype=torch.uint8, device=device) if need else None


def gemm(packed: torch.Tensor, codes: torch.Tensor, scales: torch.Tensor, n: int, k: int,
         y: torch.Tensor | None = None, workspace: torch.Tensor | None = None) -> torch.Tensor:
    """W4A4 product: fp32 [m, n] (row stride y.stride(0)).  The workspace is
    allocated here unless given (uint8, at least gemm_workspace_bytes)."""
    m = codes.shape[0]
    _need(packed, "packed", torch.uint8, packed_weight_bytes(n, k) if m and n else 0)
    _need(codes, "codes", torch.uint8, m * (k // 2))
    _need(scales, "scales", torch.float32, m * (k // 32) * 4)
    need = gemm_workspace_bytes(m, n, k)
    _check_out(y, workspace, m, n, need)
    _require_cuda(packed, codes, scales, y, workspace)
    y = _output(y, m, n, codes.device)
    workspace = _workspace(workspace, need, codes.device)
    _check(lib().w4a4_gemm(_ptr(packed), _ptr(codes), _ptr(scales), _ptr(y), m, n, k, y.stride(0),
                           _ptr(workspace), 0 if workspace is None else workspace.numel(),
                           _stream(codes.device)), "w4a4_gemm")
    return y


def gemm_noalloc(packed: torch.Tensor, codes: torch.Tensor, scales: torch.Tensor, n: int, k: int,
                 y: torch.Tensor | None = None) -> torch.Tensor:
    """W4A4 product with the library's own fixed scratch (no workspace
    allocated anywhere; y is allocated here only when not given)."""
    m = codes.shape[0]
    _need(packed, "packed", torch.uint8, packed_weight_bytes(n, k) if m and n else 0)
    _need(codes, "codes", torch.uint8, m * (k // 2))
    _need(scales, "scales", torch.float32, m * (k // 32) * 4)
    _check_out(y, None, m, n, 0)
    _require_cuda(packed, codes, scales, y)
    y = _output(y, m, n, codes.device)
    _check(lib().w4a4_gemm_noalloc(_ptr(packed), _ptr(codes), _ptr(scales), _ptr(y), m, n, k, y.stride(0),
                                   _stream(codes.device)), "w4a4_gemm_noalloc")
    return y


def rotate_quantize_gemm_workspace_bytes(m: int, n: int, k: int) -> int:
    return int(lib().w4a4_rotate_quantize_gemm_workspace_bytes(m, n, k))


def fused_workspace(m: int, n: int, k: int, device) -> torch.Tensor:
    """A zero-filled workspace for rotate_quantize_gemm (zero before its first
    use; the calls keep it ready for the next)."""
    return torch.zeros(max(256, rotate_quantize_gemm_workspace_bytes(m, n, k)), dtype=torch.uint8, device=device)


def rotate_quantize_gemm(x: torch.Tensor, packed: torch.Tensor, n: int, k: int | None = None,
                         y: torch.Tensor | None = None, codes: torch.Tensor | None = None,
                         scales: torch.Tensor | None = None, workspace: torch.Tensor | None = None):
    """Rotate-quantise x fp16/fp32 [m, >=k] and multiply with the packed
    weights in one call (one launch for m <= 16): returns (y fp32 [m, n],
    codes, scales).  The workspace must come from fused_workspace (or be
    zeroed likewise); a new one is made when none is given."""
    dt, k = _act_dtype(x), _k_of(x, k)
    m = x.shape[0]
    _need(packed, "packed", torch.uint8, packed_weight_bytes(n, k) if m and n else 0)
    need = rotate_quantize_gemm_workspace_bytes(m, n, k)
    _check_out(y, workspace, m, n, need)
    m, codes, scales = _quantiser_outputs(x, k, codes, scales, k // 2, torch.uint8)
    _require_cuda(packed, y, workspace)
    y = _output(y, m, n, x.device)
    if workspace is None:
        workspace = fused_workspace(m, n, k, x.device)
    _check(lib().w4a4_rotate_quantize_gemm(_ptr(x), dt, m, k, x.stride(0), _ptr(packed), n, _ptr(y), y.stride(0),
                                           _ptr(codes), _ptr(scales), _ptr(workspace), workspace.numel(),
                                           _stream(x.device)), "w4a4_rotate_quantize_gemm")
    return y, codes, scales


def prepare_act(codes: torch.Tensor, scales: torch.Tensor, k: int,
                out: torch.Tensor | None = None) -> torch.Tensor:
    """Activation codes + scales -> prepared matrix-core operand (uint8, private layout)."""
    m = codes.shape[0]
    _need(codes, "codes", torch.uint8, m * (k // 2))
    _need(scales, "scales", torch.float32, m * (k // 32) * 4)
    if out is not None:
        _need(out, "out", torch.uint8, act_operand_bytes(m, k))
    _require_cuda(codes, scales, out)
    if out is None:
        out = torch.empty(max(1, act_operand_bytes(m, k)), dtype=torch.uint8, device=codes.device)
    _check(lib().w4a4_gemm_prepare_act(_ptr(codes), _ptr(scales), m, k, _ptr(out), out.numel(),
                                       _stream(codes.device)), "w4a4_gemm_prepare_act")
    return out


def gemm_prepared_workspace_bytes(m: int, n: int, k: int) -> int:
    return int(lib().w4a4_gemm_prepared_workspace_bytes(m, n, k))


def gemm_prepared(packed: torch.Tensor, act: torch.Tensor, m: int, n: int, k: int,
                  y: torch.Tensor | None = None, workspace: torch.Tensor | None = None) -> torch.Tensor:
    """W4A4 product on a prepared activation: fp32 [m, n] (row stride y.stride(0)).
    The split-K workspace is allocated here when one is needed and not given."""
    _need(packed, "packed", torch.uint8, packed_weight_bytes(n, k) if m and n else 0)
    _need(act, "act", torch.uint8, act_operand_bytes(m, k))
    need = gemm_prepared_workspace_bytes(m, n, k)
    _check_out(y, workspace, m, n, need)
    _require_cuda(packed, act, y, workspace)
    y = _output(y, m, n, act.device)
    workspace = _workspace(workspace, need, act.device)
    _check(lib().w4a4_gemm_prepared(_ptr(packed), _ptr(act), _ptr(y), m, n, k, y.stride(0), _ptr(workspace),
                                    0 if workspace is None else workspace.numel(), _stream(act.device)),
           "w4a4_gemm_prepared")
    return y


def small_act_operand_bytes(m: int, k: int) -> int:
    return int(lib().w4a4_small_act_operand_bytes(m, k))


def rotate_quantize_prepare_small(x: torch.Tensor, act: torch.Tensor, k: int | None = None,
                                  codes: torch.Tensor | None = None, scales: torch.Tensor | None = None):
    """rotate_quantize_act for m <= 16 rows that also writes the record-ordered
    operand of the m <= 16 product into `act`."""
    dt, k = _act_dtype(x), _k_of(x, k)
    if x.shape[0] > 16:
        raise W4A4Error(f"rotate_quantize_prepare_small: {x.shape[0]} rows (at most 16)")
    _need(act, "act", torch.uint8, small_act_operand_bytes(x.shape[0], k))
    m, codes, scales = _quantiser_outputs(x, k, codes, scales, k // 2, torch.uint8)
    _require_cuda(act)
    _check(lib().w4a4_rotate_quantize_prepare_small(_ptr(x), dt, m, k, x.stride(0), _ptr(codes), _ptr(scales),
                                                    _ptr(act), act.numel(), _stream(x.device)),
           "w4a4_rotate_quantize_prepare_small")
    return codes, scales


def gemm_prepared_small(packed: torch.Tensor, act: torch.Tensor, m: int, n: int, k: int,
                        y: torch.Tensor | None = None, workspace: torch.Tensor | None = None) -> torch.Tensor:
    """The m <= 16 product on a record-ordered operand: fp32 [m, n] (row
    stride y.stride(0)); the same result as gemm on the same codes and scales.
    The workspace (K splits) is allocated here when needed and not given."""
    if m > 16:
        raise W4A4Error(f"gemm_prepared_small: {m} rows (at most 16)")
    _need(packed, "packed", torch.uint8, packed_weight_bytes(n, k) if m and n else 0)
    _need(act, "act", torch.uint8, small_act_operand_bytes(m, k))
    need = gemm_workspace_bytes(m, n, k)
    _check_out(y, workspace, m, n, need)
    _require_cuda(packed, act, y, workspace)
    y = _output(y, m, n, act.device)
    workspace = _workspace(workspace, need, act.device)
    _check(lib().w4a4_gemm_prepared_small(_ptr(packed), _ptr(act), _ptr(y), m, n, k, y.stride(0),
                                          _ptr(workspace), 0 if workspace is None else workspace.numel(),
                                          _stream(act.device)), "w4a4_gemm_prepared_small")
    return y


def _gemm_id_args(packed, n_expert, codes, scales, act_rows_per_token, n_tokens, top_k, n, k, y, code_bytes):
    if act_rows_per_token not in (1, top_k):
        raise W4A4Error(f"act_rows_per_token = {act_rows_per_token}, expected 1 or top_k = {top_k}")
    rows = n_tokens * act_rows_per_token
    _need(packed, "packed", torch.uint8, n_expert * packed_weight_bytes(n, k))
    _need(codes, "codes", None, rows * code_bytes)
    _need(scales, "scales", torch.float32, rows * (k // 32) * 4)
    if y is not None:
        _need(y, "y", torch.float32, n_tokens * top_k * n * 4)
    _require_cuda(packed, codes, scales, y)
    if y is None:
        y = torch.empty((n_tokens, top_k, n), dtype=torch.float32, device=codes.device)
    return y


def gemm_id(packed: torch.Tensor, n_expert: int, codes: torch.Tensor, scales: torch.Tensor,
            act_rows_per_token: int, ids: torch.Tensor, n: int, k: int, y: torch.Tensor | None = None,
            workspace: torch.Tensor | None = None) -> torch.Tensor:
    """MUL_MAT_ID: fp32 [n_tokens, top_k, n]."""
    if ids is None or ids.dim() != 2:
        raise W4A4Error("ids must be an int32 [n_tokens, top_k] matrix")
    _need(ids, "ids", torch.int32)
    n_tokens, top_k = ids.shape
    _need(codes, "codes", torch.uint8)
    y = _gemm_id_args(packed, n_expert, codes, scales, act_rows_per_token, n_tokens, top_k, n, k, y, k // 2)
    need = gemm_id_workspace_bytes(n_expert, n_tokens, top_k)
    workspace = _workspace(workspace, need, ids.device) if need else _workspace(workspace, 1, ids.device)
    _require_cuda(ids, workspace)
    _check(lib().w4a4_gemm_id(_ptr(packed), n_expert, _ptr(codes), _ptr(scales), act_rows_per_token,
                              _ptr(ids), n_tokens, top_k, _ptr(y), n, k, _ptr(workspace),
                              workspace.numel(), _stream(ids.device)), "w4a4_gemm_id")
    return y


def gemm_id_route(ids: torch.Tensor, n_expert: int, workspace: torch.Tensor | None = None) -> torch.Tensor:
    """MUL_MAT_ID routing of ids [n_tokens, top_k] into a workspace (returned)."""
    if ids is None or ids.dim() != 2:
        raise W4A4Error("ids must be an int32 [n_tokens, top_k] matrix")
    _need(ids, "ids", torch.int32)
    n_tokens, top_k = ids.shape
    need = max(1, gemm_id_workspace_bytes(n_expert, n_tokens, top_k))
    workspace = _workspace(workspace, need, ids.device)
    _require_cuda(ids, workspace)
    _check(lib().w4a4_gemm_id_route(_ptr(ids), n_expert, n_tokens, top_k, _ptr(workspace), workspace.numel(),
                                    _stream(ids.device)), "w4a4_gemm_id_route")
    return workspace


def gemm_id_routed(packed: torch.Tensor, n_expert: int, codes: torch.Tensor, scales: torch.Tensor,
                   act_rows_per_token: int, n_tokens: int, top_k: int, n: int, k: int, workspace: torch.Tensor,
                   y: torch.Tensor | None = None) -> torch.Tensor:
    """MUL_MAT_ID on a routing from gemm_id_route: fp32 [n_tokens, top_k, n]."""
    _need(codes, "codes", torch.uint8)
    _need(workspace, "workspace", torch.uint8, gemm_id_workspace_bytes(n_expert, n_tokens, top_k))
    y = _gemm_id_args(packed, n_expert, codes, scales, act_rows_per_token, n_tokens, top_k, n, k, y, k // 2)
    _require_cuda(workspace)
    _check(lib().w4a4_gemm_id_routed(_ptr(packed), n_expert, _ptr(codes), _ptr(scales), act_rows_per_token,
                                     n_tokens, top_k, _ptr(y), n, k, _ptr(workspace), workspace.numel(),
                                     _stream(codes.device)), "w4a4_gemm_id_routed")
    return y


def rotate_quantize_act8(x: torch.Tensor, k: int | None = None, codes: torch.Tensor | None = None,
                         scales: torch.Tensor | None = None):
    """W4A8-H32 activations: x fp16/fp32 [m, >=k] -> (codes int8 [m, k], scales fp32 [m, k/32])."""
    dt, k = _act_dtype(x), _k_of(x, k)
    m, codes, scales = _quantiser_outputs(x, k, codes, scales, k, torch.int8)
    _check(lib().w4a4_rotate_quantize_act8(_ptr(x), dt, m, k, x.stride(0), _ptr(codes), _ptr(scales),
                                           _stream(x.device)), "w4a4_rotate_quantize_act8")
    return codes, scales


def gemm_a8(packed: torch.Tensor, codes: torch.Tensor, scales: torch.Tensor, n: int, k: int,
            y: torch.Tensor | None = None, workspace: torch.Tensor | None = None) -> torch.Tensor:
    """W4A8-H32 product: fp32 [m, n] (row stride y.stride(0))."""
    m = codes.shape[0]
    _need(packed, "packed", torch.uint8, packed_weight_bytes(n, k) if m and n else 0)
    _need(codes, "codes", torch.int8, m * k)
    _need(scales, "scales", torch.float32, m * (k // 32) * 4)
    need = int(lib().w4a4_gemm_a8_workspace_bytes(m, n, k))
    _check_out(y, workspace, m, n, need)
    _require_cuda(packed, codes, scales, y, workspace)
    y = _output(y, m, n, codes.device)
    workspace = _workspace(workspace, need, codes.device)
    _check(lib().w4a4_gemm_a8(_ptr(packed), _ptr(codes), _ptr(scales), _ptr(y), m, n, k, y.stride(0),
                              _ptr(workspace), 0 if workspace is None else workspace.numel(),
                              _stream(codes.device)), "w4a4_gemm_a8")
    return y


def act8_operand_bytes(m: int, k: int) -> int:
    return int(lib().w4a4_act8_operand_bytes(m, k))


def rotate_quantize_prepare8(x: torch.Tensor, act: torch.Tensor, k: int | None = None,
                             codes: torch.Tensor | None = None, scales: torch.Tensor | None = None):
    """rotate_quantize_act8 that also writes the int8 matrix-core operand into `act`."""
    dt, k = _act_dtype(x), _k_of(x, k)
    _need(act, "act", torch.uint8, act8_operand_bytes(x.shape[0], k))
    m, codes, scales = _quantiser_outputs(x, k, codes, scales, k, torch.int8)
    _require_cuda(act)
    _check(lib().w4a4_rotate_quantize_prepare8(_ptr(x), dt, m, k, x.stride(0), _ptr(codes), _ptr(scales),
                                               _ptr(act), act.numel(), _stream(x.device)),
           "w4a4_rotate_quantize_prepare8")
    return codes, scales


def gemm_a8_prepared(packed: torch.Tensor, act: torch.Tensor, m: int, n: int, k: int,
                     y: torch.Tensor | None = None) -> torch.Tensor:
    """W4A8-H32 product on a prepared int8 operand: fp32 [m, n] (row stride y.stride(0))."""
    _need(packed, "packed", torch.uint8, packed_weight_bytes(n, k) if m and n else 0)
    _need(act, "act", torch.uint8, act8_operand_bytes(m, k))
    _check_out(y, None, m, n, 0)
    _require_cuda(packed, act, y)
    y = _output(y, m, n, act.device)
    _check(lib().w4a4_gemm_a8_prepared(_ptr(packed), _ptr(act), _ptr(y), m, n, k, y.stride(0),
                                       _stream(act.device)), "w4a4_gemm_a8_prepared")
    return y


def prepare_weights(w: torch.Tensor) -> torch.Tensor:
    """Offline step on the GPU: fp32 [n, k] -> rotated Q4_0 -> packed buffer."""
    n, k = w.shape
    return repack_q4_0_h32(quantize_q4_0_h32(w), n, k)


# --------------------------------------------------------------------------
# Unrotated W4A4 ablation: the same GEMM entry points, nothing rotated
# --------------------------------------------------------------------------

def quantize_q4_0(w: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """fp32 [n, k] (row stride w.stride(0)) -> plain (unrotated) Q4_0 bytes uint8 [n, k/32, 18]."""
    if w is None or w.dim() != 2:
        raise W4A4Error("w must be a 2-D fp32 matrix")
    n, k = w.shape
    _need_rows(w, "w", torch.float32, n, k)
    if out is not None:
        _need(out, "out", torch.uint8, q4_0_bytes(n, k))
    _require_cuda(w, out)
    if out is None:
        out = torch.empty((n, k // 32, 18), dtype=torch.uint8, device=w.device)
    _check(lib().w4a4_quantize_q4_0(_ptr(w), n, k, w.stride(0), _ptr(out), _stream(w.device)), "w4a4_quantize_q4_0")
    return out


def quantize_act(x: torch.Tensor, k: int | None = None, codes: torch.Tensor | None = None,
                 scales: torch.Tensor | None = None):
    """x fp16/fp32 [m, >=k] -> unrotated int4 (codes uint8 [m, k/2], scales fp32 [m, k/32])."""
    dt, k = _act_dtype(x), _k_of(x, k)
    m, codes, scales = _quantiser_outputs(x, k, codes, scales, k // 2, torch.uint8)
    _check(lib().w4a4_quantize_act(_ptr(x), dt, m, k, x.stride(0), _ptr(codes), _ptr(scales), _stream(x.device)),
           "w4a4_quantize_act")
    return codes, scales


def prepare_weights_plain(w: torch.Tensor) -> torch.Tensor:
    """fp32 [n, k] -> plain (unrotated) Q4_0 -> packed buffer (the ablation's weights)."""
    n, k = w.shape
    return repack_q4_0_h32(quantize_q4_0(w), n, k)


# --------------------------------------------------------------------------
# Rotated W4A16: the rotated Q4_0 weights against rotated fp16 activations
# --------------------------------------------------------------------------

def w16_blocks(k: int) -> int:
    """Blocks per row of a tiled fp16 operand (k / 32 padded to a multiple of 8)."""
    return (k // 32 + 7) // 8 * 8


def w16_to_rows(buf: torch.Tensor, rows: int, k: int) -> torch.Tensor:
    """A tiled fp16 operand as a row-major [rows, k] view copy (layout only)."""
    nbp, tiles = w16_blocks(k), (rows + 31) // 32
    t = buf.reshape(tiles, nbp, 2, 2, 32, 8).permute(0, 4, 1, 2, 3, 5)
    return t.reshape(tiles * 32, nbp * 32)[:rows, :k].contiguous()


def dequantize_w16(q4: torch.Tensor, n: int, k: int, out: torch.Tensor | None = None) -> torch.Tensor:
    """Q4_0 bytes -> tiled fp16 weights (flat, w4a4_w16_weight_bytes(n, k) bytes)."""
    need = int(lib().w4a4_w16_weight_bytes(n, k))
    _need(q4, "q4", torch.uint8, q4_0_bytes(n, k))
    if out is not None:
        _need(out, "out", torch.float16, need)
    _require_cuda(q4, out)
    if out is None:
        out = torch.empty(need // 2, dtype=torch.float16, device=q4.device)
    _check(lib().w4a4_dequantize_w16(_ptr(q4), n, k, _ptr(out), out.numel() * out.element_size(),
                                     _stream(q4.device)), "w4a4_dequantize_w16")
    return out


def rotate_act16(x: torch.Tensor, k: int | None = None, out: torch.Tensor | None = None) -> torch.Tensor:
    """x fp16/fp32 [m, >=k] -> tiled rotated fp16 activations (flat, w4a4_w16_act_bytes(m, k) bytes)."""
    dt, k = _act_dtype(x), _k_of(x, k)
    m = x.shape[0]
    _need_rows(x, "x", None, m, k)
    need = int(lib().w4a4_w16_act_bytes(m, k))
    if out is not None:
        _need(out, "out", torch.float16, need)
    _require_cuda(x, out)
    if out is None:
        out = torch.empty(need // 2, dtype=torch.float16, device=x.device)
    _check(lib().w4a4_rotate_act16(_ptr(x), dt, m, k, x.stride(0), _ptr(out), out.numel() * out.element_size(),
                                   _stream(x.device)), "w4a4_rotate_act16")
    return out


def gemm_w16(w16: torch.Tensor, a16: torch.Tensor, m: int, n: int, k: int,
             y: torch.Tensor | None = None) -> torch.Tensor:
    """W4A16 product of the two tiled fp16 operands: fp32 [m, n] (row stride y.stride(0))."""
    _need(w16, "w16", torch.float16, int(lib().w4a4_w16_weight_bytes(n, k)))
    _need(a16, "a16", torch.float16, int(lib().w4a4_w16_act_bytes(m, k)))
    _check_out(y, None, m, n, 0)
    _require_cuda(w16, a16, y)
    y = _output(y, m, n, a16.device)
    _check(lib().w4a4_gemm_w16(_ptr(w16), _ptr(a16), _ptr(y), m, n, k, y.stride(0), _stream(a16.device)),
           "w4a4_gemm_w16")
    return y
