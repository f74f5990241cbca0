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
            "w4a4_gemm_prepared_workspace_bytes": ([I64, I64, I64], SZ),
            "w4a4_gemm": ([P, P, P, P, I64, I64, I64, I64, P, SZ, P], ST),
            "w4a4_gemm_id_workspace_bytes": ([I64, I64, I64], SZ),
            "w4a4_rotate_quantize_act8": ([P, ST, I64, I64, I64, P, P, P], ST),
            "w4a4_quantize_q4_0": ([P, I64, I64, I64, P, P], ST),
            "w4a4_quantize_act": ([P, ST, I64, I64, I64, P, P, P], ST),
            "w4a4_gemm_a8_workspace_bytes": ([I64, I64, I64], SZ),
            "w4a4_gemm_a8": ([P, P, P, P, I64, I64, I64, I64, P, SZ, P], ST),
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
    _require_cuda(w, out)
    assert w.dtype == torch.float32 and w.dim() == 2 and w.stride(1) == 1
    n, k = w.shape
    if out is None:
        out = torch.empty((n, k // 32, 18), dtype=torch.uint8, device=w.device)
    _check(lib().w4a4_quantize_q4_0_h32(_ptr(w), n, k, w.stride(0), _ptr(out), _stream(w.device)),
           "w4a4_quantize_q4_0_h32")
    return out


def repack_q4_0_h32(q4: torch.Tensor, n: int, k: int, out: torch.Tensor | None = None) -> torch.Tensor:
    """Rotated Q4_0 bytes -> packed weight buffer (uint8, private layout)."""
    _require_cuda(q4, out)
    if out is None:
        out = torch.empty(packed_weight_bytes(n, k), dtype=torch.uint8, device=q4.device)
    _check(lib().w4a4_repack_q4_0_h32(_ptr(q4), _ptr(out), n, k, _stream(q4.device)),
           "w4a4_repack_q4_0_h32")
    return out


def rotate_quantize_act(x: torch.Tensor, k: int | None = None, codes: torch.Tensor | None = None,
                        scales: torch.Tensor | None = None):
    """x fp16/fp32 [m, >=k] (row stride x.stride(0)) -> (codes uint8 [m, k/2], scales fp32 [m, k/32])."""
    _require_cuda(x, codes, scales)
    assert x.dim() == 2 and x.stride(1) == 1
    dt = {torch.float32: DTYPE_F32, torch.float16: DTYPE_F16}.get(x.dtype)
    if dt is None:
        raise W4A4Error(f"unsupported activation dtype {x.dtype}")
    m = x.shape[0]
    k = x.shape[1] if k is None else k
    if codes is None:
        codes = torch.empty((m, k // 2), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty((m, k // 32), dtype=torch.float32, device=x.device)
    _check(lib().w4a4_rotate_quantize_act(_ptr(x), dt, m, k, x.stride(0), _ptr(codes), _ptr(scales),
                                          _stream(x.device)), "w4a4_rotate_quantize_act")
    return codes, scales


def rotate_quantize_prepare(x: torch.Tensor, act: torch.Tensor, k: int | None = None,
                            codes: torch.Tensor | None = None, scales: torch.Tensor | None = None):
    """rotate_quantize_act that also writes the matrix-core operand into `act`."""
    _require_cuda(x, act, codes, scales)
    assert x.dim() == 2 and x.stride(1) == 1
    dt = {torch.float32: DTYPE_F32, torch.float16: DTYPE_F16}.get(x.dtype)
    if dt is None:
        raise W4A4Error(f"unsupported activation dtype {x.dtype}")
    m = x.shape[0]
    k = x.shape[1] if k is None else k
    if codes is None:
        codes = torch.empty((m, k // 2), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty((m, k // 32), dtype=torch.float32, device=x.device)
    _check(lib().w4a4_rotate_quantize_prepare(_ptr(x), dt, m, k, x.stride(0), _ptr(codes), _ptr(scales), _ptr(act),
                                              act.numel(), _stream(x.device)), "w4a4_rotate_quantize_prepare")
    return codes, scales


def gemm(packed: torch.Tensor, codes: torch.Tensor, scales: torch.Tensor, n: int, k: int,
         y: torch.Tensor | None = None, workspace: torch.Tensor | None = None) -> torch.Tensor:
    """W4A4 product: fp32 [m, n] (row stride y.stride(0)).  The workspace is
    allocated here unless given (uint8, at least gemm_workspace_bytes)."""
    _require_cuda(packed, codes, scales, y, workspace)
    m = codes.shape[0]
    if y is None:
        y = torch.empty((m, n), dtype=torch.float32, device=codes.device)
    assert y.stride(1) == 1
    need = gemm_workspace_bytes(m, n, k)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=codes.device)
    _check(lib().w4a4_gemm(_ptr(packed), _ptr(codes), _ptr(scales), _ptr(y), m, n, k, y.stride(0),
                           _ptr(workspace), 0 if workspace is None else workspace.numel(),
                           _stream(codes.device)), "w4a4_gemm")
    return y


def prepare_act(codes: torch.Tensor, scales: torch.Tensor, k: int,
                out: torch.Tensor | None = None) -> torch.Tensor:
    """Activation codes + scales -> prepared matrix-core operand (uint8, private layout)."""
    _require_cuda(codes, scales, out)
    m = codes.shape[0]
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
    _require_cuda(packed, act, y, workspace)
    if y is None:
        y = torch.empty((m, n), dtype=torch.float32, device=act.device)
    assert y.stride(1) == 1
    need = gemm_prepared_workspace_bytes(m, n, k)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=act.device)
    _check(lib().w4a4_gemm_prepared(_ptr(packed), _ptr(act), _ptr(y), m, n, k, y.stride(0), _ptr(workspace),
                                    0 if workspace is None else workspace.numel(), _stream(act.device)),
           "w4a4_gemm_prepared")
    return y


def gemm_id(packed: torch.Tensor, n_expert: int, codes: torch.Tensor, scales: torch.Tensor,
            act_rows_per_token: int, ids: torch.Tensor, n: int, k: int, y: torch.Tensor | None = None,
            workspace: torch.Tensor | None = None) -> torch.Tensor:
    """MUL_MAT_ID: fp32 [n_tokens, top_k, n]."""
    _require_cuda(packed, codes, scales, ids, y, workspace)
    assert ids.dtype == torch.int32 and ids.dim() == 2
    n_tokens, top_k = ids.shape
    if y is None:
        y = torch.empty((n_tokens, top_k, n), dtype=torch.float32, device=ids.device)
    need = gemm_id_workspace_bytes(n_expert, n_tokens, top_k)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=ids.device)
    _check(lib().w4a4_gemm_id(_ptr(packed), n_expert, _ptr(codes), _ptr(scales), act_rows_per_token,
                              _ptr(ids.contiguous()), n_tokens, top_k, _ptr(y), n, k, _ptr(workspace),
                              workspace.numel(), _stream(ids.device)), "w4a4_gemm_id")
    return y


def gemm_id_route(ids: torch.Tensor, n_expert: int, workspace: torch.Tensor | None = None) -> torch.Tensor:
    """MUL_MAT_ID routing of ids [n_tokens, top_k] into a workspace (returned)."""
    _require_cuda(ids, workspace)
    assert ids.dtype == torch.int32 and ids.dim() == 2 and ids.is_contiguous()
    n_tokens, top_k = ids.shape
    if workspace is None:
        workspace = torch.empty(max(1, gemm_id_workspace_bytes(n_expert, n_tokens, top_k)), dtype=torch.uint8,
                                device=ids.device)
    _check(lib().w4a4_gemm_id_route(_ptr(ids), n_expert, n_tokens, top_k, _ptr(workspace), workspace.numel(),
                                    _stream(ids.device)), "w4a4_gemm_id_route")
    return workspace


def gemm_id_routed(packed: torch.Tensor, n_expert: int, codes: torch.Tensor, scales: torch.Tensor,
                   act_rows_per_token: int, n_tokens: int, top_k: int, n: int, k: int, workspace: torch.Tensor,
                   y: torch.Tensor | None = None) -> torch.Tensor:
    """MUL_MAT_ID on a routing from gemm_id_route: fp32 [n_tokens, top_k, n]."""
    _require_cuda(packed, codes, scales, workspace, y)
    if y is None:
        y = torch.empty((n_tokens, top_k, n), dtype=torch.float32, device=codes.device)
    _check(lib().w4a4_gemm_id_routed(_ptr(packed), n_expert, _ptr(codes), _ptr(scales), act_rows_per_token,
                                     n_tokens, top_k, _ptr(y), n, k, _ptr(workspace), workspace.numel(),
                                     _stream(codes.device)), "w4a4_gemm_id_routed")
    return y


def rotate_quantize_act8(x: torch.Tensor, k: int | None = None, codes: torch.Tensor | None = None,
                         scales: torch.Tensor | None = None):
    """W4A8-H32 activations: x fp16/fp32 [m, >=k] -> (codes int8 [m, k], scales fp32 [m, k/32])."""
    _require_cuda(x, codes, scales)
    assert x.dim() == 2 and x.stride(1) == 1
    dt = {torch.float32: DTYPE_F32, torch.float16: DTYPE_F16}.get(x.dtype)
    if dt is None:
        raise W4A4Error(f"unsupported activation dtype {x.dtype}")
    m = x.shape[0]
    k = x.shape[1] if k is None else k
    if codes is None:
        codes = torch.empty((m, k), dtype=torch.int8, device=x.device)
    if scales is None:
        scales = torch.empty((m, k // 32), dtype=torch.float32, device=x.device)
    _check(lib().w4a4_rotate_quantize_act8(_ptr(x), dt, m, k, x.stride(0), _ptr(codes), _ptr(scales),
                                           _stream(x.device)), "w4a4_rotate_quantize_act8")
    return codes, scales


def gemm_a8(packed: torch.Tensor, codes: torch.Tensor, scales: torch.Tensor, n: int, k: int,
            y: torch.Tensor | None = None, workspace: torch.Tensor | None = None) -> torch.Tensor:
    """W4A8-H32 product: fp32 [m, n] (row stride y.stride(0))."""
    _require_cuda(packed, codes, scales, y, workspace)
    m = codes.shape[0]
    if y is None:
        y = torch.empty((m, n), dtype=torch.float32, device=codes.device)
    assert y.stride(1) == 1
    need = int(lib().w4a4_gemm_a8_workspace_bytes(m, n, k))
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=codes.device)
    _check(lib().w4a4_gemm_a8(_ptr(packed), _ptr(codes), _ptr(scales), _ptr(y), m, n, k, y.stride(0),
                              _ptr(workspace), 0 if workspace is None else workspace.numel(),
                              _stream(codes.device)), "w4a4_gemm_a8")
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
    _require_cuda(w, out)
    assert w.dtype == torch.float32 and w.dim() == 2 and w.stride(1) == 1
    n, k = w.shape
    if out is None:
        out = torch.empty((n, k // 32, 18), dtype=torch.uint8, device=w.device)
    _check(lib().w4a4_quantize_q4_0(_ptr(w), n, k, w.stride(0), _ptr(out), _stream(w.device)), "w4a4_quantize_q4_0")
    return out


def quantize_act(x: torch.Tensor, k: int | None = None, codes: torch.Tensor | None = None,
                 scales: torch.Tensor | None = None):
    """x fp16/fp32 [m, >=k] -> unrotated int4 (codes uint8 [m, k/2], scales fp32 [m, k/32])."""
    _require_cuda(x, codes, scales)
    assert x.dim() == 2 and x.stride(1) == 1
    dt = {torch.float32: DTYPE_F32, torch.float16: DTYPE_F16}.get(x.dtype)
    if dt is None:
        raise W4A4Error(f"unsupported activation dtype {x.dtype}")
    m = x.shape[0]
    k = x.shape[1] if k is None else k
    if codes is None:
        codes = torch.empty((m, k // 2), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty((m, k // 32), dtype=torch.float32, device=x.device)
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
    _require_cuda(q4, out)
    need = int(lib().w4a4_w16_weight_bytes(n, k))
    if out is None:
        out = torch.empty(need // 2, dtype=torch.float16, device=q4.device)
    _check(lib().w4a4_dequantize_w16(_ptr(q4), n, k, _ptr(out), out.numel() * out.element_size(),
                                     _stream(q4.device)), "w4a4_dequantize_w16")
    return out


def rotate_act16(x: torch.Tensor, k: int | None = None, out: torch.Tensor | None = None) -> torch.Tensor:
    """x fp16/fp32 [m, >=k] -> tiled rotated fp16 activations (flat, w4a4_w16_act_bytes(m, k) bytes)."""
    _require_cuda(x, out)
    assert x.dim() == 2 and x.stride(1) == 1
    dt = {torch.float32: DTYPE_F32, torch.float16: DTYPE_F16}.get(x.dtype)
    if dt is None:
        raise W4A4Error(f"unsupported activation dtype {x.dtype}")
    m = x.shape[0]
    k = x.shape[1] if k is None else k
    if out is None:
        out = torch.empty(int(lib().w4a4_w16_act_bytes(m, k)) // 2, dtype=torch.float16, device=x.device)
    _check(lib().w4a4_rotate_act16(_ptr(x), dt, m, k, x.stride(0), _ptr(out), out.numel() * out.element_size(),
                                   _stream(x.device)), "w4a4_rotate_act16")
    return out


def gemm_w16(w16: torch.Tensor, a16: torch.Tensor, m: int, n: int, k: int,
             y: torch.Tensor | None = None) -> torch.Tensor:
    """W4A16 product of the two tiled fp16 operands: fp32 [m, n] (row stride y.stride(0))."""
    _require_cuda(w16, a16, y)
    if y is None:
        y = torch.empty((m, n), dtype=torch.float32, device=a16.device)
    assert y.stride(1) == 1
    _check(lib().w4a4_gemm_w16(_ptr(w16), _ptr(a16), _ptr(y), m, n, k, y.stride(0), _stream(a16.device)),
           "w4a4_gemm_w16")
    return y
