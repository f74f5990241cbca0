"""Second, independent implementation of the activation quantisers -- TEST
INFRASTRUCTURE, used only to pin the C oracle.

The pages print no rounding rule for the activations (1bit-MONSTER engine
docs, page "The lean option: ROCmFP4, ROCmI4 and Hadamard Q4_0", section
"Hadamard-rotated Q4_0: W4A4 prompt processing": the activations alone are
rounded to 4 bits after the per-block rotation).  The oracle fixes one fp32
operation sequence for it (readings R4, R5, R8, R9 and R10 in the header of
oracle/oracle.c), and the GPU is judged bit for bit against that sequence, so
the oracle's C code is checked here against a second implementation of the
same readings written separately: whole arrays of blocks at once in numpy
float32 (every operation one IEEE single-precision rounding), where the C
code walks one block at a time.

  R4   butterflies: stage h = 1, 2, 4, 8, 16; within each run of 2h values the
       first half becomes a + b and the second a - b (a from the first half,
       b from the second);
  R5   amax = max |v|; d = amax / 7; a block with d below the smallest normal
       fp32 is all zeros with scale 0; otherwise id = 1 / d, code =
       clamp(round half away from zero of v * id, -7, 7), scale = d * c32;
  R8   as R5 with 127 in place of 7;
  R9   as R5 without the butterflies, scale = d;
  R10  fp16 of v * c32 (nearest even), v the R4 butterflies.

Rounding half away from zero is taken in float64, where |r| + 1/2 is exact
for every float32 r, instead of the C code's truncate-and-compare.
Nothing here is imported by the product or by the oracle.
"""
from __future__ import annotations

import numpy as np

QK = 32
F32_TINY = np.float32(np.finfo(np.float32).tiny)      # smallest normal float32
C32 = np.float32(1.0 / np.sqrt(np.float64(32.0)))      # 1/sqrt(32) rounded to float32


def blocks_of(x: np.ndarray, k: int | None = None) -> np.ndarray:
    """[m, ldx] fp16/fp32 -> float32 [m * k/32, 32] (fp16 -> fp32 is exact)."""
    m, ldx = x.shape
    k = ldx if k is None else k
    return np.ascontiguousarray(x[:, :k]).astype(np.float32).reshape(m * (k // QK), QK)


def butterflies(v: np.ndarray) -> np.ndarray:
    """R4 on every row of a float32 [B, 32] array."""
    v = np.asarray(v, np.float32)
    nb = v.shape[0]
    h = 1
    while h < QK:
        w = v.reshape(nb, QK // (2 * h), 2, h)
        a, b = w[:, :, 0, :], w[:, :, 1, :]
        v = np.stack([a + b, a - b], axis=2).reshape(nb, QK)
        h *= 2
    return v


def round_half_away(r: np.ndarray) -> np.ndarray:
    r64 = r.astype(np.float64)
    return np.copysign(np.floor(np.abs(r64) + 0.5), r64)


def quantise(v: np.ndarray, qmax: int, fold_c32: bool):
    """Rows of v (float32 [B, 32]) -> (codes int8 [B, 32], scales float32 [B])."""
    amax = np.max(np.abs(v), axis=1)
    d = amax / np.float32(qmax)
    live = d >= F32_TINY
    d_live = np.where(live, d, np.float32(1.0))
    inv = np.float32(1.0) / d_live
    r = v * inv[:, None]
    q = np.clip(round_half_away(r), -qmax, qmax).astype(np.int8)
    q[~live] = 0
    s = (d * C32) if fold_c32 else d
    s = np.where(live, s, np.float32(0.0)).astype(np.float32)
    return q, s


def pack_nibbles(q: np.ndarray, m: int, k: int) -> np.ndarray:
    """int4 codes [m * k/32, 32] -> bytes [m, k/2]: byte j of a block holds code
    j (low nibble) and code j + 16 (high nibble), two's complement."""
    u = (q.astype(np.int16) & 0xF).astype(np.uint8)
    return (u[:, :16] | (u[:, 16:] << 4)).reshape(m, k // 2)


def rotate_quantize_act(x: np.ndarray, k: int | None = None):
    """R4 + R5: (codes uint8 [m, k/2], scales float32 [m, k/32])."""
    m = x.shape[0]
    k = x.shape[1] if k is None else k
    q, s = quantise(butterflies(blocks_of(x, k)), 7, True)
    return pack_nibbles(q, m, k), s.reshape(m, k // QK)


def rotate_quantize_act8(x: np.ndarray, k: int | None = None):
    """R4 + R8: (codes int8 [m, k], scales float32 [m, k/32])."""
    m = x.shape[0]
    k = x.shape[1] if k is None else k
    q, s = quantise(butterflies(blocks_of(x, k)), 127, True)
    return q.reshape(m, k), s.reshape(m, k // QK)


def quantize_act_plain(x: np.ndarray, k: int | None = None):
    """R9: (codes uint8 [m, k/2], scales float32 [m, k/32]), no rotation."""
    m = x.shape[0]
    k = x.shape[1] if k is None else k
    q, s = quantise(blocks_of(x, k), 7, False)
    return pack_nibbles(q, m, k), s.reshape(m, k // QK)


def rotate_act16(x: np.ndarray, k: int | None = None) -> np.ndarray:
    """R4 + R10: float16 [m, k]."""
    m = x.shape[0]
    k = x.shape[1] if k is None else k
    with np.errstate(over="ignore"):  # beyond the fp16 range: inf, as the rounding rule says
        return (butterflies(blocks_of(x, k)) * C32).astype(np.float16).reshape(m, k)
