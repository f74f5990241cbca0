// Activation rotation + int4 quantisation, one pass over the activations.
//
// 1bit-MONSTER engine docs, "The lean option: ROCmFP4, ROCmI4 and Hadamard
// Q4_0", section "Hadamard-rotated Q4_0: W4A4 prompt processing".  The
// weights are 4-bit already; at run time it is the activations that get
// rounded to 4 bits.  Each 32-element block first goes through the 32-point
// Walsh-Hadamard transform that was applied to the weights offline: every
// output mixes all 32 inputs, so one large input no longer decides the
// block's scale on its own, and since the transform is orthogonal, dot
// products of rotated rows equal those of the original rows.
//
// Mapping: four lanes per (row, 32-element block), lane L holding elements
// 8L .. 8L + 7: butterfly stages 1, 2 and 4 run inside the lane, stages 8 and
// 16 exchange values with lane L ^ 1 and L ^ 2 through DPP quad permutes (no
// LDS traffic); the absmax is two more permutes, and each lane then derives
// the block's scale itself.  A wave covers 16 rows of one block, so the
// block's matrix-core operand record (see common.h) is written as coalesced
// 128-byte runs per plane.
//
// The fp32 operation sequence is fixed and the same as a serial evaluation:
// in stage h = 1, 2, 4, 8, 16 each pair (i, i + h) with i & h == 0 becomes
// (v_i + v_{i+h}, v_i - v_{i+h}) with IEEE add and subtract; correctly
// rounded division and reciprocal; multiply without contraction; round half
// away from zero.
#pragma once

#include "common.h"

namespace w4a4 {

constexpr float kInvSqrt32f = 0x1.6a09e6p-3f;  // fp32(1/sqrt(32)), bits 0x3E3504F3

__device__ __forceinline__ float round_half_away(float x) {
    const float t = truncf(x);
    const float frac = fabsf(__fsub_rn(x, t));
    return frac >= 0.5f ? __fadd_rn(t, x < 0.0f ? -1.0f : 1.0f) : t;
}


// Eight consecutive elements as fp32 (exact from fp16).  mode 2: 16-byte
// aligned groups; mode 1: 4-element groups aligned (8 bytes fp16, 16 bytes
// fp32); mode 0: one element at a time.
__device__ __forceinline__ void load8(const float *p, int mode, float v[8]) {
    if (mode > 0) {
        const float4 f0 = reinterpret_cast<const float4 *>(p)[0], f1 = reinterpret_cast<const float4 *>(p)[1];
        v[0] = f0.x; v[1] = f0.y; v[2] = f0.z; v[3] = f0.w;
        v[4] = f1.x; v[5] = f1.y; v[6] = f1.z; v[7] = f1.w;
    } else {
#pragma unroll
        for (int j = 0; j < 8; j++) v[j] = p[j];
    }
}
__device__ __forceinline__ void halves_to_float(uint32_t u, float &lo, float &hi) {
    lo = __half2float(__ushort_as_half((uint16_t)(u & 0xffff)));
    hi = __half2float(__ushort_as_half((uint16_t)(u >> 16)));
}
__device__ __forceinline__ void load8(const __half *p, int mode, float v[8]) {
    if (mode == 2) {
        const uint4 u = *reinterpret_cast<const uint4 *>(p);
        halves_to_float(u.x, v[0], v[1]); halves_to_float(u.y, v[2], v[3]);
        halves_to_float(u.z, v[4], v[5]); halves_to_float(u.w, v[6], v[7]);
    } else if (mode == 1) {
        const uint2 u0 = reinterpret_cast<const uint2 *>(p)[0], u1 = reinterpret_cast<const uint2 *>(p)[1];
        halves_to_float(u0.x, v[0], v[1]); halves_to_float(u0.y, v[2], v[3]);
        halves_to_float(u1.x, v[4], v[5]); halves_to_float(u1.y, v[6], v[7]);
    } else {
#pragma unroll
        for (int j = 0; j < 8; j++) v[j] = __half2float(p[j]);
    }
}

// Value of lane (self ^ 1), (self ^ 2) or (self + 1, clamped) within a quad of
// lanes: DPP quad permutes.
constexpr int QP_XOR1 = 0xB1;  // quad_perm [1, 0, 3, 2]
constexpr int QP_XOR2 = 0x4E;  // quad_perm [2, 3, 0, 1]
constexpr int QP_NEXT = 0xF9;  // quad_perm [1, 2, 3, 3]
template <int CTRL>
__device__ __forceinline__ uint32_t quad_u32(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xF, 0xF, true);
}
template <int CTRL>
__device__ __forceinline__ float quad_f32(float v) {
    return __uint_as_float(quad_u32<CTRL>(__float_as_uint(v)));
}

// The five butterfly stages of one block held by a quad of lanes (lane L:
// elements 8L .. 8L + 7): stages 1, 2, 4 in the lane, 8 and 16 with lane
// L ^ 1, L ^ 2.  Stage h turns each pair (i, i + h) with i & h == 0 into
// (v_i + v_{i+h}, v_i - v_{i+h}).
__device__ __forceinline__ void fwht32_quad(float v[8], int L) {
#pragma unroll
    for (int h = 1; h < 8; h <<= 1) {
#pragma unroll
        for (int i = 0; i < 8; i++) {
            if (i & h) continue;
            const float a0 = v[i], a1 = v[i + h];
            v[i] = __fadd_rn(a0, a1);
            v[i + h] = __fsub_rn(a0, a1);
        }
    }
    {
        const bool upper = L & 1;
#pragma unroll
        for (int i = 0; i < 8; i++) {
            const float p = quad_f32<QP_XOR1>(v[i]);
            v[i] = upper ? __fsub_rn(p, v[i]) : __fadd_rn(v[i], p);  // (lower - upper) / (lower + upper)
        }
    }
    {
        const bool upper = L & 2;
#pragma unroll
        for (int i = 0; i < 8; i++) {
            const float p = quad_f32<QP_XOR2>(v[i]);
            v[i] = upper ? __fsub_rn(p, v[i]) : __fadd_rn(v[i], p);
        }
    }
}

// One (row, block) of the quantiser, held by a quad of lanes (lane L of the
// quad: elements 8L .. 8L + 7 at src): the butterflies (unless ROTATE is
// false), the absmax, the scale s and this lane's 8 codes.  live: the row
// and block exist (uniform per quad; a dead quad quantises zeros).  Every
// lane of the quad must take part (the butterflies and the absmax exchange
// values through quad permutes).
template <typename T, int QMAX, bool ROTATE>
__device__ __forceinline__ void quantise_quad(const T *src, int mode, bool live, int L, int q[8], float &s) {
    float v[8];
    if (live) {
        load8(src, mode, v);
    } else {
#pragma unroll
        for (int t = 0; t < 8; t++) v[t] = 0.0f;
    }
    if constexpr (ROTATE) fwht32_quad(v, L);

    float amax = 0.0f;
#pragma unroll
    for (int t = 0; t < 8; t++) amax = fmaxf(amax, fabsf(v[t]));
    amax = fmaxf(amax, quad_f32<QP_XOR1>(amax));
    amax = fmaxf(amax, quad_f32<QP_XOR2>(amax));

    const float d = __fdiv_rn(amax, (float)QMAX);
    const bool nonzero = d >= 1.17549435e-38f;  // FLT_MIN: zero and subnormal scales give a zero block
    const float id = nonzero ? __fdiv_rn(1.0f, d) : 0.0f;
    s = !nonzero ? 0.0f : ROTATE ? __fmul_rn(d, kInvSqrt32f) : d;
#pragma unroll
    for (int t = 0; t < 8; t++)
        q[t] = nonzero ? (int)fminf((float)QMAX, fmaxf(-(float)QMAX, round_half_away(__fmul_rn(v[t], id)))) : 0;
}

// The public int4 codes of a block (byte j = code j | code j + 16 << 4) from
// its quad: lane L < 2 writes bytes 8L .. 8L + 7 (its codes and those of lane
// L + 2), lane 0 the scale.  Every lane of the quad must take part.
// COHERENT: device-scope stores (written through to where every compute unit
// of the device reads them), for readers in the same launch.
template <bool COHERENT = false>
__device__ __forceinline__ void store_codes4(const int q[8], float s, int L, bool live, uint8_t *blk_codes,
                                             float *blk_scale) {
    uint32_t nib0 = 0, nib1 = 0;  // this lane's 8 codes, one nibble each, in byte positions
#pragma unroll
    for (int i = 0; i < 4; i++) {
        nib0 |= (uint32_t)(q[i] & 0xF) << (8 * i);
        nib1 |= (uint32_t)(q[4 + i] & 0xF) << (8 * i);
    }
    const uint32_t hi0 = quad_u32<QP_XOR2>(nib0), hi1 = quad_u32<QP_XOR2>(nib1);
    if (live && L < 2) {
        const uint32_t lo = nib0 | hi0 << 4, hi = nib1 | hi1 << 4;
        if constexpr (COHERENT) {
            __hip_atomic_store(reinterpret_cast<uint64_t *>(blk_codes + 8 * L), (uint64_t)hi << 32 | lo,
                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (L == 0)
                __hip_atomic_store(reinterpret_cast<uint32_t *>(blk_scale), __float_as_uint(s), __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
        } else {
            *reinterpret_cast<uint2 *>(blk_codes + 8 * L) = make_uint2(lo, hi);
            if (L == 0) *blk_scale = s;
        }
    }
}

// Row r of a block's operand record (see common.h) from the quad that holds
// the row: its 32 codes as one 192-bit string of fp6 fields, lane L's 8 codes
// (fields f) at bit 48 L; lanes 0, 1, 2 write 64-bit parts 0, 1, 2 of the
// string, lane 3 the scale operand `sop`.  Every lane of the quad must take
// part (the parts cross lanes through a quad permute).
__device__ __forceinline__ void put_quad_row(const uint32_t f[8], int L, uint8_t *rec, int r, uint2 sop) {
    uint64_t mine = 0;
#pragma unroll
    for (int t = 0; t < 8; t++) mine |= (uint64_t)f[t] << (6 * t);
    const uint64_t next = (uint64_t)quad_u32<QP_NEXT>((uint32_t)mine) |
                          (uint64_t)quad_u32<QP_NEXT>((uint32_t)(mine >> 32)) << 32;
    if (L < 3) {
        const uint64_t part = L == 0 ? (mine | next << 48) : L == 1 ? (mine >> 16 | next << 32) : (mine >> 32 | next << 16);
        reinterpret_cast<uint2 *>(rec + 256 * L)[r] = make_uint2((uint32_t)part, (uint32_t)(part >> 32));
    } else {
        reinterpret_cast<uint2 *>(rec + MX_CODE_BYTES)[r] = sop;
    }
}

// One workgroup = 32 rows (row tile blockIdx.y) x 2 neighbouring blocks
// (2 blockIdx.x and 2 blockIdx.x + 1), four lanes per (row, block): wave w
// takes block w / 2 and rows 16 (w % 2) .. + 15, lane 4 i + L row i, elements
// 8L .. 8L + 7.  With `act` set, also writes the blocks' operand records for
// the matrix-core GEMM (the blocks then run over the padded block count;
// padding rows and blocks get zero records).
//
// QMAX = 7: int4 codes (W4A4).  QMAX = 127: int8 codes for the exact int8
// path on a rotated file (W4A8), one signed byte per element in `codes`
// ([m][k]), same rotation, d = amax / 127; with `act` set, the operand
// records of the int8 matrix-core product, two planes per row tile
// ([row tile][plane][padded block][1 KB]): every code a = 16 h + l with
// h = (a + 8) >> 4, plane 0 the h codes and the scale operand, plane 1 the l
// codes and a zero scale operand.
// ROTATE = false: the unrotated W4A4 ablation (section "MoE: W4A4 on the
// experts"): no butterflies, and the stored scale is d itself (there is no
// normalisation to fold in).
// With `sma` set (W4A4, m <= 16): also the record-ordered operand of the
// m <= 16 product (common.h); the blocks then run over whole quads, and rows
// m .. 15 and blocks past nb get zero codes and scales.
constexpr int RQ_BLOCKS = 2;  // blocks per workgroup
template <typename T, int QMAX = 7, bool ROTATE = true>
__global__ __launch_bounds__(128 * RQ_BLOCKS) void rotate_quantize_kernel(const T *__restrict__ x, int64_t m,
                                                                          int64_t k, int64_t ldx, int mode,
                                                                          uint8_t *__restrict__ codes,
                                                                          float *__restrict__ scales,
                                                                          uint8_t *__restrict__ act,
                                                                          uint8_t *__restrict__ sma = nullptr) {
    static_assert(QMAX == 7 || QMAX == 127, "int4 or int8 codes");
    const int64_t nb = k / QK;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, L = lane & 3;
    const int r = (wave & 1) * 16 + (lane >> 2);  // row within the tile
    const int64_t b = (int64_t)blockIdx.x * RQ_BLOCKS + (wave >> 1), row = (int64_t)blockIdx.y * 32 + r;
    const bool live = row < m && b < nb;  // uniform per quad

    int q[8];
    float s;
    quantise_quad<T, QMAX, ROTATE>(x + row * ldx + b * QK + 8 * L, mode, live, L, q, s);

    if constexpr (QMAX == 127) {  // int8 codes: lane L writes elements 8L .. 8L + 7
        if (live) {
            uint32_t w0 = 0, w1 = 0;
#pragma unroll
            for (int i = 0; i < 4; i++) {
                w0 |= (uint32_t)(q[i] & 0xFF) << (8 * i);
                w1 |= (uint32_t)(q[4 + i] & 0xFF) << (8 * i);
            }
            *reinterpret_cast<uint2 *>(codes + row * k + b * QK + 8 * L) = make_uint2(w0, w1);
            if (L == 0) scales[row * nb + b] = s;
        }
        if (act && b < mx_blocks(k)) {
            uint32_t fh[8], fl[8];
#pragma unroll
            for (int t = 0; t < 8; t++) {
                const int h = (q[t] + 8) >> 4;  // floor: h in [-8, 8], q - 16 h in [-8, 7]
                fh[t] = fp6_e2m3_of(h);
                fl[t] = fp6_e2m3_of(q[t] - 16 * h);
            }
            uint8_t *rec = act + ((int64_t)blockIdx.y * 2 * mx_blocks(k) + b) * MX_REC;
            put_quad_row(fh, L, rec, r, act_scale_operand(s));
            put_quad_row(fl, L, rec + mx_blocks(k) * MX_REC, r, make_uint2(0, 0));
        }
        return;
    }

    if (codes) store_codes4(q, s, L, live, codes + row * (k / 2) + b * 16, scales + row * nb + b);

    if (sma && row < SMA_ROWS && b < sq_quads(k) * SQ_BLOCKS) {  // uniform per quad
        const int64_t qd = b / SQ_BLOCKS;
        const int j = (int)(b % SQ_BLOCKS);
        store_codes4(q, s, L, true, sma + qd * SMA_CODE_BYTES + row * 64 + j * 16,
                     reinterpret_cast<float *>(sma + sq_quads(k) * SMA_CODE_BYTES + qd * SMA_SCALE_BYTES +
                                               row * 16 + j * 4));
    }

    if (act && b < mx_blocks(k)) {  // the operand record of (row tile, block)
        uint32_t f[8];
#pragma unroll
        for (int t = 0; t < 8; t++) f[t] = fp6_e2m3_of(q[t]);
        put_quad_row(f, L, act + ((int64_t)blockIdx.y * mx_blocks(k) + b) * MX_REC, r, act_scale_operand(s));
    }
}

}  // namespace w4a4
