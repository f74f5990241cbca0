// Activation rotation + int4 quantisation, one pass over the activations.
//
// 1bit-MONSTER engine docs, "The lean option: ROCmFP4, ROCmI4 and Hadamard
// Q4_0", section "Hadamard-rotated Q4_0: W4A4 prompt processing": only the
// activations are rounded to 4 bits, and a 32-point Walsh-Hadamard rotation
// spreads a block's few large values before rounding so they no longer force a
// coarse scale on the rest.  The same per-block rotation was applied to the
// weights offline, so the product is unchanged in exact arithmetic.
//
// Mapping: one thread per 32-element block, the whole transform in registers
// (the pass is a single read of the activations and is bound by memory and
// launch latency, not arithmetic).  The fp32 operation sequence is fixed:
// IEEE add and subtract per stage in the order h = 1, 2, 4, 8, 16, correctly
// rounded division and reciprocal, multiply without contraction, round half
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

// Load the 32 elements of one block as fp32 (exact from fp16).
__device__ __forceinline__ void load_block(const float *__restrict__ p, float v[QK]) {
    const float4 *q = reinterpret_cast<const float4 *>(p);
#pragma unroll
    for (int i = 0; i < QK / 4; i++) {
        const float4 f = q[i];
        v[4 * i] = f.x; v[4 * i + 1] = f.y; v[4 * i + 2] = f.z; v[4 * i + 3] = f.w;
    }
}
__device__ __forceinline__ void load_block(const __half *__restrict__ p, float v[QK]) {
    const uint4 *q = reinterpret_cast<const uint4 *>(p);
#pragma unroll
    for (int i = 0; i < QK / 8; i++) {
        const uint4 u = q[i];
        const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int j = 0; j < 4; j++) {
            v[8 * i + 2 * j] = __half2float(__ushort_as_half((uint16_t)(w[j] & 0xffff)));
            v[8 * i + 2 * j + 1] = __half2float(__ushort_as_half((uint16_t)(w[j] >> 16)));
        }
    }
}

// One thread per 32-element block, all in registers: unnormalised FWHT,
// amax, scale, codes, packing.  Loads are 16-byte vectors when the row stride
// and base keep every block 16-byte aligned (checked on the host); the
// element-wise variant below covers any other stride.
template <typename T, bool VEC>
__global__ __launch_bounds__(256) void rotate_quantize_kernel(const T *__restrict__ x, int64_t m,
                                                              int64_t k, int64_t ldx,
                                                              uint8_t *__restrict__ codes,
                                                              float *__restrict__ scales) {
    const int64_t nb = k / QK;
    const int64_t blk = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (blk >= m * nb) return;
    const int64_t row = blk / nb, b = blk % nb;
    const T *src = x + row * ldx + b * QK;

    float v[QK];
    if constexpr (VEC) {
        load_block(src, v);
    } else {
#pragma unroll
        for (int t = 0; t < QK; t++) {
            if constexpr (sizeof(T) == 4) v[t] = src[t];
            else v[t] = __half2float(src[t]);
        }
    }

    // (a, b) -> (a + b, a - b) for the pair (i, i + h), h = 1, 2, 4, 8, 16
#pragma unroll
    for (int h = 1; h < QK; h <<= 1) {
#pragma unroll
        for (int i = 0; i < QK; i++) {
            if (i & h) continue;
            const float a0 = v[i], a1 = v[i + h];
            v[i] = __fadd_rn(a0, a1);
            v[i + h] = __fsub_rn(a0, a1);
        }
    }

    float amax = 0.0f;
#pragma unroll
    for (int t = 0; t < QK; t++) amax = fmaxf(amax, fabsf(v[t]));

    const float d = __fdiv_rn(amax, 7.0f);
    uint32_t packed[4] = {0u, 0u, 0u, 0u};
    float s = 0.0f;
    if (d >= 1.17549435e-38f) {  // FLT_MIN: zero and subnormal scales give a zero block
        const float id = __fdiv_rn(1.0f, d);
#pragma unroll
        for (int j = 0; j < QK / 2; j++) {
            const float r0 = fminf(7.0f, fmaxf(-7.0f, round_half_away(__fmul_rn(v[j], id))));
            const float r1 = fminf(7.0f, fmaxf(-7.0f, round_half_away(__fmul_rn(v[j + 16], id))));
            const uint32_t byte = ((uint32_t)(int)r0 & 0xFu) | (((uint32_t)(int)r1 & 0xFu) << 4);
            packed[j >> 2] |= byte << (8 * (j & 3));
        }
        s = __fmul_rn(d, kInvSqrt32f);
    }
    // byte j of the block: code j (low nibble) | code j + 16 (high nibble)
    *reinterpret_cast<uint4 *>(codes + row * (k / 2) + b * 16) =
        make_uint4(packed[0], packed[1], packed[2], packed[3]);
    scales[row * nb + b] = s;
}

}  // namespace w4a4
