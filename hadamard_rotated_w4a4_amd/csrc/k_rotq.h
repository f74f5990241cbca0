// Activation rotation + int4 quantisation, one pass over the activations.
//
// 1bit-MONSTER engine docs, "The lean option: ROCmFP4, ROCmI4 and Hadamard
// Q4_0", section "Hadamard-rotated Q4_0: W4A4 prompt processing": only the
// activations are rounded to 4 bits, and a 32-point Walsh-Hadamard rotation
// spreads a block's few large values before rounding so they no longer force a
// coarse scale on the rest.  The same per-block rotation was applied to the
// weights offline, so the product is unchanged in exact arithmetic.
//
// Lane mapping: 32 lanes per block, one element per lane, two blocks per
// wave64.  The butterflies exchange across lanes (xor 1, 2, 4, 8, 16 never
// leaves the 32-lane half), the amax is a 5-step xor max, and each lane
// quantises its own element.  The fp32 operation sequence is fixed: IEEE add
// and subtract per stage in the order h = 1, 2, 4, 8, 16, correctly rounded
// division and reciprocal, multiply without contraction, round half away.
#pragma once

#include "common.h"

namespace w4a4 {

constexpr float kInvSqrt32f = 0x1.6a09e6p-3f;  // fp32(1/sqrt(32)), bits 0x3E3504F3

__device__ __forceinline__ float round_half_away(float x) {
    const float t = truncf(x);
    const float frac = fabsf(__fsub_rn(x, t));
    return frac >= 0.5f ? __fadd_rn(t, x < 0.0f ? -1.0f : 1.0f) : t;
}

template <typename T>
__device__ __forceinline__ float load_act(const T *p);
template <>
__device__ __forceinline__ float load_act<float>(const float *p) { return *p; }
template <>
__device__ __forceinline__ float load_act<__half>(const __half *p) { return __half2float(*p); }

template <typename T>
__global__ __launch_bounds__(256) void rotate_quantize_kernel(const T *__restrict__ x, int64_t m,
                                                              int64_t k, int64_t ldx,
                                                              uint8_t *__restrict__ codes,
                                                              float *__restrict__ scales) {
    const int64_t nb = k / QK;
    const int64_t gblk = (int64_t)blockIdx.x * (blockDim.x / QK) + (threadIdx.x / QK);
    if (gblk >= m * nb) return;  // uniform across the 32 lanes of one block
    const int t = threadIdx.x & (QK - 1);
    const int64_t row = gblk / nb, b = gblk % nb;

    float v = load_act<T>(x + row * ldx + b * QK + t);

    // unnormalised FWHT: (a, b) -> (a + b, a - b) for the pair (i, i + h)
#pragma unroll
    for (int h = 1; h < QK; h <<= 1) {
        const float p = __shfl_xor(v, h, QK);
        v = (t & h) ? __fsub_rn(p, v) : __fadd_rn(v, p);
    }

    float amax = fabsf(v);
#pragma unroll
    for (int h = 1; h < QK; h <<= 1) amax = fmaxf(amax, __shfl_xor(amax, h, QK));

    const float d = __fdiv_rn(amax, 7.0f);
    int q = 0;
    float s = 0.0f;
    if (d >= 1.17549435e-38f) {  // FLT_MIN: zero and subnormal scales give a zero block
        const float id = __fdiv_rn(1.0f, d);
        float r = round_half_away(__fmul_rn(v, id));
        r = fminf(7.0f, fmaxf(-7.0f, r));
        q = (int)r;
        s = __fmul_rn(d, kInvSqrt32f);
    }

    // byte j (j < 16) = code j (low nibble) | code j + 16 (high nibble)
    const int hi = __shfl_down(q, 16, QK);
    if (t < 16) {
        codes[row * (k / 2) + b * 16 + t] = (uint8_t)((q & 0xF) | ((hi & 0xF) << 4));
    }
    if (t == 0) scales[row * nb + b] = s;
}

}  // namespace w4a4
