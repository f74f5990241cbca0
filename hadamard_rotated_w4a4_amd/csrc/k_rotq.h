// Activation rotation + int4 quantisation, one pass over the activations.
//
// 1bit-MONSTER engine docs, "The lean option: ROCmFP4, ROCmI4 and Hadamard
// Q4_0", section "Hadamard-rotated Q4_0: W4A4 prompt processing": only the
// activations are rounded to 4 bits, and a 32-point Walsh-Hadamard rotation
// spreads a block's few large values before rounding so they no longer force a
// coarse scale on the rest.  The same per-block rotation was applied to the
// weights offline, so the product is unchanged in exact arithmetic.
//
// Mapping: eight lanes per 32-element block, four consecutive elements per
// lane (one 8-byte fp16 load).  The butterflies of distance 1 and 2 are
// in-lane, those of distance 4, 8 and 16 exchange values with lane L ^ 1,
// L ^ 2, L ^ 4 of the block's eight; the absmax is a three-step exchange too.
// A workgroup of 512 threads covers 32 rows of two neighbouring blocks: each
// row's two blocks are one 128-byte line of fp16 input, read by one
// workgroup (with one block per workgroup, neighbouring workgroups land on
// different XCDs and both fetch the line), and each half writes its block's
// matrix-core operand record (see common.h) in one coalesced kilobyte.
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

// value of lane (self ^ mask) within the 8-lane group of a block
__device__ __forceinline__ float xchg(float v, int mask) { return __shfl_xor(v, mask, 8); }
__device__ __forceinline__ uint32_t xchg(uint32_t v, int mask) { return (uint32_t)__shfl_xor((int)v, mask, 8); }

// Four consecutive elements as fp32 (exact from fp16).
__device__ __forceinline__ void load4(const float *p, bool vec, float v[4]) {
    if (vec) {
        const float4 f = *reinterpret_cast<const float4 *>(p);
        v[0] = f.x; v[1] = f.y; v[2] = f.z; v[3] = f.w;
    } else {
        for (int i = 0; i < 4; i++) v[i] = p[i];
    }
}
__device__ __forceinline__ void load4(const __half *p, bool vec, float v[4]) {
    if (vec) {
        const uint2 u = *reinterpret_cast<const uint2 *>(p);
        v[0] = __half2float(__ushort_as_half((uint16_t)(u.x & 0xffff)));
        v[1] = __half2float(__ushort_as_half((uint16_t)(u.x >> 16)));
        v[2] = __half2float(__ushort_as_half((uint16_t)(u.y & 0xffff)));
        v[3] = __half2float(__ushort_as_half((uint16_t)(u.y >> 16)));
    } else {
        for (int i = 0; i < 4; i++) v[i] = __half2float(p[i]);
    }
}

// One workgroup = 32 rows (row tile blockIdx.y) x two 32-element blocks
// (2 blockIdx.x and 2 blockIdx.x + 1); thread t: block half t / 256, row
// r = (t / 8) % 32 of the tile, lane L = t % 8 of the block, elements
// 4L .. 4L + 3.  `vec`: every 4-element group is aligned for one vector load
// (checked on the host).  With `act` set, also writes the block's operand
// record for the matrix-core GEMM (the blocks then run over the padded block
// count, an even number; padding rows and blocks get zero records).
//
// QMAX = 7: int4 codes (W4A4).  QMAX = 127: int8 codes for the exact int8
// path on a rotated file (W4A8), one signed byte per element in `codes`
// ([m][k]), same rotation, d = amax / 127; no operand record.
// ROTATE = false: the unrotated W4A4 ablation (section "MoE: W4A4 on the
// experts"): no butterflies, and the stored scale is d itself (there is no
// normalisation to fold in).
constexpr int RQ_BLOCKS = 2;  // blocks per workgroup
template <typename T, int QMAX = 7, bool ROTATE = true>
__global__ __launch_bounds__(256 * RQ_BLOCKS) void rotate_quantize_kernel(const T *__restrict__ x, int64_t m,
                                                                          int64_t k, int64_t ldx, bool vec,
                                                                          uint8_t *__restrict__ codes,
                                                                          float *__restrict__ scales,
                                                                          uint8_t *__restrict__ act) {
    static_assert(QMAX == 7 || QMAX == 127, "int4 or int8 codes");
    const int64_t nb = k / QK;
    const int tid = threadIdx.x, L = tid & 7, r = (tid >> 3) & 31;
    const int64_t b = (int64_t)blockIdx.x * RQ_BLOCKS + (tid >> 8), row = (int64_t)blockIdx.y * 32 + r;
    const bool live = row < m && b < nb;  // uniform per 8-lane group

    float v[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    if (live) load4(x + row * ldx + b * QK + 4 * L, vec, v);

    if constexpr (ROTATE) {
        // distance 1 and 2: inside the lane
        {
            const float a0 = v[0], a1 = v[1], a2 = v[2], a3 = v[3];
            v[0] = __fadd_rn(a0, a1); v[1] = __fsub_rn(a0, a1);
            v[2] = __fadd_rn(a2, a3); v[3] = __fsub_rn(a2, a3);
        }
        {
            const float a0 = v[0], a1 = v[1], a2 = v[2], a3 = v[3];
            v[0] = __fadd_rn(a0, a2); v[2] = __fsub_rn(a0, a2);
            v[1] = __fadd_rn(a1, a3); v[3] = __fsub_rn(a1, a3);
        }
        // distance 4, 8, 16: partner lane L ^ 1, L ^ 2, L ^ 4 holds the other element
#pragma unroll
        for (int mask = 1; mask < 8; mask <<= 1) {
            const bool upper = (L & mask) != 0;
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const float p = xchg(v[i], mask);
                v[i] = upper ? __fsub_rn(p, v[i]) : __fadd_rn(v[i], p);  // (lower - upper) / (lower + upper)
            }
        }
    }

    float amax = fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3])));
#pragma unroll
    for (int mask = 1; mask < 8; mask <<= 1) amax = fmaxf(amax, xchg(amax, mask));

    const float d = __fdiv_rn(amax, (float)QMAX);
    const bool nonzero = d >= 1.17549435e-38f;  // FLT_MIN: zero and subnormal scales give a zero block
    const float id = nonzero ? __fdiv_rn(1.0f, d) : 0.0f;
    const float s = !nonzero ? 0.0f : ROTATE ? __fmul_rn(d, kInvSqrt32f) : d;
    int q[4];
#pragma unroll
    for (int i = 0; i < 4; i++)
        q[i] = nonzero ? (int)fminf((float)QMAX, fmaxf(-(float)QMAX, round_half_away(__fmul_rn(v[i], id)))) : 0;

    if constexpr (QMAX == 127) {  // int8 codes: lane L writes elements 4L .. 4L + 3
        if (live) {
            const uint32_t word = (uint32_t)(q[0] & 0xFF) | (uint32_t)(q[1] & 0xFF) << 8 |
                                  (uint32_t)(q[2] & 0xFF) << 16 | (uint32_t)(q[3] & 0xFF) << 24;
            reinterpret_cast<uint32_t *>(codes + row * k + b * QK)[L] = word;
            if (L == 0) scales[row * nb + b] = s;
        }
        return;
    }

    // public codes: byte j = code j | code j + 16 << 4; lane L < 4 writes bytes 4L .. 4L + 3
    const uint32_t mine = (q[0] & 0xF) | (q[1] & 0xF) << 4 | (q[2] & 0xF) << 8 | (q[3] & 0xF) << 12;
    const uint32_t high = xchg(mine, 4);  // codes 16 + 4L .. of lane L + 4
    if (live && b < nb && codes) {
        if (L < 4) {
            uint32_t word = 0;
#pragma unroll
            for (int i = 0; i < 4; i++) word |= (((mine >> (4 * i)) & 0xF) | ((high >> (4 * i)) & 0xF) << 4) << (8 * i);
            reinterpret_cast<uint32_t *>(codes + row * (k / 2) + b * 16)[L] = word;
        }
        if (L == 0) scales[row * nb + b] = s;
    }

    if (act && b < mx_blocks(k)) {
        // operand record of (row tile, block): row r's 32 codes are one 192-bit
        // string of fp6 fields; this thread's four codes are its 24 bits at
        // bit 24 L.  Lanes 0, 3 and 6 write the planes (bits 64 p .. 64 p + 63).
        uint32_t f24 = 0;
#pragma unroll
        for (int i = 0; i < 4; i++) f24 |= fp6_e2m3_of(live ? q[i] : 0) << (6 * i);
        const uint32_t n1 = (uint32_t)__shfl_down((int)f24, 1, 8), n2 = (uint32_t)__shfl_down((int)f24, 2, 8);
        const uint32_t p1 = (uint32_t)__shfl_up((int)f24, 1, 8);  // lanes L + 1, L + 2, L - 1
        uint8_t *rec = act + ((int64_t)blockIdx.y * mx_blocks(k) + b) * MX_REC;
        if (L == 0) reinterpret_cast<uint2 *>(rec)[r] = make_uint2(f24 | n1 << 24, n1 >> 8 | n2 << 16);
        if (L == 3) reinterpret_cast<uint2 *>(rec + 256)[r] = make_uint2(p1 >> 16 | f24 << 8, n1 | n2 << 24);
        if (L == 6) reinterpret_cast<uint2 *>(rec + 512)[r] = make_uint2(p1 >> 8 | f24 << 16, f24 >> 16 | n1 << 8);
        if (L == 0) {
            // exact bf16 split s = s1 + s2 + s3 (truncations; each remainder is exact)
            const float sl = live ? s : 0.0f;
            const uint32_t h1 = __float_as_uint(sl) & 0xFFFF0000u;
            const float r1 = __fsub_rn(sl, __uint_as_float(h1));
            const uint32_t h2 = __float_as_uint(r1) & 0xFFFF0000u;
            const float r2 = __fsub_rn(r1, __uint_as_float(h2));
            const uint32_t h3 = __float_as_uint(r2) & 0xFFFF0000u;
            reinterpret_cast<uint2 *>(rec + MX_CODE_BYTES)[r] = make_uint2((h1 >> 16) | h2, h3 >> 16);
        }
    }
}

}  // namespace w4a4
