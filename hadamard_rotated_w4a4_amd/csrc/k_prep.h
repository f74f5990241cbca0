// Offline weight preparation and the one-time repack.
//
// 1bit-MONSTER engine docs, "The lean option: ROCmFP4, ROCmI4 and Hadamard
// Q4_0", section "Hadamard-rotated Q4_0: W4A4 prompt processing": the weights
// are rotated once by the 32-point Walsh-Hadamard transform per 32-element
// block along K and quantised to plain Q4_0; the W4A4 kernel reads the Q4_0
// codes bit for bit, using that q ^ 8 read as a signed nibble is q - 8.
#pragma once

#include "common.h"

namespace w4a4 {

// fp64(1/sqrt(32)) correctly rounded (= fp64(sqrt(2)) / 8).
__device__ constexpr double kInvSqrt32d = 0.17677669529663688110021109052621763;

// One thread per 32-element block: rotate in fp64, round to fp32, quantise to
// Q4_0.  ROTATE = false: plain Q4_0 of the unrotated block (the weights of the
// unrotated W4A4 ablation, section "MoE: W4A4 on the experts").
template <bool ROTATE = true>
__global__ __launch_bounds__(256) void quantize_q4_0_h32_kernel(const float *__restrict__ w,
                                                                 int64_t n, int64_t k, int64_t ldw,
                                                                 uint8_t *__restrict__ q4) {
    const int64_t nb = k / QK;
    const int64_t blk = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (blk >= n * nb) return;
    const int64_t row = blk / nb, b = blk % nb;
    const float *src = w + row * ldw + b * QK;

    float x[QK];
#pragma unroll
    for (int j = 0; j < QK; j++) x[j] = src[j];

    float r[QK];
    float amax = 0.0f, mx = 0.0f;
#pragma unroll
    for (int t = 0; t < QK; t++) {
        if constexpr (ROTATE) {
            double u = 0.0;
#pragma unroll
            for (int j = 0; j < QK; j++) {
                // H[t][j] = (-1)^popcount(t & j); adding +-x_j is exact per term
                const bool neg = __builtin_popcount((unsigned)(t & j)) & 1;
                u = __dadd_rn(u, neg ? -(double)x[j] : (double)x[j]);
            }
            r[t] = (float)__dmul_rn(u, kInvSqrt32d);
        } else {
            r[t] = x[t];
        }
        const float a = fabsf(r[t]);
        if (a > amax) { amax = a; mx = r[t]; }
    }
    const float d = __fdiv_rn(mx, -8.0f);
    const float id = d != 0.0f ? __fdiv_rn(1.0f, d) : 0.0f;
    const __half dh = __float2half_rn(opaque(d));  // keeps the sign of a zero scale
    uint8_t *dst = q4 + blk * 18;
    const uint16_t dbits = __half_as_ushort(dh);
    dst[0] = (uint8_t)(dbits & 0xff);
    dst[1] = (uint8_t)(dbits >> 8);
#pragma unroll
    for (int j = 0; j < QK / 2; j++) {
        int q0 = (int)__fadd_rn(__fmul_rn(r[j], id), 8.5f);
        int q1 = (int)__fadd_rn(__fmul_rn(r[j + 16], id), 8.5f);
        q0 = q0 > 15 ? 15 : q0;
        q1 = q1 > 15 ? 15 : q1;
        dst[2 + j] = (uint8_t)(q0 | (q1 << 4));
    }
}

// Matrix-core operand records (see common.h), one thread per (tile, padded
// block, column).  Padding columns and blocks get zero codes and zero scales.
__global__ __launch_bounds__(256) void repack_mx_kernel(const uint8_t *__restrict__ q4, int64_t n,
                                                        int64_t k, uint8_t *__restrict__ packed) {
    const int64_t nb = k / QK, nbp = mx_blocks(k);
    const int64_t tiles = padded_n(n) / TILE_N;
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (gid >= tiles * nbp * 32) return;
    const int c = (int)(gid & 31);
    const int64_t tb = gid >> 5;  // tile * nbp + b
    const int64_t tile = tb / nbp, b = tb % nbp;
    const int64_t col = tile * TILE_N + c;
    uint32_t w[6] = {0, 0, 0, 0, 0, 0};
    uint32_t sw = 0;
    if (col < n && b < nb) {
        const uint8_t *blk = q4 + (col * nb + b) * 18;
        uint32_t f[32];
        for (int j = 0; j < 16; j++) {
            f[j] = fp6_e2m3_of((int)(blk[2 + j] & 0xF) - 8);        // code j
            f[j + 16] = fp6_e2m3_of((int)(blk[2 + j] >> 4) - 8);    // code j + 16
        }
        pack_fp6x32(f, w);
        // 64 * d: the MFMA reads codes as q / 8
        sw = weight_scale_operand(__half2float(__ushort_as_half((uint16_t)(blk[0] | (blk[1] << 8)))) * 64.0f);
    }
    uint8_t *rec = packed + tb * MX_REC;
    put_mx_row(rec, c, w);
    reinterpret_cast<uint32_t *>(rec + MX_CODE_BYTES)[c] = sw;
    reinterpret_cast<uint32_t *>(rec + MX_CODE_BYTES)[32 + c] = 0;  // unused tail of the record
}

// Streaming records (see common.h), one thread per (tile, padded block,
// column).
__global__ __launch_bounds__(256) void repack_sq_kernel(const uint8_t *__restrict__ q4, int64_t n,
                                                        int64_t k, uint8_t *__restrict__ packed) {
    const int64_t nb = k / QK, nq = sq_quads(k);
    const int64_t tiles = padded_n(n) / TILE_N;
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (gid >= tiles * nq * SQ_BLOCKS * 32) return;
    const int c = (int)(gid & 31);
    const int64_t tb = gid >> 5;  // tile * 4 nq + padded block
    const int64_t tile = tb / (nq * SQ_BLOCKS), b = tb % (nq * SQ_BLOCKS);
    const int64_t col = tile * TILE_N + c;
    uint4 w = make_uint4(0, 0, 0, 0);
    uint16_t dbits = 0;
    if (col < n && b < nb) {
        const uint8_t *blk = q4 + (col * nb + b) * 18;
        uint32_t u[4];
        for (int i = 0; i < 4; i++)
            u[i] = ((uint32_t)blk[2 + 4 * i] | (uint32_t)blk[3 + 4 * i] << 8 | (uint32_t)blk[4 + 4 * i] << 16 |
                    (uint32_t)blk[5 + 4 * i] << 24) ^ 0x88888888u;  // q ^ 8: signed nibble q - 8
        w = k8_words(make_uint4(u[0], u[1], u[2], u[3]));
        dbits = (uint16_t)(blk[0] | (blk[1] << 8));
    }
    uint8_t *rec = packed + sq_section_offset(n, k) + (tile * nq + b / SQ_BLOCKS) * SQ_REC;
    const int j = (int)(b % SQ_BLOCKS);
    // word w goes to lane 32 (w / 2) + c, at 8 (j % 2) + 4 (w % 2) of its 16 B
    // in the half (j / 2) of the record
    const uint32_t words[4] = {w.x, w.y, w.z, w.w};
    for (int wd = 0; wd < 4; wd++)
        *reinterpret_cast<uint32_t *>(rec + (j >> 1) * 1024 + (32 * (wd >> 1) + c) * 16 + (j & 1) * 8 + (wd & 1) * 4) =
            words[wd];
    // d goes to lane 32 (j % 2) + c, low half for blocks 0 and 1, high for 2 and 3
    reinterpret_cast<uint16_t *>(rec + SQ_SCALE_OFF + (32 * (j & 1) + c) * 4)[j >> 1] = dbits;
}

}  // namespace w4a4
