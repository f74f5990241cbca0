// Rotated W4A16: the rotated Q4_0 file with its activations rotated but not
// rounded to 4 bits.
//
// 1bit-MONSTER engine docs, "The lean option: ROCmFP4, ROCmI4 and Hadamard
// Q4_0", section "Hadamard-rotated Q4_0: W4A4 prompt processing": the same
// rotated files also run on a route where the activations are rotated (as a
// matmul) and stay at 16 bits, with no W4A4.
//
// On the matrix cores this is a plain fp16 GEMM: the activations rotated as
// for W4A4 and rounded to fp16 once, the Q4_0 weights dequantised to
// fp16(d * (q - 8)) once (the block scale folded into the weight, so no
// per-block epilogue remains), and v_mfma_f32_32x32x16_f16 accumulating in
// its own registers.  Both operands are row-major fp16 matrices padded with
// zeros to whole 32-row tiles and to the padded block count (a multiple of
// MX_BLOCK_PAD blocks): the global-to-LDS loads gather each MFMA fragment
// straight from the rows and never read past a buffer.
#pragma once

#include "common.h"
#include "k_dense.h"
#include "k_rotq.h"

namespace w4a4 {

typedef _Float16 v8h __attribute__((ext_vector_type(8)));

// Row stride (elements) of both padded fp16 operands.
__host__ __device__ inline int64_t w16_row_stride(int64_t k) { return mx_blocks(k) * QK; }

// ---------------------------------------------------------------------------
// Operands
// ---------------------------------------------------------------------------
// Weights: one thread per (padded row, padded block): fp16(d * (q - 8)) for
// the 32 elements, zeros past n and past the last block.  The fp32 product
// of an fp16 scale and a 4-bit integer is exact; it is still kept apart from
// the conversion, since the fused form the compiler would pick
// (v_fma_mixlo_f16, d * q + 0) turns the -0 of a negative scale times a
// zero code into +0.
__global__ __launch_bounds__(256) void dequantize_w16_kernel(const uint8_t *__restrict__ q4, int64_t n, int64_t k,
                                                             _Float16 *__restrict__ w16) {
    const int64_t nb = k / QK, nbp = mx_blocks(k), rows = padded_n(n);
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (gid >= rows * nbp) return;
    const int64_t row = gid / nbp, b = gid % nbp;
    uint32_t h[16];
    if (row < n && b < nb) {
        const uint8_t *blk = q4 + (row * nb + b) * 18;
        const float d = __half2float(__ushort_as_half((uint16_t)(blk[0] | (blk[1] << 8))));
#pragma unroll
        for (int j = 0; j < 16; j += 2) {
            // elements j, j + 1 (low nibbles) and j + 16, j + 17 (high nibbles)
            float e0 = __fmul_rn(d, (float)((int)(blk[2 + j] & 0xF) - 8));
            float e1 = __fmul_rn(d, (float)((int)(blk[3 + j] & 0xF) - 8));
            float e2 = __fmul_rn(d, (float)((int)(blk[2 + j] >> 4) - 8));
            float e3 = __fmul_rn(d, (float)((int)(blk[3 + j] >> 4) - 8));
            asm volatile("" : "+v"(e0), "+v"(e1), "+v"(e2), "+v"(e3));
            h[j / 2] = (uint32_t)__half_as_ushort(__float2half_rn(e0)) | (uint32_t)__half_as_ushort(__float2half_rn(e1)) << 16;
            h[8 + j / 2] = (uint32_t)__half_as_ushort(__float2half_rn(e2)) | (uint32_t)__half_as_ushort(__float2half_rn(e3)) << 16;
        }
    } else {
#pragma unroll
        for (int j = 0; j < 16; j++) h[j] = 0;
    }
    uint4 *dst = reinterpret_cast<uint4 *>(w16 + row * w16_row_stride(k) + b * QK);
#pragma unroll
    for (int j = 0; j < 4; j++) dst[j] = make_uint4(h[4 * j], h[4 * j + 1], h[4 * j + 2], h[4 * j + 3]);
}

// Activations: as rotate_quantize_kernel's mapping (four lanes per (row,
// block)), the butterflies, then fp16(fl(v * c32)); zeros past m and past
// the last block.
template <typename T>
__global__ __launch_bounds__(256) void rotate_act16_kernel(const T *__restrict__ x, int64_t m, int64_t k,
                                                           int64_t ldx, int mode, _Float16 *__restrict__ a16) {
    const int64_t nb = k / QK;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, L = lane & 3;
    const int r = (wave & 1) * 16 + (lane >> 2);
    const int64_t b = (int64_t)blockIdx.x * 2 + (wave >> 1), row = (int64_t)blockIdx.y * 32 + r;
    if (b >= mx_blocks(k)) return;  // uniform per wave
    const bool live = row < m && b < nb;
    float v[8];
    if (live) {
        load8(x + row * ldx + b * QK + 8 * L, mode, v);
    } else {
#pragma unroll
        for (int t = 0; t < 8; t++) v[t] = 0.0f;
    }
    fwht32_quad(v, L);
    // two roundings, fp32 then fp16: the empty asm keeps the compiler from
    // fusing the product and the conversion into one fp16-rounded
    // multiply-add (one rounding, which differs on rare ties)
    float p[8];
#pragma unroll
    for (int t = 0; t < 8; t++) {
        p[t] = __fmul_rn(v[t], kInvSqrt32f);
        asm volatile("" : "+v"(p[t]));
    }
    uint32_t h[4];
#pragma unroll
    for (int j = 0; j < 4; j++)
        h[j] = (uint32_t)__half_as_ushort(__float2half_rn(p[2 * j])) |
               (uint32_t)__half_as_ushort(__float2half_rn(p[2 * j + 1])) << 16;
    *reinterpret_cast<uint4 *>(a16 + row * w16_row_stride(k) + b * QK + 8 * L) = make_uint4(h[0], h[1], h[2], h[3]);
}

// ---------------------------------------------------------------------------
// The GEMM: y = a16 * w16^T
// ---------------------------------------------------------------------------
// Workgroup: 4 waves (2 x 2), each a 64 x 64 tile of 2 x 2 MFMA tiles: a
// 128 x 128 output tile.  K in stages of one 32-element block through a
// ring of W16_NS LDS stage buffers filled by global-to-LDS loads.  In a
// stage, the fragment of (32-row tile t, K half h) is 1 KB at (2 t + h) KB:
// lane l holds row l % 32, elements 16 h + 8 (l / 32) .. + 7 of the block.
constexpr int W16_NS = 4;
constexpr int W16_RT = 4, W16_CT = 4;                               // 32-row / 32-column tiles per workgroup
constexpr int W16_STAGE = (W16_RT + W16_CT) * 2 * 1024;            // 16 KB
constexpr int W16_DMA_PER_WAVE = (W16_RT + W16_CT) * 2 / 4;        // 4

struct W16Args {
    const _Float16 *a16;   // [rtiles * 32][w16_row_stride(k)]
    const _Float16 *w16;   // [padded_n(n)][w16_row_stride(k)]
    float *y;
    int64_t ldy, m, n, k;
};

__global__ __launch_bounds__(256) void gemm_w16_kernel(W16Args a) {
    __shared__ __attribute__((aligned(1024))) uint8_t smem[W16_NS * W16_STAGE];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    const int64_t kp = w16_row_stride(a.k), nbp = mx_blocks(a.k);
    const int64_t rtiles = (a.m + 31) / 32, ctiles = padded_n(a.n) / TILE_N;

    int64_t bx, by;
    mx_tile_of(blockIdx.x, (a.n + 127) / 128, (a.m + 127) / 128, bx, by);
    const int64_t rt0 = by * W16_RT, ct0 = bx * W16_CT;

    // this wave's loads: tile t = wave * 2 + (d / 2), half h = d % 2 (row
    // tiles first, then column tiles); tiles past the matrix are clamped to
    // the last one (their outputs are never stored)
    const uint8_t *src[W16_DMA_PER_WAVE];
    uint32_t dst[W16_DMA_PER_WAVE];
    const uint32_t smem_base = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)smem;
#pragma unroll
    for (int d = 0; d < W16_DMA_PER_WAVE; d++) {
        const int t = wave * 2 + (d >> 1), h = d & 1;
        const _Float16 *base = t < W16_RT ? a.a16 + min(rt0 + t, rtiles - 1) * 32 * kp
                                          : a.w16 + min(ct0 + t - W16_RT, ctiles - 1) * 32 * kp;
        src[d] = uniform_ptr(reinterpret_cast<const uint8_t *>(base + 16 * h));
        dst[d] = (uint32_t)((2 * t + h) * 1024);
    }
    const uint32_t voff = (uint32_t)((lane & 31) * kp * 2 + 16 * (lane >> 5));
    const int nstages = (int)nbp;
    auto issue = [&](int stage, int slot) {
        // past the last stage the ring reloads the last one (never computed)
        const int64_t b = min(stage, nstages - 1);
        const uint32_t lds = __builtin_amdgcn_readfirstlane(smem_base + slot * W16_STAGE);
#pragma unroll
        for (int d = 0; d < W16_DMA_PER_WAVE; d++) dma16s(src[d] + b * QK * 2, voff, lds + dst[d]);
    };

    v16f acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; i++)
#pragma unroll
        for (int j = 0; j < 2; j++)
#pragma unroll
            for (int v = 0; v < 16; v++) acc[i][j][v] = 0.0f;

    v8h af[2][2][2], bf[2][2][2];  // [buffer][tile][half]
    auto load_frags = [&](const uint8_t *st, int buf) {
#pragma unroll
        for (int i = 0; i < 2; i++)
#pragma unroll
            for (int h = 0; h < 2; h++) {
                af[buf][i][h] = lds_read<v8h>(st + (2 * (wm * 2 + i) + h) * 1024 + 16 * lane);
                bf[buf][i][h] = lds_read<v8h>(st + (2 * (W16_RT + wn * 2 + i) + h) * 1024 + 16 * lane);
            }
    };

#pragma unroll
    for (int x = 0; x < W16_NS - 1; x++) issue(x, x);
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(W16_DMA_PER_WAVE * (W16_NS - 2)) : "memory");
    __syncthreads();
    load_frags(smem, 0);

    // stages in pairs so that the operand buffer of each is fixed at compile time
    for (int s0 = 0; s0 < nstages; s0 += 2) {
#pragma unroll
        for (int u = 0; u < 2; u++) {
            const int s = s0 + u;
            // stage s + 1 has landed for this wave; after the barrier for every
            // wave, and stage s - 1's slot (read during stage s - 1) is free
            asm volatile("s_waitcnt vmcnt(%0)" ::"n"(W16_DMA_PER_WAVE * (W16_NS - 3)) : "memory");
            __syncthreads();
            issue(s + W16_NS - 1, (s + W16_NS - 1) % W16_NS);
            load_frags(smem + ((s + 1) % W16_NS) * W16_STAGE, u ^ 1);
#pragma unroll
            for (int i = 0; i < 2; i++)
#pragma unroll
                for (int j = 0; j < 2; j++)
#pragma unroll
                    for (int h = 0; h < 2; h++)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[u][i][h], bf[u][j][h], acc[i][j], 0, 0, 0);
        }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // no load may still be writing LDS at exit

    const int c = lane & 31;
#pragma unroll
    for (int i = 0; i < 2; i++) {
        const int64_t rbase = (rt0 + wm * 2 + i) * 32;
#pragma unroll
        for (int j = 0; j < 2; j++) {
            const int64_t col = (ct0 + wn * 2 + j) * 32 + c;
            if (col >= a.n) continue;
#pragma unroll
            for (int v = 0; v < 16; v++) {
                const int64_t r = rbase + mfma32_row(v, lane);
                if (r < a.m) a.y[r * a.ldy + col] = acc[i][j][v];
            }
        }
    }
}

}  // namespace w4a4
