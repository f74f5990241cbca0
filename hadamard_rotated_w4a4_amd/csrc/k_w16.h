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
// its own registers.  Both operands are stored pre-tiled in the MFMA's
// fragment order, so each global-to-LDS load copies 1 KB of contiguous
// memory (a row-major operand would touch 32 cache lines for 64 bytes each
// per load):
//   [32-row tile][padded block][K half h][lane l][8 elements]
// element (r, t) sits in tile r / 32, block t / 32, half (t % 32) / 16, lane
// (r % 32) + 32 ((t % 16) / 8), slot t % 8; 2 KB per (tile, block).  Rows are
// padded to whole tiles and blocks to a multiple of MX_BLOCK_PAD, with zeros,
// so the GEMM loads whole stages without bounds checks.
#pragma once

#include "common.h"
#include "k_dense.h"
#include "k_rotq.h"

namespace w4a4 {

typedef _Float16 v8h __attribute__((ext_vector_type(8)));

constexpr int W16_TILE_BLOCK = 2048;  // bytes per (32-row tile, block) of a tiled operand

// Bytes of a tiled operand of `rows` rows.
__host__ __device__ inline int64_t w16_operand_bytes(int64_t rows, int64_t k) {
    return (rows + 31) / 32 * mx_blocks(k) * W16_TILE_BLOCK;
}

// Element index of piece p (elements 8 p .. 8 p + 7 of block b) of row r.
__device__ __forceinline__ int64_t w16_piece(int64_t r, int64_t b, int p, int64_t nbp) {
    return ((((r >> 5) * nbp + b) * 2 + (p >> 1)) * 64 + (r & 31) + 32 * (p & 1)) * 8;
}

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
#pragma unroll
    for (int p = 0; p < 4; p++)
        *reinterpret_cast<uint4 *>(w16 + w16_piece(row, b, p, nbp)) = make_uint4(h[4 * p], h[4 * p + 1], h[4 * p + 2], h[4 * p + 3]);
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
    *reinterpret_cast<uint4 *>(a16 + w16_piece(row, b, L, mx_blocks(k))) = make_uint4(h[0], h[1], h[2], h[3]);
}

// ---------------------------------------------------------------------------
// The GEMM: y = a16 * w16^T
// ---------------------------------------------------------------------------
// Workgroup: 4 waves (2 x 2), each a 64 x 64 tile of 2 x 2 MFMA tiles: a
// 128 x 128 output tile.  K in stages of one 32-element block through a
// ring of W16_NS LDS stage buffers filled by global-to-LDS loads.  In a
// stage, the fragment of (32-row tile t, K half h) is 1 KB at (2 t + h) KB,
// a copy of the operand's 1 KB (lane l: row l % 32, elements
// 16 h + 8 (l / 32) .. + 7 of the block).
constexpr int W16_NS = 4;
constexpr int W16_RT = 4, W16_CT = 4;                               // 32-row / 32-column tiles per workgroup
constexpr int W16_STAGE = (W16_RT + W16_CT) * 2 * 1024;            // 16 KB
constexpr int W16_DMA_PER_WAVE = (W16_RT + W16_CT) * 2 / 4;        // 4

struct W16Args {
    const _Float16 *a16;   // tiled, ceil(m / 32) row tiles
    const _Float16 *w16;   // tiled, padded_n(n) / 32 row tiles
    float *y;
    int64_t ldy, m, n, k;
};

// One whole 128 x 128 tile (workgroup index id).
__device__ __forceinline__ void w16_tile(const W16Args &a, int64_t id, uint8_t *smem) {
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    const int64_t nbp = mx_blocks(a.k);
    const int64_t rtiles = (a.m + 31) / 32, ctiles = padded_n(a.n) / TILE_N;

    int64_t bx, by;
    mx_tile_of(id, (a.n + 127) / 128, (a.m + 127) / 128, bx, by);
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
        const uint8_t *base = t < W16_RT ? reinterpret_cast<const uint8_t *>(a.a16) + min(rt0 + t, rtiles - 1) * nbp * W16_TILE_BLOCK
                                         : reinterpret_cast<const uint8_t *>(a.w16) + min(ct0 + t - W16_RT, ctiles - 1) * nbp * W16_TILE_BLOCK;
        src[d] = uniform_ptr(base + h * 1024);
        dst[d] = (uint32_t)((2 * t + h) * 1024);
    }
    const uint32_t voff = (uint32_t)(lane * 16);
    const int nstages = (int)nbp;
    auto issue = [&](int stage, int slot) {
        // past the last stage the ring reloads the last one (never computed)
        const int64_t b = min(stage, nstages - 1);
        const uint32_t lds = __builtin_amdgcn_readfirstlane(smem_base + slot * W16_STAGE);
#pragma unroll
        for (int d = 0; d < W16_DMA_PER_WAVE; d++) dma16s(src[d] + b * W16_TILE_BLOCK, voff, lds + dst[d]);
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
            // all of stage s + 1's fragment reads are issued before stage s's
            // MFMAs, so their latency hides behind them (the scheduler would
            // otherwise sink each read to just before its first use)
            load_frags(smem + ((s + 1) % W16_NS) * W16_STAGE, u ^ 1);
            __builtin_amdgcn_sched_barrier(0);
            // K half outermost: four independent accumulators between the
            // two MFMAs that share one
#pragma unroll
            for (int h = 0; h < 2; h++)
#pragma unroll
                for (int i = 0; i < 2; i++)
#pragma unroll
                    for (int j = 0; j < 2; j++)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[u][i][h], bf[u][j][h], acc[i][j], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
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

// Leftover tiles (as in the W4A4 GEMM): when the whole tiles leave a
// partial last round, each leftover tile is split into 16 pieces of 32 x 32,
// one workgroup each, its 4 waves over a quarter of K each.  A wave streams
// its own fragments (A and B, both halves of one block per stage) through
// its own LDS ring, waits only for its own loads, and the quarters meet in
// LDS in ascending K order.
constexpr int W16_PIECES = W16_RT * W16_CT;
constexpr int W16_PNS = 4;                      // stages per wave ring
constexpr int W16_PSTAGE = 4 * 1024;            // A h0, A h1, B h0, B h1

__device__ __forceinline__ void w16_piece(const W16Args &a, int64_t first_tile, int64_t id, uint8_t *smem) {
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int64_t nbp = mx_blocks(a.k);
    const int64_t rtiles = (a.m + 31) / 32, ctiles = padded_n(a.n) / TILE_N;

    int64_t bx, by;
    mx_tile_of(first_tile + id / W16_PIECES, (a.n + 127) / 128, (a.m + 127) / 128, bx, by);
    const int sub = (int)(id % W16_PIECES);
    const int64_t rt = by * W16_RT + sub / W16_CT, ct = bx * W16_CT + sub % W16_CT;
    // pieces past the matrix edge compute on clamped tiles and store nothing
    const uint8_t *abase = uniform_ptr(reinterpret_cast<const uint8_t *>(a.a16) + min(rt, rtiles - 1) * nbp * W16_TILE_BLOCK);
    const uint8_t *bbase = uniform_ptr(reinterpret_cast<const uint8_t *>(a.w16) + min(ct, ctiles - 1) * nbp * W16_TILE_BLOCK);

    // this wave's quarter of the blocks (nbp is a multiple of 8: never empty)
    const int64_t b0 = nbp / 4 * wave;
    const int nst = (int)(nbp / 4);
    uint8_t *ring = smem + wave * W16_PNS * W16_PSTAGE;
    const uint32_t ring_lds =
        __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)ring);
    const uint32_t voff = lane * 16;
    auto issue = [&](int stage, int slot) {
        // past the last stage the ring reloads the last one (never computed)
        const int64_t off = (b0 + min(stage, nst - 1)) * W16_TILE_BLOCK;
        const uint32_t lds = ring_lds + slot * W16_PSTAGE;
        dma16s(abase + off, voff, lds);
        dma16s(abase + off + 1024, voff, lds + 1024);
        dma16s(bbase + off, voff, lds + 2048);
        dma16s(bbase + off + 1024, voff, lds + 3072);
    };

    v16f acc;
#pragma unroll
    for (int v = 0; v < 16; v++) acc[v] = 0.0f;
#pragma unroll
    for (int x = 0; x < W16_PNS - 1; x++) issue(x, x);
    for (int s = 0; s < nst; s++) {
        // stage s has landed: only the W16_PNS - 2 stages after it may be in flight
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"(4 * (W16_PNS - 2)) : "memory");
        const uint8_t *st = ring + (s % W16_PNS) * W16_PSTAGE + 16 * lane;
        const v8h a0 = lds_read<v8h>(st), a1 = lds_read<v8h>(st + 1024);
        const v8h b0f = lds_read<v8h>(st + 2048), b1f = lds_read<v8h>(st + 3072);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(a0, b0f, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(a1, b1f, acc, 0, 0, 0);
        // the reads above have fed their MFMAs before the slot they came from
        // can be refilled (three stages later)
        __builtin_amdgcn_sched_barrier(0);
        issue(s + W16_PNS - 1, (s + W16_PNS - 1) % W16_PNS);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // no load may still be writing the ring

    // the quarters meet in LDS (the rings are free now) in ascending K order
    __syncthreads();
    float *red = reinterpret_cast<float *>(smem);
#pragma unroll
    for (int v = 0; v < 16; v++) red[(wave * 16 + v) * 64 + lane] = acc[v];
    __syncthreads();
    for (int i = tid; i < 16 * 64; i += 256) {
        const int v = i / 64, l = i % 64;
        const float sum = ((red[(0 * 16 + v) * 64 + l] + red[(1 * 16 + v) * 64 + l]) + red[(2 * 16 + v) * 64 + l]) +
                          red[(3 * 16 + v) * 64 + l];
        const int64_t r = rt * 32 + mfma32_row(v, l), col = ct * 32 + (l & 31);
        if (rt < rtiles && r < a.m && col < a.n) a.y[r * a.ldy + col] = sum;
    }
}

static_assert(4 * W16_PNS * W16_PSTAGE <= W16_NS * W16_STAGE, "the piece rings fit the tile's LDS");

// One launch: workgroups below main_wgs take whole tiles (XCD-aware order),
// the rest the pieces of the leftover tiles, which fill the CUs that the last
// whole tiles leave idle (workgroups are dispatched in index order).
__global__ __launch_bounds__(256) void gemm_w16_kernel(W16Args a, int64_t main_wgs, int64_t first_piece_tile) {
    __shared__ __attribute__((aligned(1024))) uint8_t smem[W16_NS * W16_STAGE];
    if ((int64_t)blockIdx.x < main_wgs) w16_tile(a, blockIdx.x, smem);
    else w16_piece(a, first_piece_tile, blockIdx.x - main_wgs, smem);
}

}  // namespace w4a4
