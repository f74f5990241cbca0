// MUL_MAT_ID product that streams the experts' 4-bit weight records.
//
// 1bit-MONSTER engine docs, "The lean option: ROCmFP4, ROCmI4 and Hadamard
// Q4_0", section "MoE: W4A4 on the experts": the expert matmuls take the same
// W4A4 path as the dense ones -- int4 x int4 block dots, per-block scaling.
//
// The experts of a micro-batch get few rows each (tens, a few hundred for the
// popular ones), so the product is bound by streaming the weights, as for
// m <= 16.  Work item = (expert tile of GS_ROWS routed rows, chunk of
// GS_WAVES column tiles): the workgroup stages its rows' activations in LDS
// straight from the activation rows (the routing's row permutation picks
// them; no gathered copy is written), then each wave streams one 32-column
// tile's 2304-byte records (the m <= 16 layout, 0.5625 B per weight) through
// a 2-deep register ring.  Per block and wave: 4 int8 16x16x32 MFMAs (two
// 16-row halves x columns c and 16 + c), then per output the scale product
// and a fused multiply-add (codes enter as 16 x nibble, so d is scaled by
// 2^-8).  Long K is staged in chunks (gs_kchunk blocks).  Each
// workgroup scatters its rows to y.  Each XCD takes a contiguous share of
// the expert-ordered items, so an expert's row tiles share one L2 and read
// its weights from HBM about once.
//
// The same kernel runs a plain (dense) product as one "expert" holding every
// row (no routing), and takes int8 activation codes (A8: the exact int8 path
// on a rotated file, staged as 8-byte K-group entries and fed to the MFMA as
// they are; d is then scaled by 2^-4).
#pragma once

#include "common.h"
#include "k_route.h"

namespace w4a4 {

constexpr int GS_ROWS = 32;     // routed rows per item (two 16-row MFMA halves)
constexpr int GS_WAVES = 8;     // waves per workgroup, one column tile each
// blocks of activations staged per pass (a multiple of 4): 40 KB of K8
// words and scales, or 36 KB of int8 codes and scales
template <bool A8>
constexpr int gs_kchunk() { return A8 ? 32 : 64; }
template <bool A8>
constexpr int gs_stage_bytes() { return gs_kchunk<A8>() * (4 * GS_ROWS * (A8 ? 8 : 4) + GS_ROWS * 4); }

struct GsArgs {
    const uint8_t *codes;    // activation codes [rows][k/2] (A8: [rows][k])
    const float *scales;     // activation scales [rows][k/32]
    const uint8_t *packed;   // packed weights of expert 0; expert e at + e * expert_bytes
    int64_t expert_bytes;
    float *y;                // [n_tokens * top_k][n] (dense: [rows][ldy])
    int64_t ldy, n, k;
    int64_t dense_rows;      // >= 0: a plain product of this many rows, no routing
    Routing g;
    int top_k, per_slot;     // activation row of routed row i: i (per slot) or i / top_k
    int64_t n_rows;          // routed rows (tokens x slots); those past offsets[E] have invalid ids
    int64_t col_chunks;      // ceil(tiles / GS_WAVES)
};

template <bool A8>
__global__ __launch_bounds__(64 * GS_WAVES) void gemm_grouped_stream_kernel(GsArgs a) {
    constexpr int KCHUNK = gs_kchunk<A8>();
    constexpr int ROW_BYTES = A8 ? QK : QK / 2;  // activation code bytes per (row, block)
    __shared__ __attribute__((aligned(16))) uint8_t smem[gs_stage_bytes<A8>()];
    __shared__ int64_t src_row[GS_ROWS];
    __shared__ int32_t out_row[GS_ROWS];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int64_t k = a.k, nb = k / QK, nq = sq_quads(k);
    const int64_t tiles = padded_n(a.n) / TILE_N;

    const bool dense = a.dense_rows >= 0;
    // workgroup 0 first zeroes the output rows of invalid ids (the routing put
    // them after the valid rows), whatever item it takes after
    if (!dense && blockIdx.x == 0) {
        const int64_t first = a.g.offsets[a.g.n_expert], bad = a.n_rows - first;
        for (int64_t i = tid; i < bad * a.n; i += 64 * GS_WAVES)
            a.y[(int64_t)a.g.perm[first + i / a.n] * a.ldy + i % a.n] = 0.0f;
    }

    // item: contiguous share per XCD (ids x, x + 8, ... run on XCD x)
    const int64_t rtiles = dense ? (a.dense_rows + GS_ROWS - 1) / GS_ROWS : a.g.tile_prefix[a.g.n_expert];
    const int64_t items = rtiles * a.col_chunks, per_xcd = (items + 7) / 8;
    const int64_t j = blockIdx.x / 8, item = (blockIdx.x % 8) * per_xcd + j;
    if (j >= per_xcd || item >= items) return;  // uniform
    const int64_t rt = item / a.col_chunks, cc = item % a.col_chunks;
    const int e = dense ? 0 : expert_of_tile(a.g, rt);
    const int64_t cnt = dense ? a.dense_rows : a.g.offsets[e + 1] - a.g.offsets[e];
    const int64_t row_lo = (dense ? rt : rt - a.g.tile_prefix[e]) * GS_ROWS;
    if (tid < GS_ROWS) {
        const int64_t local = row_lo + tid;
        int64_t src = -1;
        int32_t orow = -1;
        if (local < cnt) {
            orow = dense ? (int32_t)local : a.g.perm[a.g.offsets[e] + local];
            src = dense || a.per_slot ? orow : orow / a.top_k;
        }
        src_row[tid] = src;
        out_row[tid] = orow;
    }

    // this wave's column tile (a last chunk's extra waves stream the last
    // tile again and store nothing)
    const int64_t tile = cc * GS_WAVES + wave;
    const int64_t ltile = min(tile, tiles - 1);
    const uint8_t *sq = a.packed + e * a.expert_bytes + sq_section_offset(a.n, k) + ltile * nq * SQ_REC;
    const int lo16 = lane * 16, d16 = SQ_SCALE_OFF + (lane & 15) * 16;

    float acc[2][2][4];  // [row half][column half][4 rows]
#pragma unroll
    for (int h = 0; h < 2; h++)
#pragma unroll
        for (int c2 = 0; c2 < 2; c2++)
#pragma unroll
            for (int i = 0; i < 4; i++) acc[h][c2][i] = 0.0f;

    uint32_t *act = reinterpret_cast<uint32_t *>(smem);                            // [block][g][row]
    uint2 *act8 = reinterpret_cast<uint2 *>(smem);                                 // A8: [block][g][row]
    float *asc = reinterpret_cast<float *>(smem + KCHUNK * 4 * GS_ROWS * (A8 ? 8 : 4));  // [block][row]

    for (int64_t c0 = 0; c0 < nb; c0 += KCHUNK) {
        const int kc = (int)min((int64_t)KCHUNK, nb - c0);  // blocks of this chunk
        const int nr = (kc + SQ_BLOCKS - 1) / SQ_BLOCKS;         // its records (the last may be padded)
        __syncthreads();  // the row table is written; the previous chunk's reads are done
        // stage: one (row, block) per thread and step; rows past the expert's
        // count and blocks past nb are zero
        for (int i = tid; i < nr * SQ_BLOCKS * GS_ROWS; i += 64 * GS_WAVES) {
            const int bl = i / GS_ROWS, r = i % GS_ROWS;
            const int64_t b = c0 + bl, src = src_row[r];
            uint4 u = make_uint4(0, 0, 0, 0), u1 = make_uint4(0, 0, 0, 0);
            float s = 0.0f;
            if (src >= 0 && b < nb) {
                const uint4 *p = reinterpret_cast<const uint4 *>(a.codes + src * (k / 32 * ROW_BYTES) + b * ROW_BYTES);
                u = p[0];
                if constexpr (A8) u1 = p[1];
                s = a.scales[src * nb + b];
            }
            if constexpr (A8) {
                act8[(bl * 4 + 0) * GS_ROWS + r] = make_uint2(u.x, u.y);  // codes 0..7
                act8[(bl * 4 + 1) * GS_ROWS + r] = make_uint2(u.z, u.w);
                act8[(bl * 4 + 2) * GS_ROWS + r] = make_uint2(u1.x, u1.y);
                act8[(bl * 4 + 3) * GS_ROWS + r] = make_uint2(u1.z, u1.w);
            } else {
                const uint4 w = k8_words(u);
                act[(bl * 4 + 0) * GS_ROWS + r] = w.x;
                act[(bl * 4 + 1) * GS_ROWS + r] = w.y;
                act[(bl * 4 + 2) * GS_ROWS + r] = w.z;
                act[(bl * 4 + 3) * GS_ROWS + r] = w.w;
            }
            asc[bl * GS_ROWS + r] = s;
        }
        __syncthreads();

        // this wave's records of the chunk, in order, through a 2-deep ring
        const __amdgpu_buffer_rsrc_t wbuf = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint8_t *>(sq + (c0 / SQ_BLOCKS) * SQ_REC), 0, nr * SQ_REC, 0x00020000);
        struct Rec {
            v4u c0, c1, d;
        };
        auto load = [&](int i, Rec &R) {  // slots past the chunk reload its last record (a cache hit)
            const int off = __builtin_amdgcn_readfirstlane(min(i, nr - 1) * SQ_REC);
            R.c0 = __builtin_amdgcn_raw_buffer_load_b128(wbuf, lo16, off, 0);
            __builtin_amdgcn_sched_barrier(0);
            R.c1 = __builtin_amdgcn_raw_buffer_load_b128(wbuf, lo16 + 1024, off, 0);
            __builtin_amdgcn_sched_barrier(0);
            R.d = __builtin_amdgcn_raw_buffer_load_b128(wbuf, d16, off, 0);
            __builtin_amdgcn_sched_barrier(0);
        };
        constexpr float UNSCALE = A8 ? 1.0f / 16.0f : 1.0f / 256.0f;  // the operands' 16 x factors
        auto block = [&](int bl, uint32_t w0, uint32_t w1, uint32_t dpair) {
            const long b0 = widen_k8(w0), b1 = widen_k8(w1);
            const float d0 = __half2float(__ushort_as_half((uint16_t)(dpair & 0xFFFF))) * UNSCALE;
            const float d1 = __half2float(__ushort_as_half((uint16_t)(dpair >> 16))) * UNSCALE;
#pragma unroll
            for (int h = 0; h < 2; h++) {
                // row h * 16 + lane % 16, K-group lane / 16
                const int ai = (bl * 4 + (lane >> 4)) * GS_ROWS + h * 16 + (lane & 15);
                long av;
                if constexpr (A8) {
                    const uint2 u = act8[ai];
                    av = (long)((uint64_t)u.y << 32 | u.x);
                } else {
                    av = widen_k8(act[ai]);
                }
                const v4i S0 = mfma_i8_16x16x32(av, b0);
                const v4i S1 = mfma_i8_16x16x32(av, b1);
                const float4 s4 = *reinterpret_cast<const float4 *>(asc + bl * GS_ROWS + h * 16 + 4 * (lane >> 4));
                const float sv[4] = {s4.x, s4.y, s4.z, s4.w};
#pragma unroll
                for (int i = 0; i < 4; i++) {
                    acc[h][0][i] = fmaf((float)S0[i], __fmul_rn(sv[i], d0), acc[h][0][i]);
                    acc[h][1][i] = fmaf((float)S1[i], __fmul_rn(sv[i], d1), acc[h][1][i]);
                }
            }
        };
        auto compute = [&](int i, const Rec &R) {
            const int bl = i * SQ_BLOCKS;
            block(bl + 0, R.c0[0], R.c0[1], R.d[0]);
            block(bl + 1, R.c0[2], R.c0[3], R.d[1]);
            block(bl + 2, R.c1[0], R.c1[1], R.d[2]);
            block(bl + 3, R.c1[2], R.c1[3], R.d[3]);
        };
        Rec r0, r1;
        load(0, r0);
        for (int i = 0; i < nr; i += 2) {
            load(i + 1, r1);
            __builtin_amdgcn_sched_barrier(0);
            compute(i, r0);
            __builtin_amdgcn_sched_barrier(0);
            if (i + 1 >= nr) break;
            load(i + 2, r0);
            __builtin_amdgcn_sched_barrier(0);
            compute(i + 1, r1);
            __builtin_amdgcn_sched_barrier(0);
        }
    }

    // scatter: output row of local row r is out_row[r]
    if (tile >= tiles) return;
#pragma unroll
    for (int h = 0; h < 2; h++)
#pragma unroll
        for (int c2 = 0; c2 < 2; c2++) {
            const int64_t col = tile * TILE_N + c2 * 16 + (lane & 15);
            if (col >= a.n) continue;
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const int r = h * 16 + 4 * (lane >> 4) + i;
                const int32_t orow = out_row[r];
                if (orow >= 0) a.y[(int64_t)orow * a.ldy + col] = acc[h][c2][i];
            }
        }
}

}  // namespace w4a4
