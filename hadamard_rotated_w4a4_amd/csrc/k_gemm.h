// W4A4 GEMMs on int8 MFMA (gfx950 v_mfma_i32_32x32x32_i8).
//
// 1bit-MONSTER engine docs, "The lean option: ROCmFP4, ROCmI4 and Hadamard
// Q4_0", section "Hadamard-rotated Q4_0: W4A4 prompt processing": int4 weights
// times int4 rotated activations on the matrix units; section "MoE: W4A4 on
// the experts": the expert matmuls (MUL_MAT_ID) do the same.  CDNA4 has no
// int4 matrix instruction, so the 4-bit codes are widened to int8 (as 16 *
// code) and one 32x32x32 MFMA computes one Q4_0 block's integer dot for a
// 32x32 output tile; K-step 32 = one block.  Each block's int32 sums are
// scaled by d_w[n][b] * s[m][b] into fp32 accumulators (the per-block
// epilogue), in ascending block order.
#pragma once

#include "common.h"

namespace w4a4 {

struct GemmArgs {
    const uint8_t *codes;    // activation codes [rows][k/2]
    const float *scales;     // activation scales [rows][k/32]
    const uint8_t *packed;   // packed weights (expert 0 for the grouped case)
    int64_t expert_bytes;    // packed bytes per expert
    float *y;                // output rows of ldy floats
    int64_t ldy;
    int64_t m, n, k;
    // grouped (MUL_MAT_ID) routing, produced by route_kernel
    const int32_t *perm;         // [n_rows]: row ids t*top_k + j, grouped by expert
    const int32_t *offsets;      // [E+1] start of each expert's rows in perm
    const int32_t *tile_prefix;  // [E+1] prefix count of row tiles per expert
    int n_expert;
    int top_k;
    int act_rows_per_token;
};

// -------------------------------------------------------------------------
// Tiled kernel: WAVES_M x WAVES_N waves, each owning TM x TN 32x32 MFMA tiles;
// BKB Q4_0 blocks staged in LDS per step.
// -------------------------------------------------------------------------
// How the per-block scale product s[m] * d_w[n] of a 32x32 tile is formed on
// the matrix cores: a 32x32x8 bf16 MFMA over exact bf16 splits of the scales,
// or a 32x32x2 fp32 MFMA over the scales themselves (one fp32 rounding).
enum ScaleMfma { kScaleBf16 = 0, kScaleF32 = 1 };

template <int WAVES_M, int WAVES_N, int TM, int TN, int BKB, int SCALE = kScaleBf16>
struct TileCfg {
    static constexpr int BM = WAVES_M * TM * 32;
    static constexpr int BN = WAVES_N * TN * 32;
    static constexpr int NT = 64 * WAVES_M * WAVES_N;
    static constexpr int NTILES = BN / 32;
    static constexpr int kBKB = BKB;
    static constexpr int kWM = WAVES_M, kWN = WAVES_N, kTM = TM, kTN = TN, kScale = SCALE;
};

template <class C, bool GROUPED>
__global__ __launch_bounds__(C::NT) void gemm_tiled_kernel(GemmArgs a) {
    constexpr int BM = C::BM, BN = C::BN, BKB = C::kBKB, NTILES = C::NTILES;
    constexpr int TM = C::kTM, TN = C::kTN, NT = C::NT;
    // Operands are unpacked once per workgroup while staging: each row (A) or
    // column (B) of a block becomes 2 x 16 int8 (one MFMA lane's operand per
    // lane group).  Rows are padded by 16 bytes so that the staging writes of
    // neighbouring lanes (different blocks, same row) fall in different banks.
    constexpr int AP = BM + 1;
    __shared__ uint4 sA[BKB][AP][2];              // int8 activation operands
    __shared__ uint4 sB[BKB][NTILES][64];         // int8 weight operands, MFMA lane order
    // operands of the scale-product MFMA, 16 bytes per row / column and block:
    // bf16 splits (lane group g reads half g), or {scale, 0, ...} as fp32
    // (lane group 0 reads the scale, group 1 the zero)
    constexpr bool SCALE_F32 = C::kScale == kScaleF32;
    __shared__ uint4 sAP[BKB][AP];
    __shared__ uint4 sBP[BKB][BN];
    __shared__ int sArow[BM];  // activation row of each tile row, -1 if none
    __shared__ int sOrow[BM];  // output row

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / C::kWN, wn = wave % C::kWN;
    const int g = lane >> 5, c = lane & 31;
    const int64_t k = a.k, nb = k / QK;
    const int64_t tiles_n = padded_n(a.n) / TILE_N;

    // Dense launches use a 1-D grid in an XCD-aware order.  Workgroups are
    // dealt to the 8 XCDs round-robin, so ids x, x + 8, x + 16, ... share an
    // XCD and its L2: the row tiles of one weight column tile are given ids
    // x + 8y, i.e. the same XCD and close in dispatch time, and the weights
    // they share are read from HBM about once.
    int64_t bx, by;
    if constexpr (GROUPED) {
        bx = blockIdx.x;
        by = blockIdx.y;
    } else {
        constexpr int64_t XCDS = 8;
        const int64_t nx = (a.n + C::BN - 1) / C::BN, ny = (a.m + BM - 1) / BM;
        const int64_t id = blockIdx.x, group = id / (XCDS * ny), in = id % (XCDS * ny);
        const int64_t width = min(XCDS, nx - group * XCDS);  // columns in this group (last may be short)
        bx = group * XCDS + in % width;
        by = in / width;
    }
    const int64_t tile0 = bx * NTILES;

    int valid_rows;
    const uint8_t *wbase = a.packed;
    if constexpr (GROUPED) {
        const int ty = (int)by;
        if (ty >= a.tile_prefix[a.n_expert]) return;  // uniform: whole workgroup exits
        int lo = 0, hi = a.n_expert;                  // largest e with tile_prefix[e] <= ty
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (a.tile_prefix[mid] <= ty) lo = mid; else hi = mid;
        }
        const int e = lo;
        const int row0 = (ty - a.tile_prefix[e]) * BM;
        const int cnt = a.offsets[e + 1] - a.offsets[e];
        valid_rows = min(BM, cnt - row0);
        for (int r = tid; r < BM; r += NT) {
            int ar = -1, orow = 0;
            if (r < valid_rows) {
                orow = a.perm[a.offsets[e] + row0 + r];
                ar = a.act_rows_per_token == 1 ? orow / a.top_k : orow;
            }
            sArow[r] = ar;
            sOrow[r] = orow;
        }
        wbase = a.packed + (int64_t)e * a.expert_bytes;
    } else {
        const int64_t row0 = by * BM;
        valid_rows = (int)min((int64_t)BM, a.m - row0);
        for (int r = tid; r < BM; r += NT) {
            sArow[r] = r < valid_rows ? (int)(row0 + r) : -1;
            sOrow[r] = (int)(row0 + r);
        }
    }
    const uint8_t *wcodes = wbase;
    const uint16_t *wscales = reinterpret_cast<const uint16_t *>(wbase + packed_code_bytes(a.n, k));
    __syncthreads();

    // ---- per-thread staging slots, fixed across K steps ----
    // A: (row, block) pairs; B: 16-byte pieces of (tile, block) codes and
    // single fp16 scales.  Each slot keeps a source pointer that advances by
    // BKB blocks per step, the block it stages, and whether its row/tile exists.
    constexpr int A_WORK = BM * BKB, B_WORK = NTILES * BKB * 32;
    constexpr int A_SLOTS = (A_WORK + NT - 1) / NT, B_SLOTS = (B_WORK + NT - 1) / NT;
    const uint8_t *a_src[A_SLOTS];
    const float *s_src[A_SLOTS];
    int a_bb[A_SLOTS];
    bool a_ok[A_SLOTS];
#pragma unroll
    for (int p = 0; p < A_SLOTS; p++) {
        const int i = tid + p * NT;
        const int r = i / BKB, bb = i % BKB;
        const int ar = i < A_WORK ? sArow[r] : -1;
        a_ok[p] = ar >= 0;
        a_bb[p] = bb;
        a_src[p] = a.codes + (int64_t)(ar >= 0 ? ar : 0) * (k / 2) + bb * 16;
        s_src[p] = a.scales + (int64_t)(ar >= 0 ? ar : 0) * nb + bb;
    }
    const uint4 *b_src[B_SLOTS];
    const uint16_t *d_src[B_SLOTS];
    int b_bb[B_SLOTS];
    bool b_ok[B_SLOTS];
#pragma unroll
    for (int p = 0; p < B_SLOTS; p++) {
        const int i = tid + p * NT;
        const int t = i / (BKB * 32), rem = i % (BKB * 32), bb = rem / 32, q = rem % 32;
        const int64_t tile = tile0 + t;
        b_ok[p] = i < B_WORK && tile < tiles_n;
        b_bb[p] = bb;
        const int64_t tb = (b_ok[p] ? tile : 0) * nb + bb;
        b_src[p] = reinterpret_cast<const uint4 *>(wcodes + tb * TILE_CODE_BYTES) + q;
        d_src[p] = wscales + tb * TILE_SCALE_HALFS + q;
    }
    uint4 a_reg[A_SLOTS], b_reg[B_SLOTS];
    float s_reg[A_SLOTS];
    uint16_t d_reg[B_SLOTS];

    auto load_stage = [&](int64_t kb0) {
#pragma unroll
        for (int p = 0; p < A_SLOTS; p++) {
            a_reg[p] = make_uint4(0, 0, 0, 0);
            s_reg[p] = 0.0f;
            if (a_ok[p] && kb0 + a_bb[p] < nb) {
                a_reg[p] = *reinterpret_cast<const uint4 *>(a_src[p] + kb0 * 16);
                s_reg[p] = s_src[p][kb0];
            }
        }
#pragma unroll
        for (int p = 0; p < B_SLOTS; p++) {
            b_reg[p] = make_uint4(0, 0, 0, 0);
            d_reg[p] = 0;
            if (b_ok[p] && kb0 + b_bb[p] < nb) {
                b_reg[p] = b_src[p][kb0 * (TILE_CODE_BYTES / 16)];
                d_reg[p] = d_src[p][kb0 * TILE_SCALE_HALFS];
            }
        }
    };
    auto store_stage = [&]() {
#pragma unroll
        for (int p = 0; p < A_SLOTS; p++) {
            const int i = tid + p * NT;
            if (i < A_WORK) {
                const int r = i / BKB, bb = i % BKB;
                const uint4 q = a_reg[p];
                const v4i lo = unpack_nibbles_x16(q.x, q.y), hi = unpack_nibbles_x16(q.z, q.w);
                sA[bb][r][0] = make_uint4(lo.x, lo.y, lo.z, lo.w);
                sA[bb][r][1] = make_uint4(hi.x, hi.y, hi.z, hi.w);
                sAP[bb][r] = SCALE_F32 ? make_uint4(__float_as_uint(s_reg[p]), 0, 0, 0) : split_scale_a(s_reg[p]);
            }
        }
#pragma unroll
        for (int p = 0; p < B_SLOTS; p++) {
            const int i = tid + p * NT;
            if (i < B_WORK) {
                const int t = i / (BKB * 32), rem = i % (BKB * 32), bb = rem / 32, q = rem % 32;
                const uint4 w = b_reg[p];  // the packed operands of lanes 2q and 2q + 1
                const v4i l0 = unpack_nibbles_x16(w.x, w.y), l1 = unpack_nibbles_x16(w.z, w.w);
                sB[bb][t][2 * q] = make_uint4(l0.x, l0.y, l0.z, l0.w);
                sB[bb][t][2 * q + 1] = make_uint4(l1.x, l1.y, l1.z, l1.w);
                // / 256 (exact) undoes the 16 x 16 scaling of the unpacked operands
                const float dsc = __half2float(__ushort_as_half(d_reg[p])) * (1.0f / 256.0f);
                sBP[bb][t * 32 + q] = SCALE_F32 ? make_uint4(__float_as_uint(dsc), 0, 0, 0) : split_scale_b(dsc);
            }
        }
    };

    float acc[TM][TN][16];
#pragma unroll
    for (int i = 0; i < TM; i++)
#pragma unroll
        for (int j = 0; j < TN; j++)
#pragma unroll
            for (int v = 0; v < 16; v++) acc[i][j][v] = 0.0f;

    const int wrow0 = wm * TM * 32;  // first tile row of this wave
    load_stage(0);
    for (int64_t kb0 = 0; kb0 < nb; kb0 += BKB) {
        store_stage();
        __syncthreads();
        if (kb0 + BKB < nb) load_stage(kb0 + BKB);  // in flight during the compute below

        // ---- compute: per 32x32 tile and block, S on int8 MFMA, s*d_w on a float MFMA ----
#pragma unroll
        for (int bb = 0; bb < BKB; bb++) {
            v4i af[TM], bf[TN];
            uint2 ap[TM], bp[TN];
#pragma unroll
            for (int i = 0; i < TM; i++) {
                af[i] = __builtin_bit_cast(v4i, sA[bb][wrow0 + i * 32 + c][g]);
                if constexpr (SCALE_F32)
                    ap[i].x = reinterpret_cast<const uint32_t *>(&sAP[bb][wrow0 + i * 32 + c])[g];
                else
                    ap[i] = reinterpret_cast<const uint2 *>(&sAP[bb][wrow0 + i * 32 + c])[g];
            }
#pragma unroll
            for (int j = 0; j < TN; j++) {
                bf[j] = __builtin_bit_cast(v4i, sB[bb][wn * TN + j][lane]);
                if constexpr (SCALE_F32)
                    bp[j].x = reinterpret_cast<const uint32_t *>(&sBP[bb][(wn * TN + j) * 32 + c])[g];
                else
                    bp[j] = reinterpret_cast<const uint2 *>(&sBP[bb][(wn * TN + j) * 32 + c])[g];
            }
            // Empty tile rows carry zero codes and zero scales, so they add 0;
            // no branch here keeps each block's MFMAs and epilogue in one
            // basic block for the scheduler.
#pragma unroll
            for (int i = 0; i < TM; i++) {
#pragma unroll
                for (int j = 0; j < TN; j++) {
                    const v16i S = mfma_i8_32x32x32(af[i], bf[j]);
                    v16f P;
                    if constexpr (SCALE_F32)
                        P = mfma_f32_32x32x2(__uint_as_float(ap[i].x), __uint_as_float(bp[j].x));
                    else
                        P = mfma_bf16_32x32x8(ap[i], bp[j]);
#pragma unroll
                    for (int v = 0; v < 16; v++) acc[i][j][v] = fmaf((float)S[v], P[v], acc[i][j][v]);
                }
            }
        }
        __syncthreads();
    }

    // ---- store ----
#pragma unroll
    for (int i = 0; i < TM; i++) {
        if (wrow0 + i * 32 >= valid_rows) continue;
#pragma unroll
        for (int j = 0; j < TN; j++) {
            const int64_t col = (tile0 + wn * TN + j) * 32 + c;
            if (col >= a.n) continue;
#pragma unroll
            for (int v = 0; v < 16; v++) {
                const int r = wrow0 + i * 32 + mfma32_row(v, lane);
                if (r < valid_rows) a.y[(int64_t)sOrow[r] * a.ldy + col] = acc[i][j][v];
            }
        }
    }
}

// -------------------------------------------------------------------------
// MUL_MAT_ID routing: one workgroup groups the (token, slot) rows by expert
// and counts each expert's row tiles; rows with an invalid id are zeroed.
// -------------------------------------------------------------------------
constexpr int ROUTE_THREADS = 1024;
constexpr int ROUTE_MAX_EXPERTS = 8192;

// Counting lives in LDS (one workgroup), so every count and cursor update is
// seen by the whole workgroup after a barrier.
__global__ __launch_bounds__(ROUTE_THREADS) void route_kernel(const int32_t *__restrict__ ids, int n_rows,
                                                              int n_expert, int tile_rows,
                                                              int32_t *__restrict__ offsets,
                                                              int32_t *__restrict__ tile_prefix,
                                                              int32_t *__restrict__ perm, float *__restrict__ y,
                                                              int64_t n) {
    __shared__ int cnt[ROUTE_MAX_EXPERTS];
    __shared__ int part[ROUTE_THREADS];
    __shared__ int tpart[ROUTE_THREADS];
    const int tid = threadIdx.x;
    for (int e = tid; e < n_expert; e += ROUTE_THREADS) cnt[e] = 0;
    __syncthreads();
    for (int i = tid; i < n_rows; i += ROUTE_THREADS) {
        const int e = ids[i];
        if (e >= 0 && e < n_expert) atomicAdd(&cnt[e], 1);
    }
    __syncthreads();
    // exclusive scans of row counts and of row tiles, over contiguous per-thread chunks
    const int per = (n_expert + ROUTE_THREADS - 1) / ROUTE_THREADS;
    const int e0 = min(tid * per, n_expert), e1 = min(e0 + per, n_expert);
    int s = 0, ts = 0;
    for (int e = e0; e < e1; e++) { s += cnt[e]; ts += (cnt[e] + tile_rows - 1) / tile_rows; }
    part[tid] = s;
    tpart[tid] = ts;
    __syncthreads();
    for (int off = 1; off < ROUTE_THREADS; off <<= 1) {
        const int pa = tid >= off ? part[tid - off] : 0;
        const int pb = tid >= off ? tpart[tid - off] : 0;
        __syncthreads();
        part[tid] += pa;
        tpart[tid] += pb;
        __syncthreads();
    }
    int run = part[tid] - s, trun = tpart[tid] - ts;
    for (int e = e0; e < e1; e++) {
        const int ce = cnt[e];
        offsets[e] = run;
        tile_prefix[e] = trun;
        cnt[e] = run;  // becomes the expert's scatter cursor
        run += ce;
        trun += (ce + tile_rows - 1) / tile_rows;
    }
    if (tid == ROUTE_THREADS - 1) {
        offsets[n_expert] = part[tid];
        tile_prefix[n_expert] = tpart[tid];
    }
    __syncthreads();
    for (int i = tid; i < n_rows; i += ROUTE_THREADS) {
        const int e = ids[i];
        if (e >= 0 && e < n_expert) {
            perm[atomicAdd(&cnt[e], 1)] = i;
        } else {
            for (int64_t j = 0; j < n; j++) y[(int64_t)i * n + j] = 0.0f;
        }
    }
}

// Fill rows of y with zeros (used when k == 0: an empty sum).
__global__ void zero_rows_kernel(float *y, int64_t m, int64_t n, int64_t ldy) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < m * n) y[(i / n) * ldy + i % n] = 0.0f;
}

}  // namespace w4a4
