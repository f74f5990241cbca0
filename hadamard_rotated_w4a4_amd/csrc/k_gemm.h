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
template <int WAVES_M, int WAVES_N, int TM, int TN, int BKB>
struct TileCfg {
    static constexpr int BM = WAVES_M * TM * 32;
    static constexpr int BN = WAVES_N * TN * 32;
    static constexpr int NT = 64 * WAVES_M * WAVES_N;
    static constexpr int NTILES = BN / 32;
    static constexpr int kBKB = BKB;
    static constexpr int kWM = WAVES_M, kWN = WAVES_N, kTM = TM, kTN = TN;
};

template <class C, bool GROUPED>
__global__ __launch_bounds__(C::NT) void gemm_tiled_kernel(GemmArgs a) {
    constexpr int BM = C::BM, BKB = C::kBKB, NTILES = C::NTILES;
    constexpr int TM = C::kTM, TN = C::kTN, NT = C::NT;
    __shared__ uint4 sA[BKB][BM];               // packed activation codes
    __shared__ uint2 sB[BKB][NTILES][64];       // packed weight codes, MFMA lane order
    __shared__ __attribute__((aligned(16))) float sSa[BKB][BM];  // activation scales
    __shared__ float sDw[BKB][NTILES * 32];     // weight scales / 256
    __shared__ int sArow[BM];                   // activation row of each tile row, -1 if none
    __shared__ int sOrow[BM];                   // output row

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / C::kWN, wn = wave % C::kWN;
    const int g = lane >> 5, c = lane & 31;
    const int64_t k = a.k, nb = k / QK;
    const int64_t tiles_n = padded_n(a.n) / TILE_N;
    const int64_t tile0 = (int64_t)blockIdx.x * NTILES;

    int valid_rows;
    const uint8_t *wbase = a.packed;
    if constexpr (GROUPED) {
        const int ty = blockIdx.y;
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
        const int64_t row0 = (int64_t)blockIdx.y * BM;
        valid_rows = (int)min((int64_t)BM, a.m - row0);
        for (int r = tid; r < BM; r += NT) {
            sArow[r] = r < valid_rows ? (int)(row0 + r) : -1;
            sOrow[r] = (int)(row0 + r);
        }
    }
    const uint8_t *wcodes = wbase;
    const uint16_t *wscales = reinterpret_cast<const uint16_t *>(wbase + packed_code_bytes(a.n, k));
    __syncthreads();

    float acc[TM][TN][16];
#pragma unroll
    for (int i = 0; i < TM; i++)
#pragma unroll
        for (int j = 0; j < TN; j++)
#pragma unroll
            for (int v = 0; v < 16; v++) acc[i][j][v] = 0.0f;

    const int wrow0 = wm * TM * 32;  // first tile row of this wave
    for (int64_t kb0 = 0; kb0 < nb; kb0 += BKB) {
        // ---- stage BKB blocks into LDS ----
        for (int i = tid; i < BM * BKB; i += NT) {
            const int r = i / BKB, bb = i % BKB;
            const int ar = sArow[r];
            uint4 v = make_uint4(0, 0, 0, 0);
            float s = 0.0f;
            if (ar >= 0 && kb0 + bb < nb) {
                v = *reinterpret_cast<const uint4 *>(a.codes + (int64_t)ar * (k / 2) + (kb0 + bb) * 16);
                s = a.scales[(int64_t)ar * nb + kb0 + bb];
            }
            sA[bb][r] = v;
            sSa[bb][r] = s;
        }
        for (int i = tid; i < NTILES * BKB * 32; i += NT) {
            const int t = i / (BKB * 32), rem = i % (BKB * 32), bb = rem / 32, q = rem % 32;
            const int64_t tile = tile0 + t;
            uint4 v = make_uint4(0, 0, 0, 0);
            if (tile < tiles_n && kb0 + bb < nb)
                v = reinterpret_cast<const uint4 *>(wcodes + (tile * nb + kb0 + bb) * TILE_CODE_BYTES)[q];
            reinterpret_cast<uint4 *>(&sB[bb][t][0])[q] = v;
        }
        for (int i = tid; i < NTILES * BKB * 32; i += NT) {
            const int t = i / (BKB * 32), rem = i % (BKB * 32), bb = rem / 32, cc = rem % 32;
            const int64_t tile = tile0 + t;
            float d = 0.0f;
            if (tile < tiles_n && kb0 + bb < nb)
                d = __half2float(__ushort_as_half(wscales[(tile * nb + kb0 + bb) * TILE_SCALE_HALFS + cc]));
            sDw[bb][t * 32 + cc] = d * (1.0f / 256.0f);  // exact: undoes the 16 x 16 operand scaling
        }
        __syncthreads();

        // ---- compute ----
#pragma unroll
        for (int bb = 0; bb < BKB; bb++) {
            v4i af[TM], bf[TN];
#pragma unroll
            for (int i = 0; i < TM; i++) {
                const uint2 p = reinterpret_cast<const uint2 *>(&sA[bb][wrow0 + i * 32 + c])[g];
                af[i] = unpack_nibbles_x16(p.x, p.y);
            }
#pragma unroll
            for (int j = 0; j < TN; j++) {
                const uint2 p = sB[bb][wn * TN + j][lane];
                bf[j] = unpack_nibbles_x16(p.x, p.y);
            }
            float dw[TN];
#pragma unroll
            for (int j = 0; j < TN; j++) dw[j] = sDw[bb][(wn * TN + j) * 32 + c];
#pragma unroll
            for (int i = 0; i < TM; i++) {
                if (wrow0 + i * 32 >= valid_rows) continue;  // uniform: tile rows all empty
                float sa[16];
#pragma unroll
                for (int q = 0; q < 4; q++) {
                    const float4 s4 = *reinterpret_cast<const float4 *>(&sSa[bb][wrow0 + i * 32 + 8 * q + 4 * g]);
                    sa[4 * q + 0] = s4.x; sa[4 * q + 1] = s4.y; sa[4 * q + 2] = s4.z; sa[4 * q + 3] = s4.w;
                }
#pragma unroll
                for (int j = 0; j < TN; j++) {
                    const v16i S = mfma_i8_32x32x32(af[i], bf[j]);
#pragma unroll
                    for (int v = 0; v < 16; v++)
                        acc[i][j][v] = fmaf((float)S[v], sa[v] * dw[j], acc[i][j][v]);
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
// Small-M kernel (m <= 16): weight streaming.  One workgroup per 32-column
// tile; its W waves take interleaved K blocks, each weight byte is read from
// HBM exactly once, the activation scales are staged in LDS per chunk, and
// the waves' partial sums are reduced in LDS before one store.
// -------------------------------------------------------------------------
constexpr int SMALL_M_MAX = 16;
constexpr int SMALL_CHUNK = 256;  // blocks of activation scales staged per pass

template <int W>
__global__ __launch_bounds__(64 * W) void gemm_small_m_kernel(GemmArgs a) {
    __shared__ __attribute__((aligned(16))) float sSa[SMALL_CHUNK][SMALL_M_MAX];
    __shared__ float sRed[W][8][64];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 5, c = lane & 31;
    const int64_t k = a.k, nb = k / QK;
    const int64_t tile = blockIdx.x;
    const int m = (int)a.m;
    const uint2 *wcodes = reinterpret_cast<const uint2 *>(a.packed) + tile * nb * 64;
    const uint16_t *wscales =
        reinterpret_cast<const uint16_t *>(a.packed + packed_code_bytes(a.n, k)) + tile * nb * TILE_SCALE_HALFS;
    const bool arow_ok = c < m;
    const uint8_t *arow = a.codes + (int64_t)(arow_ok ? c : 0) * (k / 2) + 8 * g;

    float acc[8];
#pragma unroll
    for (int v = 0; v < 8; v++) acc[v] = 0.0f;

    for (int64_t cb = 0; cb < nb; cb += SMALL_CHUNK) {
        const int chunk = (int)min((int64_t)SMALL_CHUNK, nb - cb);
        for (int i = tid; i < chunk * SMALL_M_MAX; i += 64 * W) {
            const int bb = i / SMALL_M_MAX, r = i % SMALL_M_MAX;
            sSa[bb][r] = r < m ? a.scales[(int64_t)r * nb + cb + bb] : 0.0f;
        }
        __syncthreads();
        for (int bb = wave; bb < chunk; bb += W) {
            const int64_t b = cb + bb;
            const uint2 wp = wcodes[b * 64 + lane];
            const float dw = __half2float(__ushort_as_half(wscales[b * TILE_SCALE_HALFS + c])) * (1.0f / 256.0f);
            uint2 ap = make_uint2(0, 0);
            if (arow_ok) ap = *reinterpret_cast<const uint2 *>(arow + b * 16);
            const v16i S = mfma_i8_32x32x32(unpack_nibbles_x16(ap.x, ap.y), unpack_nibbles_x16(wp.x, wp.y));
            const float4 s0 = *reinterpret_cast<const float4 *>(&sSa[bb][4 * g]);
            const float4 s1 = *reinterpret_cast<const float4 *>(&sSa[bb][8 + 4 * g]);
            acc[0] = fmaf((float)S[0], s0.x * dw, acc[0]);
            acc[1] = fmaf((float)S[1], s0.y * dw, acc[1]);
            acc[2] = fmaf((float)S[2], s0.z * dw, acc[2]);
            acc[3] = fmaf((float)S[3], s0.w * dw, acc[3]);
            acc[4] = fmaf((float)S[4], s1.x * dw, acc[4]);
            acc[5] = fmaf((float)S[5], s1.y * dw, acc[5]);
            acc[6] = fmaf((float)S[6], s1.z * dw, acc[6]);
            acc[7] = fmaf((float)S[7], s1.w * dw, acc[7]);
        }
        __syncthreads();
    }
#pragma unroll
    for (int v = 0; v < 8; v++) sRed[wave][v][lane] = acc[v];
    __syncthreads();
    for (int i = tid; i < 8 * 64; i += 64 * W) {
        const int v = i / 64, l = i % 64;
        float s = 0.0f;
#pragma unroll
        for (int w = 0; w < W; w++) s += sRed[w][v][l];
        const int r = mfma32_row(v, l);
        const int64_t col = tile * 32 + (l & 31);
        if (r < m && col < a.n) a.y[(int64_t)r * a.ldy + col] = s;
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
