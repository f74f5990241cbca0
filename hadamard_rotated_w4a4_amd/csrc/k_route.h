// MUL_MAT_ID routing and small helpers of the expert-routed product.
//
// 1bit-MONSTER engine docs, "The lean option: ROCmFP4, ROCmI4 and Hadamard
// Q4_0", section "MoE: W4A4 on the experts": the expert matmuls
// (MUL_MAT_ID) take the same W4A4 path as the dense ones; the rows routed to
// one expert are multiplied by that expert's weights.
#pragma once

#include "common.h"

namespace w4a4 {

// Expert routing as the grouped kernels read it: rows grouped by expert
// (perm), each expert's rows padded to whole tiles of the kernel's row count;
// tile_prefix[e] counts the tiles of experts before e.
struct Routing {
    const int32_t *perm;         // [n_rows] (token, slot) row ids, grouped by expert
    const int32_t *offsets;      // [E + 1] start of each expert's rows in perm
    const int32_t *tile_prefix;  // [E + 1]
    int n_expert;
};
// Expert of row tile t < tile_prefix[E]: the largest e with tile_prefix[e] <= t.
__device__ __forceinline__ int expert_of_tile(const Routing &g, int64_t t) {
    int lo = 0, hi = g.n_expert;
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (g.tile_prefix[mid] <= t) lo = mid; else hi = mid;
    }
    return lo;
}

// -------------------------------------------------------------------------
// MUL_MAT_ID routing: one workgroup groups the (token, slot) rows by expert
// and counts each expert's row tiles; rows with an invalid id go to the end
// of the permutation (perm[offsets[E] ..]), where the GEMM zeroes their
// output rows.  The routing depends on the ids alone, so one routing serves
// every product of a layer that reads the same ids.
// -------------------------------------------------------------------------
constexpr int ROUTE_THREADS = 1024;
constexpr int ROUTE_MAX_EXPERTS = 8192;
constexpr int ROUTE_KEEP = 16;  // ids per thread held in registers between the two passes

// One workgroup.  Counting lives in LDS, so every count and cursor update is
// seen by the whole workgroup after a barrier.  The ids are read once (up to
// ROUTE_KEEP per thread stay in registers for the scatter); the scans over
// the experts are wave scans plus one scan of the wave totals.
__global__ __launch_bounds__(ROUTE_THREADS) void route_kernel(const int32_t *__restrict__ ids, int n_rows,
                                                              int n_expert, int tile_rows,
                                                              int32_t *__restrict__ offsets,
                                                              int32_t *__restrict__ tile_prefix,
                                                              int32_t *__restrict__ perm) {
    __shared__ int cnt[ROUTE_MAX_EXPERTS];
    __shared__ int wrow[ROUTE_THREADS / 64], wtile[ROUTE_THREADS / 64];
    __shared__ int bad_cursor;  // next slot for a row with an invalid id
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    for (int e = tid; e < n_expert; e += ROUTE_THREADS) cnt[e] = 0;
    __syncthreads();
    int mine[ROUTE_KEEP];
#pragma unroll
    for (int q = 0; q < ROUTE_KEEP; q++) {
        const int i = tid + q * ROUTE_THREADS;
        mine[q] = i < n_rows ? ids[i] : -1;
    }
#pragma unroll
    for (int q = 0; q < ROUTE_KEEP; q++)
        if (mine[q] >= 0 && mine[q] < n_expert) atomicAdd(&cnt[mine[q]], 1);
    for (int i = tid + ROUTE_KEEP * ROUTE_THREADS; i < n_rows; i += ROUTE_THREADS) {
        const int e = ids[i];
        if (e >= 0 && e < n_expert) atomicAdd(&cnt[e], 1);
    }
    __syncthreads();
    // exclusive scans of row counts and of row tiles; thread t owns a
    // contiguous chunk of experts
    const int per = (n_expert + ROUTE_THREADS - 1) / ROUTE_THREADS;
    const int e0 = min(tid * per, n_expert), e1 = min(e0 + per, n_expert);
    int s = 0, ts = 0;
    for (int e = e0; e < e1; e++) { s += cnt[e]; ts += (cnt[e] + tile_rows - 1) / tile_rows; }
    int is = s, its = ts;  // inclusive scan within the wave
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int a = __shfl_up(is, d), b = __shfl_up(its, d);
        if (lane >= d) { is += a; its += b; }
    }
    if (lane == 63) { wrow[wave] = is; wtile[wave] = its; }
    __syncthreads();
    int before = 0, tbefore = 0;  // totals of the waves before this one
    for (int w = 0; w < wave; w++) { before += wrow[w]; tbefore += wtile[w]; }
    int run = before + is - s, trun = tbefore + its - ts;
    for (int e = e0; e < e1; e++) {
        const int ce = cnt[e];
        offsets[e] = run;
        tile_prefix[e] = trun;
        cnt[e] = run;  // becomes the expert's scatter cursor
        run += ce;
        trun += (ce + tile_rows - 1) / tile_rows;
    }
    if (tid == ROUTE_THREADS - 1) {
        offsets[n_expert] = run;
        tile_prefix[n_expert] = trun;
        bad_cursor = run;  // the valid rows end here
    }
    __syncthreads();
    auto place = [&](int i, int e) {
        perm[atomicAdd(e >= 0 && e < n_expert ? &cnt[e] : &bad_cursor, 1)] = i;
    };
#pragma unroll
    for (int q = 0; q < ROUTE_KEEP; q++) {
        const int i = tid + q * ROUTE_THREADS;
        if (i < n_rows) place(i, mine[q]);
    }
    for (int i = tid + ROUTE_KEEP * ROUTE_THREADS; i < n_rows; i += ROUTE_THREADS) place(i, ids[i]);
}

// Fill rows of y with zeros (used when k == 0: an empty sum).
__global__ void zero_rows_kernel(float *y, int64_t m, int64_t n, int64_t ldy) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < m * n; i += stride)
        y[(i / n) * ldy + i % n] = 0.0f;
}

}  // namespace w4a4
