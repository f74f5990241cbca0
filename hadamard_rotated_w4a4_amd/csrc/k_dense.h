// Dense W4A4 GEMM for m > 16 on the gfx950 matrix cores.
//
// 1bit-MONSTER engine docs, "The lean option: ROCmFP4, ROCmI4 and Hadamard
// Q4_0", section "Hadamard-rotated Q4_0: W4A4 prompt processing": int4
// weights times int4 rotated activations on the matrix units, each block's
// integer dot scaled into fp32.
//
// The integer dot of one Q4_0 block for a 32x32 output tile is one
// v_mfma_scale_f32_32x32x64_f8f6f4 with FP6 E2M3 operands: every code q in
// [-8, 7] is exactly q / 8 in E2M3, each product is exact and every partial
// sum is a multiple of 1/64 far below 2^24, so the fp32 result is the integer
// dot S exactly (scaled by 1/64).  Each K half of the instruction carries 16
// of the block's 32 codes (padded with zeros), so a lane reads 12 bytes of
// operand per block.  The MFMA hands back fp32, so the epilogue needs no
// int -> float convert.
//
// Per 32x32 tile and block the exact epilogue is one fp32 multiply-add per
// output, y += (s[m] * d_w[n]) * S.  The scale product P = s (x) d_w is an
// outer product formed by a bf16 MFMA over exact splits of the scales
// (s = s1 + s2 + s3, 64 d_w = d1 + d2, all six partial products exact in
// fp32).  So a tile and block cost two MFMAs and 16 vector multiply-adds per
// lane; on gfx950 vector and matrix instructions of one SIMD overlap only
// partly, and this kernel keeps every other vector instruction out of the
// loop: operands arrive in the MFMA's register layout (weights repacked
// offline, activations by a pre-pass), by direct global-to-LDS loads.
//
// Workgroup: 4 waves (2 x 2), each owning TM x TN tiles of 32x32 (a 128 x 128
// output tile for 2 x 2).  K is walked in stages of BKB blocks through a ring
// of NS LDS stage buffers; NS - 1 stages are in flight while one is computed.
#pragma once

#include "common.h"
#include "k_route.h"

namespace w4a4 {

typedef int v8i __attribute__((ext_vector_type(8)));

// ---------------------------------------------------------------------------
// Activation pre-pass: int4 codes [m][k/2] + fp32 scales [m][k/32] -> operand
// records [ceil(m/32)][nbp][1 KB] (same shape as the weight records):
//   [0, 768)    fp6 E2M3 codes of row r, laid out as for the weights;
//   [768, 1024) per row the bf16 split {s1, s2, s3, 0} of the scale, read by
//               both lane groups of the scale-product MFMA.
// One thread per (row, padded block); padding rows and blocks are zero.
// ---------------------------------------------------------------------------
// Row r (of 32) of record `rec`: block b of activation row `src` (codes and
// scales as the rotate-quantiser writes them), or zeros for src < 0 and for
// padding blocks.
__device__ __forceinline__ void write_act_record(const uint8_t *__restrict__ codes,
                                                 const float *__restrict__ scales, int64_t src, int64_t k,
                                                 int64_t b, uint8_t *rec, int r) {
    const int64_t nb = k / QK;
    uint32_t lo[3] = {0, 0, 0}, hi[3] = {0, 0, 0};
    uint2 sop = make_uint2(0, 0);
    if (src >= 0 && b < nb) {
        const int64_t row = src;
        const uint4 q = *reinterpret_cast<const uint4 *>(codes + row * (k / 2) + b * 16);
        const uint32_t qw[4] = {q.x, q.y, q.z, q.w};
        uint32_t f0[16], f1[16];
#pragma unroll
        for (int j = 0; j < 16; j++) {
            const uint32_t byte = (qw[j >> 2] >> (8 * (j & 3))) & 0xFFu;
            f0[j] = fp6_e2m3_of(((int)(byte << 28)) >> 28);  // code j: low nibble, two's complement
            f1[j] = fp6_e2m3_of(((int)(byte << 24)) >> 28);  // code j + 16: high nibble
        }
        pack_fp6x16(f0, lo);
        pack_fp6x16(f1, hi);
        // exact bf16 split s = s1 + s2 + s3 (truncations; each remainder is exact)
        const float s = scales[row * nb + b];
        const uint32_t h1 = __float_as_uint(s) & 0xFFFF0000u;
        const float r1 = __fsub_rn(s, __uint_as_float(h1));
        const uint32_t h2 = __float_as_uint(r1) & 0xFFFF0000u;
        const float r2 = __fsub_rn(r1, __uint_as_float(h2));
        const uint32_t h3 = __float_as_uint(r2) & 0xFFFF0000u;
        sop = make_uint2((h1 >> 16) | h2, h3 >> 16);
    }
    put_mx_lane(rec, r, lo);
    put_mx_lane(rec, 32 + r, hi);
    reinterpret_cast<uint2 *>(rec + MX_CODE_BYTES)[r] = sop;
}

__global__ __launch_bounds__(256) void act_operand_kernel(const uint8_t *__restrict__ codes,
                                                          const float *__restrict__ scales, int64_t m,
                                                          int64_t k, uint8_t *__restrict__ ws) {
    const int64_t nbp = mx_blocks(k);
    const int64_t rows = (m + 31) / 32 * 32;
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (gid >= rows * nbp) return;
    // consecutive threads: consecutive rows of one block (coalesced record writes)
    const int64_t b = gid / rows, row = gid % rows;
    write_act_record(codes, scales, row < m ? row : -1, k, b, ws + ((row / 32) * nbp + b) * MX_REC,
                     (int)(row % 32));
}

// ---------------------------------------------------------------------------
// The GEMM.
// ---------------------------------------------------------------------------
struct MxArgs {
    const uint8_t *act;     // activation records [rtiles][nbp][1 KB]
    const uint8_t *wrec;    // weight records [tiles_n][nbp][1 KB]
    float *y;
    int64_t ldy, m, n, k;
};

template <int BKB_, int NS_, int TM_, int TN_>
struct MxCfg {
    static constexpr int BKB = BKB_, NS = NS_;
    static constexpr int TM = TM_, TN = TN_, WM = 2, WN = 2, NT = 256;
    static constexpr int BM = WM * TM * 32, BN = WN * TN * 32;
    static constexpr int RT = BM / 32, CT = BN / 32;
    static constexpr int STAGE_BYTES = (RT + CT) * BKB * MX_REC;
    static constexpr int DMA_PER_STAGE = (RT + CT) * BKB;  // 1 KB each
    static constexpr int DMA_PER_WAVE = DMA_PER_STAGE / 4;
    static_assert(DMA_PER_STAGE % 4 == 0, "loads split evenly over the 4 waves");
    static_assert(MX_BLOCK_PAD % BKB == 0, "stages tile the padded block range");
};

// LDS reads of one fragment.  They are volatile so that the compiler never
// merges reads of two different fragments into one instruction (that would
// scatter a fragment over non-adjacent registers and cost moves and early
// waits); immediate offsets still fold.
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
template <class T>
__device__ __forceinline__ T lds_read(const uint8_t *p) {
    return *reinterpret_cast<const volatile __attribute__((address_space(3))) T *>(
        (const __attribute__((address_space(3))) uint8_t *)p);
}

// One global-to-LDS load of 16 bytes per lane: lane l's bytes at `g` land at
// LDS byte address lds + 16 l (lds is wave-uniform, passed through M0).
__device__ __forceinline__ void dma16(const void *g, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(lds) : "memory");
}

// Workgroup tile of index id in an XCD-aware order.  Workgroups are dealt to
// the 8 XCDs round-robin, so ids x, x + 8, x + 16, ... share an XCD and its
// L2; the row tiles of one weight column tile get ids x + 8y and read those
// weights from HBM about once.  nx, ny: column and row tiles of the matrix.
__device__ __forceinline__ void mx_tile_of(int64_t id, int64_t nx, int64_t ny, int64_t &bx, int64_t &by) {
    constexpr int64_t XCDS = 8;
    const int64_t group = id / (XCDS * ny), in = id % (XCDS * ny);
    const int64_t width = min(XCDS, nx - group * XCDS);
    bx = group * XCDS + in % width;
    by = in / width;
}

// One whole tile (workgroup index id) of the main kernel.
template <class C>
__device__ __forceinline__ void mx_tile(const MxArgs &a, int64_t id, uint8_t *smem) {
    constexpr int BKB = C::BKB, NS = C::NS, TM = C::TM, TN = C::TN, RT = C::RT;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / C::WN, wn = wave % C::WN;
    const int g = lane >> 5, c = lane & 31;
    const int64_t nbp = mx_blocks(a.k);
    const int64_t rtiles = (a.m + 31) / 32, ctiles = padded_n(a.n) / TILE_N;

    int64_t bx, by;
    mx_tile_of(id, (a.n + C::BN - 1) / C::BN, (a.m + C::BM - 1) / C::BM, bx, by);
    const int64_t rt0 = by * RT, ct0 = bx * C::CT;

    // ---- this wave's loads: DMA_PER_WAVE records of 1 KB per stage ----
    // load i = wave * DMA_PER_WAVE + d covers tile i / BKB (row tiles first,
    // then column tiles), block i % BKB of the stage.  Tiles past the matrix
    // edge are clamped to the last one (their outputs are never stored).
    const uint8_t *src[C::DMA_PER_WAVE];
    uint32_t dst[C::DMA_PER_WAVE];
    const uint32_t smem_base = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)smem;
#pragma unroll
    for (int d = 0; d < C::DMA_PER_WAVE; d++) {
        const int i = wave * C::DMA_PER_WAVE + d, t = i / BKB, bb = i % BKB;
        const uint8_t *base = t < RT ? a.act + min(rt0 + t, rtiles - 1) * nbp * MX_REC
                                     : a.wrec + min(ct0 + t - RT, ctiles - 1) * nbp * MX_REC;
        src[d] = base + bb * MX_REC + lane * 16;
        dst[d] = (uint32_t)((t * BKB + bb) * MX_REC);
    }
    const int nstages = (int)(nbp / BKB);
    auto issue = [&](int stage, int slot) {
        // past the last stage the ring keeps reloading the last one (its
        // slot is never computed): the count of loads in flight stays fixed
        const int64_t kb0 = (int64_t)min(stage, nstages - 1) * BKB;
        const uint32_t lds = __builtin_amdgcn_readfirstlane(smem_base + slot * C::STAGE_BYTES);
#pragma unroll
        for (int d = 0; d < C::DMA_PER_WAVE; d++) dma16(src[d] + kb0 * MX_REC, lds + dst[d]);
    };

    // scale-product operand of the weights: lane group g reads {d_g, d_g, d_g, 0}
    const uint32_t sel0 = g ? 0x03020302u : 0x01000100u, sel1 = g ? 0x0C0C0302u : 0x0C0C0100u;

    v16f acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; i++)
#pragma unroll
        for (int j = 0; j < TN; j++)
#pragma unroll
            for (int v = 0; v < 16; v++) acc[i][j][v] = 0.0f;

    // ---- one software pipeline over all blocks ----
    // Step t of a stage = (block t / PER, tile t % PER).  The two MFMAs of
    // step t + 1 are issued around the first half of step t's multiply-adds;
    // the operands of the next block are read while the current one computes
    // (the weights' scale word is expanded only where it is used, so nothing
    // waits for those reads early).  The wait + barrier that publishes stage
    // s + 1 sits at the start of stage s's last block, so the pipeline never
    // drains at a stage boundary.
    static_assert(BKB % 2 == 0, "operand buffers alternate per block");
    static_assert(NS >= 3, "one stage in flight besides the two in use");
    constexpr int STEPS = BKB * TM * TN, PER = TM * TN;
    v8i af[2][TM] = {}, bf[2][TN] = {};  // operand dwords 3..7 are zero
    uint2 ap[2][TM];
    uint32_t bw[2][TN];
    auto load_frags = [&](const uint8_t *st, int bb, int buf) {
#pragma unroll
        for (int i = 0; i < TM; i++) {
            const uint8_t *rec = st + ((wm * TM + i) * BKB + bb) * MX_REC;
            const u32x2 f01 = lds_read<u32x2>(rec + 8 * lane);
            const uint32_t f2 = lds_read<uint32_t>(rec + 512 + 4 * lane);
            af[buf][i][0] = (int)f01.x;  // elements 3..7 stay zero
            af[buf][i][1] = (int)f01.y;
            af[buf][i][2] = (int)f2;
            const u32x2 sp = lds_read<u32x2>(rec + MX_CODE_BYTES + 8 * c);
            ap[buf][i] = make_uint2(sp.x, sp.y);
        }
#pragma unroll
        for (int j = 0; j < TN; j++) {
            const uint8_t *rec = st + ((RT + wn * TN + j) * BKB + bb) * MX_REC;
            const u32x2 f01 = lds_read<u32x2>(rec + 8 * lane);
            const uint32_t f2 = lds_read<uint32_t>(rec + 512 + 4 * lane);
            bf[buf][j][0] = (int)f01.x;
            bf[buf][j][1] = (int)f01.y;
            bf[buf][j][2] = (int)f2;
            bw[buf][j] = lds_read<uint32_t>(rec + MX_CODE_BYTES + 4 * c);
        }
    };
    auto mfma_s = [&](int buf, int i, int j) {
        return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af[buf][i], bf[buf][j], v16f{}, 2, 2, 0, 0, 0, 0);
    };
    auto mfma_p = [&](int buf, int i, int j) {
        const uint32_t w = bw[buf][j];
        return mfma_bf16_32x32x8(ap[buf][i], make_uint2(__builtin_amdgcn_perm(w, w, sel0), __builtin_amdgcn_perm(w, w, sel1)));
    };

#pragma unroll
    for (int x = 0; x < NS - 1; x++) issue(x, x);
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(C::DMA_PER_WAVE * (NS - 2)) : "memory");
    __syncthreads();
    v16f S[2], P[2];
    load_frags(smem, 0, 0);
    S[0] = mfma_s(0, 0, 0);
    P[0] = mfma_p(0, 0, 0);

    for (int s = 0; s < nstages; s++) {
        const uint8_t *st = smem + (s % NS) * C::STAGE_BYTES;
#pragma unroll
        for (int t = 0; t < STEPS; t++) {
            const int bb = t / PER, i = (t / TN) % TM, j = t % TN;
            if (t % PER == 0) {
                if (bb + 1 < BKB) {
                    load_frags(st, bb + 1, (bb + 1) & 1);
                } else {
                    // stage s + 1 has landed for this wave; after the barrier
                    // for every wave, and stage s - 1's slot is no longer read.
                    // (After the last stage this reads a reloaded stage; the
                    // MFMAs it feeds are never consumed.)
                    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(C::DMA_PER_WAVE * (NS - 3)) : "memory");
                    __syncthreads();
                    issue(s + NS - 1, (s + NS - 1) % NS);
                    load_frags(smem + ((s + 1) % NS) * C::STAGE_BYTES, 0, 0);
                }
            }
            const int t1 = (t + 1) % STEPS, b1 = (t1 / PER) & 1, i1 = (t1 / TN) % TM, j1 = t1 % TN;
            S[(t + 1) & 1] = mfma_s(b1, i1, j1);
#pragma unroll
            for (int v = 0; v < 8; v++) acc[i][j][v] = fmaf(S[t & 1][v], P[t & 1][v], acc[i][j][v]);
            __builtin_amdgcn_sched_barrier(0x0004 | 0x0010 | 0x0080);
            P[(t + 1) & 1] = mfma_p(b1, i1, j1);
#pragma unroll
            for (int v = 8; v < 16; v++) acc[i][j][v] = fmaf(S[t & 1][v], P[t & 1][v], acc[i][j][v]);
            asm volatile("" : "+v"(acc[i][j]));  // materialised here, not sunk past the loop's end
            __builtin_amdgcn_sched_barrier(0x0004 | 0x0010 | 0x0080);
        }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // no load may still be writing LDS at exit

    // ---- store ----
#pragma unroll
    for (int i = 0; i < TM; i++) {
        const int64_t rbase = (rt0 + wm * TM + i) * 32;
#pragma unroll
        for (int j = 0; j < TN; j++) {
            const int64_t col = (ct0 + wn * TN + j) * 32 + c;
            if (col >= a.n) continue;
#pragma unroll
            for (int v = 0; v < 16; v++) {
                const int64_t r = rbase + mfma32_row(v, lane);
                if (r < a.m) a.y[r * a.ldy + col] = acc[i][j][v];
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Leftover tiles.  When the workgroup tiles of a problem do not fill whole
// rounds of the GPU, whole tiles take the whole rounds and pieces the rest:
// each such workgroup computes one 32x32 piece of a leftover tile, its 4
// waves each over a quarter of K, and the quarters meet in LDS.  A wave
// streams its own operand records through its own LDS ring (no barrier until
// the reduction), two MFMAs and 16 multiply-adds per block as above.
// ---------------------------------------------------------------------------
template <int BM_, int BN_>
struct MxPieceCfg {
    static constexpr int BM = BM_, BN = BN_;                 // tile shape of the main kernel
    static constexpr int PIECES = (BM / 32) * (BN / 32);     // 32x32 pieces per leftover tile
    static constexpr int BKB = 2, NS = 4, NT = 256;          // per wave: NS stages of BKB blocks
    static constexpr int WAVE_RING = NS * BKB * 2 * MX_REC;  // A and B record per block
};

template <class C>
__device__ __forceinline__ void mx_piece(const MxArgs &a, int64_t first_tile, int64_t id, uint8_t *smem) {
    constexpr int BKB = C::BKB, NS = C::NS;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 5, c = lane & 31;
    const int64_t nbp = mx_blocks(a.k);
    const int64_t rtiles = (a.m + 31) / 32, ctiles = padded_n(a.n) / TILE_N;

    int64_t bx, by;
    mx_tile_of(first_tile + id / C::PIECES, (a.n + C::BN - 1) / C::BN, (a.m + C::BM - 1) / C::BM, bx, by);
    const int sub = (int)(id % C::PIECES);
    const int64_t rt = by * (C::BM / 32) + sub / (C::BN / 32), ct = bx * (C::BN / 32) + sub % (C::BN / 32);
    // pieces past the matrix edge compute on clamped tiles and store nothing
    const uint8_t *arec = a.act + min(rt, rtiles - 1) * nbp * MX_REC;
    const uint8_t *brec = a.wrec + min(ct, ctiles - 1) * nbp * MX_REC;

    // this wave's quarter of the blocks, in whole stages
    const int64_t nstages_all = nbp / BKB;
    const int64_t s_begin = nstages_all * wave / 4, s_end = nstages_all * (wave + 1) / 4;
    const int nst = (int)(s_end - s_begin);
    uint8_t *ring = smem + wave * C::WAVE_RING;
    const uint32_t ring_lds =
        __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)ring);
    auto issue = [&](int stage, int slot) {
        // past the last stage the ring reloads the last one (never computed)
        const int64_t kb0 = (s_begin + min(stage, max(nst - 1, 0))) * BKB;
        const uint32_t lds = ring_lds + slot * BKB * 2 * MX_REC;
#pragma unroll
        for (int bb = 0; bb < BKB; bb++) {
            dma16(arec + (kb0 + bb) * MX_REC + lane * 16, lds + (2 * bb) * MX_REC);
            dma16(brec + (kb0 + bb) * MX_REC + lane * 16, lds + (2 * bb + 1) * MX_REC);
        }
    };
    const uint32_t sel0 = g ? 0x03020302u : 0x01000100u, sel1 = g ? 0x0C0C0302u : 0x0C0C0100u;

    v16f acc;
#pragma unroll
    for (int v = 0; v < 16; v++) acc[v] = 0.0f;
    // Pipeline: the two MFMAs of block bb + 1 are issued before the
    // multiply-adds of block bb (one tile per wave leaves nothing else to
    // cover the MFMA latency).
    auto mfmas = [&](const uint8_t *st, int bb, v16f &S, v16f &P) {
        const uint8_t *ra = st + (2 * bb) * MX_REC, *rb = st + (2 * bb + 1) * MX_REC;
        v8i af = {}, bf = {};  // operand dwords 3..7 are zero
        const u32x2 a01 = lds_read<u32x2>(ra + 8 * lane), b01 = lds_read<u32x2>(rb + 8 * lane);
        af[0] = (int)a01.x; af[1] = (int)a01.y; af[2] = (int)lds_read<uint32_t>(ra + 512 + 4 * lane);
        bf[0] = (int)b01.x; bf[1] = (int)b01.y; bf[2] = (int)lds_read<uint32_t>(rb + 512 + 4 * lane);
        const u32x2 sp = lds_read<u32x2>(ra + MX_CODE_BYTES + 8 * c);
        const uint32_t w = lds_read<uint32_t>(rb + MX_CODE_BYTES + 4 * c);
        S = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af, bf, v16f{}, 2, 2, 0, 0, 0, 0);
        P = mfma_bf16_32x32x8(make_uint2(sp.x, sp.y),
                              make_uint2(__builtin_amdgcn_perm(w, w, sel0), __builtin_amdgcn_perm(w, w, sel1)));
    };
    if (nst > 0) {
#pragma unroll
        for (int x = 0; x < NS - 1; x++) issue(x, x);
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * BKB * (NS - 2)) : "memory");  // stage 0 has landed
        v16f S[2], P[2];
        mfmas(ring, 0, S[0], P[0]);
        for (int s = 0; s < nst; s++) {
            const uint8_t *st = ring + (s % NS) * BKB * 2 * MX_REC;
#pragma unroll
            for (int bb = 0; bb < BKB; bb++) {
                if (bb + 1 < BKB) {
                    mfmas(st, bb + 1, S[(bb + 1) & 1], P[(bb + 1) & 1]);
                } else {
                    // next stage: refill the slot computed last, wait for stage s + 1
                    // (after the last stage this reads a reloaded stage; unused)
                    issue(s + NS - 1, (s + NS - 1) % NS);
                    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * BKB * (NS - 2)) : "memory");
                    mfmas(ring + ((s + 1) % NS) * BKB * 2 * MX_REC, 0, S[(bb + 1) & 1], P[(bb + 1) & 1]);
                }
#pragma unroll
                for (int v = 0; v < 16; v++) acc[v] = fmaf(S[bb & 1][v], P[bb & 1][v], acc[v]);
                asm volatile("" : "+v"(acc));
                __builtin_amdgcn_sched_barrier(0x0004 | 0x0010 | 0x0080);
            }
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // no load may still be writing the ring
    }

    // the quarters meet in LDS (the rings are free now) in ascending K order
    __syncthreads();
    float *red = reinterpret_cast<float *>(smem);
#pragma unroll
    for (int v = 0; v < 16; v++) red[(wave * 16 + v) * 64 + lane] = acc[v];
    __syncthreads();
    for (int i = tid; i < 16 * 64; i += C::NT) {
        const int v = i / 64, l = i % 64;
        const float sum = ((red[(0 * 16 + v) * 64 + l] + red[(1 * 16 + v) * 64 + l]) + red[(2 * 16 + v) * 64 + l]) +
                          red[(3 * 16 + v) * 64 + l];
        const int64_t r = rt * 32 + mfma32_row(v, l), col = ct * 32 + (l & 31);
        if (rt < rtiles && r < a.m && col < a.n) a.y[r * a.ldy + col] = sum;
    }
}

// One launch for a whole product: workgroups below main_wgs take whole tiles
// (in the XCD-aware order), the rest take the pieces of the leftover tiles.
// Workgroups are dispatched in index order, so the pieces fill the CUs that
// the last whole tiles leave idle, without a second launch and its gap.
template <class C>
__global__ __launch_bounds__(C::NT) void gemm_mx_kernel(MxArgs a, int64_t main_wgs, int64_t first_piece_tile) {
    using P = MxPieceCfg<C::BM, C::BN>;
    static_assert(P::NT == C::NT, "one workgroup size for both kinds");
    constexpr int MAIN_LDS = C::NS * C::STAGE_BYTES, PIECE_LDS = 4 * P::WAVE_RING;
    __shared__ __attribute__((aligned(1024))) uint8_t smem[MAIN_LDS > PIECE_LDS ? MAIN_LDS : PIECE_LDS];
    if ((int64_t)blockIdx.x < main_wgs) mx_tile<C>(a, blockIdx.x, smem);  // uniform per workgroup
    else mx_piece<P>(a, first_piece_tile, blockIdx.x - main_wgs, smem);
}

}  // namespace w4a4
