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
// dot S exactly (scaled by 1/64).  A lane's 32 K values are one whole block
// (lanes 32..63 the next block), so one operand register set carries two
// blocks and no zero padding; the MFMA's per-lane E8M0 scales select one
// block: 1 (byte 127) on its lanes, 2^-127 (byte 0) on the other half, for
// A and B alike, so the other block's products are scaled by 2^-254 and round
// away exactly (at most 32 * 2^-254, below half the least fp32 step).  The
// MFMA hands back fp32, so the epilogue needs no int -> float convert.
//
// Per 32x32 tile and block the exact epilogue is one fp32 multiply-add per
// output, y += (s[m] * d_w[n]) * S.  The scale product P = s (x) d_w is an
// outer product, formed on the matrix cores too: the 32x32x4 bf16 MFMA in its
// two-block form gives P for both blocks of a stage in one instruction
// (lane K slots (s_1, s_1, s_2, s_2) against (d_0, d_1, d_0, d_1), with
// 64 d_w = d_0 + d_1 exact and s_1 + s_2 equal to s within 2^-16 relative;
// the four partial products are exact in fp32).  So a tile and a stage of two
// blocks cost two FP6 MFMAs, one scale-product MFMA and 32 vector
// multiply-adds per lane, and every other vector instruction is kept out of
// the loop: operands arrive in the MFMAs' register layouts (weights repacked
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
typedef int v6i __attribute__((ext_vector_type(6)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

// An FP6 operand (six dwords) as the v8i the builtin takes; the last two
// elements are left undefined (the instruction reads six registers for FP6).
__device__ __forceinline__ v8i fp6_operand(u32x2 a, u32x2 b, u32x2 c) {
    const v6i v = {(int)a.x, (int)a.y, (int)b.x, (int)b.y, (int)c.x, (int)c.y};
    return __builtin_shufflevector(v, v, 0, 1, 2, 3, 4, 5, -1, -1);
}

// The register pair {w, w}.  The copy is a byte permute with an identity
// selector the compiler cannot see through (`id_sel` = 0x03020100 from an
// opaque move), so it stays next to its use; a plain copy is coalesced into
// the LDS read of w and makes the wave wait for that read right there.
__device__ __forceinline__ uint2 dup_at_use(uint32_t w, uint32_t id_sel) {
    return make_uint2(w, __builtin_amdgcn_perm(w, w, id_sel));
}
__device__ __forceinline__ uint32_t opaque_identity_selector() {
    uint32_t v;
    asm("v_mov_b32 %0, 0x03020100" : "=v"(v));
    return v;
}

// S / 64 of the block on the lanes whose E8M0 scale byte `sel` is 127 (the
// other half of the lanes gets 0: see the file comment).
__device__ __forceinline__ v16f mfma_block(v8i a, v8i b, int sel) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, v16f{}, 2, 2, 0, sel, 0, sel);
}
// A8: S / 64 of a block from its two planes (a: h in lane group 0, l in lane
// group 1; b: the block's weights in both): the h lanes' block scale is 2^4.
__device__ __forceinline__ v16f mfma_block8(v8i a, v8i b, int g) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, v16f{}, 2, 2, 0, g ? 127 : 131, 0, 127);
}

// ---------------------------------------------------------------------------
// Activation pre-pass: int4 codes [m][k/2] + fp32 scales [m][k/32] -> operand
// records [ceil(m/32)][nbp][1 KB] (same shape as the weight records):
//   [0, 768)    fp6 E2M3 codes of row r, laid out as for the weights;
//   [768, 1024) per row the bf16 quadruple (s1, s1, s2, s2) of the scale,
//               the scale-product MFMA's A operand.
// One thread per (row, padded block); padding rows and blocks are zero.
// ---------------------------------------------------------------------------
// Row r (of 32) of record `rec`: block b of activation row `src` (codes and
// scales as the rotate-quantiser writes them), or zeros for src < 0 and for
// padding blocks.
__device__ __forceinline__ void write_act_record(const uint8_t *__restrict__ codes,
                                                 const float *__restrict__ scales, int64_t src, int64_t k,
                                                 int64_t b, uint8_t *rec, int r) {
    const int64_t nb = k / QK;
    uint32_t w[6] = {0, 0, 0, 0, 0, 0};
    uint2 sop = make_uint2(0, 0);
    if (src >= 0 && b < nb) {
        const int64_t row = src;
        const uint4 q = *reinterpret_cast<const uint4 *>(codes + row * (k / 2) + b * 16);
        const uint32_t qw[4] = {q.x, q.y, q.z, q.w};
        uint32_t f[32];
#pragma unroll
        for (int j = 0; j < 16; j++) {
            const uint32_t byte = (qw[j >> 2] >> (8 * (j & 3))) & 0xFFu;
            f[j] = fp6_e2m3_of(((int)(byte << 28)) >> 28);       // code j: low nibble, two's complement
            f[j + 16] = fp6_e2m3_of(((int)(byte << 24)) >> 28);  // code j + 16: high nibble
        }
        pack_fp6x32(f, w);
        sop = act_scale_operand(scales[row * nb + b]);
    }
    put_mx_row(rec, r, w);
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

// A8 pre-pass: int8 codes [m][k] + fp32 scales [m][k/32] -> two planes of
// operand records per row tile, [ceil(m/32)][2][nbp][1 KB]: plane 0 holds the
// h codes of every code a = 16 h + l (h = (a + 8) >> 4, l = a - 16 h) with
// the scale operand at [768, 1024), plane 1 the l codes with a zero scale
// operand.  One thread per (row, padded block); padding rows and blocks are
// zero.
__global__ __launch_bounds__(256) void act8_operand_kernel(const int8_t *__restrict__ codes,
                                                           const float *__restrict__ scales, int64_t m,
                                                           int64_t k, uint8_t *__restrict__ ws) {
    const int64_t nb = k / QK, nbp = mx_blocks(k);
    const int64_t rows = (m + 31) / 32 * 32;
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (gid >= rows * nbp) return;
    const int64_t b = gid / rows, row = gid % rows;  // consecutive threads: consecutive rows of one block
    uint32_t wh[6] = {0, 0, 0, 0, 0, 0}, wl[6] = {0, 0, 0, 0, 0, 0};
    uint2 sop = make_uint2(0, 0);
    if (row < m && b < nb) {
        const uint4 *q = reinterpret_cast<const uint4 *>(codes + row * k + b * QK);
        const uint4 q0 = q[0], q1 = q[1];
        const uint32_t qw[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
        uint32_t fh[32], fl[32];
#pragma unroll
        for (int j = 0; j < 32; j++) {
            const int a = (int)(int8_t)(qw[j >> 2] >> (8 * (j & 3)));
            const int h = (a + 8) >> 4;  // floor: h in [-8, 8], a - 16 h in [-8, 7]
            fh[j] = fp6_e2m3_of(h);
            fl[j] = fp6_e2m3_of(a - 16 * h);
        }
        pack_fp6x32(fh, wh);
        pack_fp6x32(fl, wl);
        sop = act_scale_operand(scales[row * nb + b]);
    }
    uint8_t *rh = ws + (((row / 32) * 2 + 0) * nbp + b) * MX_REC, *rl = ws + (((row / 32) * 2 + 1) * nbp + b) * MX_REC;
    put_mx_row(rh, (int)(row % 32), wh);
    reinterpret_cast<uint2 *>(rh + MX_CODE_BYTES)[row % 32] = sop;
    put_mx_row(rl, (int)(row % 32), wl);
    reinterpret_cast<uint2 *>(rl + MX_CODE_BYTES)[row % 32] = make_uint2(0, 0);
}

// ---------------------------------------------------------------------------
// The GEMM.
// ---------------------------------------------------------------------------
struct MxArgs {
    const uint8_t *act;     // activation records [rtiles][nbp][1 KB]
    const uint8_t *wrec;    // weight records [tiles_n][nbp][1 KB]
    float *y;
    int64_t ldy, m, n, k;
    int64_t splits = 1;     // K splits of every tile (1: whole K, stored to y)
    float *partial = nullptr;  // splits > 1: [splits][m][n] partial sums
};

// A8: int8 activation codes (the exact int8 path on a rotated file).  Every
// code a is 16 h + l with h = (a + 8) >> 4 in [-8, 8] and l in [-8, 7], both
// exact in E2M3; a row tile's records come in two planes (act8_operand_kernel),
// and one operand register set holds the h plane of a block in lanes 0..31
// and its l plane in lanes 32..63, against the block's weights in both lane
// groups.  One FP6 MFMA with the E8M0 scale 2^4 (byte 131) on the h lanes
// then gives 16 S_h + S_l = S, the integer dot of the int8 codes (over 64),
// exactly (|S| <= 127 * 8 * 32): a block costs one block-dot MFMA, as in
// W4A4, with no lanes masked.  A stage holds BKB blocks (1 or 2), each with
// its own operand registers, and the scale products are single-block
// 32x32x8 bf16 MFMAs (the l plane's scale operand is zero, so the second
// lane group adds nothing).
template <int BKB_, int NS_, int TM_, int TN_, bool A8_ = false>
struct MxCfg {
    static constexpr int BKB = BKB_, NS = NS_;
    static constexpr int TM = TM_, TN = TN_, WM = 2, WN = 2, NT = 256;
    static constexpr int BM = WM * TM * 32, BN = WN * TN * 32;
    static constexpr int RT = BM / 32, CT = BN / 32;
    static constexpr bool A8 = A8_;
    static constexpr int AP = A8 ? 2 : 1;  // activation record planes per row tile
    static_assert(A8 ? (BKB == 1 || BKB == 2) : BKB == 2,
                  "W4A4: two blocks per operand set; A8: the two planes of one block per operand set");
    static constexpr int STAGE_BYTES = (RT * AP + CT) * BKB * MX_REC;
    static constexpr int DMA_PER_STAGE = (RT * AP + CT) * BKB;  // 1 KB each
    static constexpr int DMA_PER_WAVE = DMA_PER_STAGE / 4;
    static_assert(DMA_PER_STAGE % 4 == 0, "loads split evenly over the 4 waves");
    static_assert(MX_BLOCK_PAD % BKB == 0, "stages tile the padded block range");
};

// LDS reads of one fragment.  They are volatile so that the compiler never
// merges reads of two different fragments into one instruction (that would
// scatter a fragment over non-adjacent registers and cost moves and early
// waits); immediate offsets still fold.
template <class T>
__device__ __forceinline__ T lds_read(const uint8_t *p) {
    return *reinterpret_cast<const volatile __attribute__((address_space(3))) T *>(
        (const __attribute__((address_space(3))) uint8_t *)p);
}

// One global-to-LDS load of 16 bytes per lane: lane l's bytes at sbase +
// voff land at LDS byte address lds + 16 l (lds is wave-uniform, passed
// through M0).  The base is wave-uniform (SGPRs) and voff a per-lane 32-bit
// byte offset, so no 64-bit vector address arithmetic is needed per load.
__device__ __forceinline__ void dma16s(const uint8_t *sbase, uint32_t voff, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase), "s"(lds) : "memory");
}

// A wave-uniform pointer, placed in SGPRs.  (The builtin returns a signed
// int: each half is widened through uint32_t, never sign-extended.)
__device__ __forceinline__ const uint8_t *uniform_ptr(const uint8_t *p) {
    const uint64_t v = (uint64_t)(uintptr_t)p;
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return (const uint8_t *)(uintptr_t)((uint64_t)hi << 32 | (uint64_t)lo);
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

    // split K: workgroups id * splits + z take K part z of one tile
    const int64_t z = a.splits > 1 ? id % a.splits : 0;
    if (a.splits > 1) id /= a.splits;
    int64_t bx, by;
    mx_tile_of(id, (a.n + C::BN - 1) / C::BN, (a.m + C::BM - 1) / C::BM, bx, by);
    const int64_t rt0 = by * RT, ct0 = bx * C::CT;

    // ---- this wave's loads: DMA_PER_WAVE records of 1 KB per stage ----
    // load i = wave * DMA_PER_WAVE + d covers tile i / BKB (row tiles first,
    // each with its AP planes, then column tiles), block i % BKB of the stage.
    // Tiles past the matrix edge are clamped to the last one (their outputs
    // are never stored).
    constexpr int AP = C::AP;
    const uint8_t *src[C::DMA_PER_WAVE];
    uint32_t dst[C::DMA_PER_WAVE];
    const uint32_t smem_base = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)smem;
#pragma unroll
    for (int d = 0; d < C::DMA_PER_WAVE; d++) {
        const int i = wave * C::DMA_PER_WAVE + d, t = i / BKB, bb = i % BKB;
        const uint8_t *base = t < RT * AP ? a.act + (min(rt0 + t / AP, rtiles - 1) * AP + t % AP) * nbp * MX_REC
                                          : a.wrec + min(ct0 + t - RT * AP, ctiles - 1) * nbp * MX_REC;
        src[d] = uniform_ptr(base + bb * MX_REC);
        dst[d] = (uint32_t)((t * BKB + bb) * MX_REC);
    }
    const uint32_t voff = lane * 16;
    // this workgroup's stages: whole pairs of stages, part z of splits
    const int64_t pairs = nbp / BKB / 2;
    const int s_lo = (int)(z * pairs / a.splits) * 2;
    const int nstages = (int)((z + 1) * pairs / a.splits) * 2 - s_lo;
    // Load d of stage `stage` into ring slot `slot`.  Past the last stage
    // the ring keeps reloading the last one (its slot is never computed): the
    // count of loads in flight stays fixed.
    auto issue_one = [&](int stage, int slot, int d) {
        const int64_t kb0 = (int64_t)(s_lo + min(stage, nstages - 1)) * BKB;
        const uint32_t lds = __builtin_amdgcn_readfirstlane(smem_base + slot * C::STAGE_BYTES);
        dma16s(src[d] + kb0 * MX_REC, voff, lds + dst[d]);
    };
    auto issue = [&](int stage, int slot) {
#pragma unroll
        for (int d = 0; d < C::DMA_PER_WAVE; d++) issue_one(stage, slot, d);
    };

    v16f acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; i++)
#pragma unroll
        for (int j = 0; j < TN; j++)
#pragma unroll
            for (int v = 0; v < 16; v++) acc[i][j][v] = 0.0f;

    // ---- one software pipeline over all blocks ----
    // A stage is two blocks; one operand register set per row / column tile
    // carries both (lanes 0..31 block 0, lanes 32..63 block 1).  Step t of a
    // stage is tile (t / TN, t % TN): its 32 multiply-adds consume the three
    // MFMAs (the scale products of both blocks and the two block dots) issued
    // during the step before, while the three MFMAs of tile t + 1 are issued
    // among them, so every MFMA has a whole step to finish.  The tiles' operand
    // registers are single: right after the MFMAs of a step have taken an
    // operand for the last time in this stage, the operand of the next stage
    // is read into its registers (at the latest one step before its first
    // use).  At step BAR of stage s the wait + barrier publish stage s + 1 and
    // the slot of stage s - 1 (read during stage s - 1) is refilled.  The
    // pipeline never drains at a stage boundary.
    static_assert(NS >= 3, "one stage in flight besides the two in use");
    constexpr int STEPS = TM * TN;
    static_assert(STEPS % 2 == 0, "the result buffers alternate by step parity");
    constexpr int PARTS = TM + TN;  // parts 0 .. TM - 1: row tiles, then the column tiles
    constexpr int BAR = 0;          // step of the barrier
    constexpr int SPAN = STEPS - BAR;  // steps that carry a stage's loads
    v8i af[TM], bf[TN];
    uint2 ap[TM];     // (s1, s1, s2, s2) of row c of block g
    uint32_t bw[TN];  // (d0, d1) of column c of block g
    const int sel0 = g ? 0 : 127, sel1 = g ? 127 : 0;  // E8M0 lane masks of blocks 0 and 1
    const uint32_t id_sel = opaque_identity_selector();
    // Operand reads of one row tile (i) or column tile (j) of a stage; lane
    // group g reads block g's record.
    auto load_a = [&](const uint8_t *st, int i) {
        const uint8_t *rec = st + ((wm * TM + i) * AP * BKB + g) * MX_REC, *p = rec + 8 * c;
        af[i] = fp6_operand(lds_read<u32x2>(p), lds_read<u32x2>(p + 256), lds_read<u32x2>(p + 512));
        const u32x2 sp = lds_read<u32x2>(rec + MX_CODE_BYTES + 8 * c);
        ap[i] = make_uint2(sp.x, sp.y);
    };
    auto load_b = [&](const uint8_t *st, int j) {
        const uint8_t *rec = st + ((RT * AP + wn * TN + j) * BKB + g) * MX_REC, *p = rec + 8 * c;
        bf[j] = fp6_operand(lds_read<u32x2>(p), lds_read<u32x2>(p + 256), lds_read<u32x2>(p + 512));
        bw[j] = lds_read<uint32_t>(rec + MX_CODE_BYTES + 4 * c);
    };
    auto load_part = [&](const uint8_t *st, int p) {
        if (p < TM) load_a(st, p);
        else load_b(st, p - TM);
    };
    // The step during which a stage issues its last MFMA on part p (the MFMAs
    // of tile t are issued at step t - 1; tile 0's at the previous stage's
    // last step, here -1): the part is reread for the next stage right after.
    auto last_issue = [](int p) {
        int last = -1;
        for (int t = 0; t < STEPS; t++)
            if ((p < TM && t / TN == p) || (p >= TM && t % TN == p - TM)) last = t - 1;
        return last < 0 ? 0 : last;
    };
    auto mfma_p = [&](int i, int j) { return mfma_bf16_32x32x4_2blk(ap[i], dup_at_use(bw[j], id_sel)); };

#pragma unroll
    for (int x = 0; x < NS - 1; x++) issue(x, x);
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(C::DMA_PER_WAVE * (NS - 2)) : "memory");
    __syncthreads();
    if constexpr (C::A8) {
        // A8: per block and tile one FP6 MFMA (both planes) and one
        // single-block scale product.  Step t of a stage is block t / TT,
        // tile t % TT; every (tile, block) part of a stage has its own
        // operand registers, reread for the next stage right after the step
        // that issues its last MFMAs, as in the W4A4 pipeline.
        constexpr int TT = TM * TN, ST8 = TT * BKB, PARTS8 = (TM + TN) * BKB;
        static_assert(ST8 % 2 == 0, "the result buffers alternate by step parity");
        v8i af8[TM][BKB], bf8[TN][BKB];
        uint2 ap8[TM][BKB];     // (s1, s1, s2, s2) of row c (the h plane; zeros in the l plane)
        uint32_t bw8[TN][BKB];  // (d0, d1) of column c
        auto load_a8 = [&](const uint8_t *st, int i, int bb) {
            const uint8_t *rec = st + (((wm * TM + i) * AP + g) * BKB + bb) * MX_REC, *p = rec + 8 * c;
            af8[i][bb] = fp6_operand(lds_read<u32x2>(p), lds_read<u32x2>(p + 256), lds_read<u32x2>(p + 512));
            const u32x2 sp = lds_read<u32x2>(rec + MX_CODE_BYTES + 8 * c);
            ap8[i][bb] = make_uint2(sp.x, sp.y);
        };
        auto load_b8 = [&](const uint8_t *st, int j, int bb) {
            const uint8_t *rec = st + ((RT * AP + wn * TN + j) * BKB + bb) * MX_REC, *p = rec + 8 * c;
            bf8[j][bb] = fp6_operand(lds_read<u32x2>(p), lds_read<u32x2>(p + 256), lds_read<u32x2>(p + 512));
            bw8[j][bb] = lds_read<uint32_t>(rec + MX_CODE_BYTES + 4 * c);
        };
        // part p: block p / (TM + TN); row tiles first, then column tiles
        auto load_part8 = [&](const uint8_t *st, int p) {
            const int bb = p / (TM + TN), q = p % (TM + TN);
            if (q < TM) load_a8(st, q, bb);
            else load_b8(st, q - TM, bb);
        };
        auto last_issue8 = [](int p) {
            const int bb = p / (TM + TN), q = p % (TM + TN);
            int last = -1;
            for (int t = 0; t < ST8; t++) {
                const int tt = t % TT;
                if (t / TT == bb && ((q < TM && tt / TN == q) || (q >= TM && tt % TN == q - TM))) last = t - 1;
            }
            return last < 0 ? 0 : last;
        };
        auto mfma_p8 = [&](int t) {
            const int bb = t / TT, tt = t % TT;
            return mfma_bf16_32x32x8(ap8[tt / TN][bb], dup_at_use(bw8[tt % TN][bb], id_sel));
        };
        auto mfma_s8 = [&](int t) {
            const int bb = t / TT, tt = t % TT;
            return mfma_block8(af8[tt / TN][bb], bf8[tt % TN][bb], g);
        };
        v16f S[2], P[2];
#pragma unroll
        for (int p = 0; p < PARTS8; p++) load_part8(smem, p);
        P[0] = mfma_p8(0);
        S[0] = mfma_s8(0);

        for (int s = 0; s < nstages; s++) {
#pragma unroll
            for (int t = 0; t < ST8; t++) {
                const int tt = t % TT, i = tt / TN, j = tt % TN, b = t & 1, b1 = b ^ 1;
                if (t == 0) {  // stage s + 1 has landed and stage s - 1's slot is free
                    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(C::DMA_PER_WAVE * (NS - 3)) : "memory");
                    __syncthreads();
                }
#pragma unroll
                for (int d = t * C::DMA_PER_WAVE / ST8; d < (t + 1) * C::DMA_PER_WAVE / ST8; d++)
                    issue_one(s + NS - 1, (s + NS - 1) % NS, d);
                const int t1 = (t + 1) % ST8;
                P[b1] = mfma_p8(t1);
#pragma unroll
                for (int v = 0; v < 8; v++) acc[i][j][v] = fmaf(S[b][v], P[b][v], acc[i][j][v]);
                __builtin_amdgcn_sched_barrier(0x0004 | 0x0010);
                S[b1] = mfma_s8(t1);
#pragma unroll
                for (int p = 0; p < PARTS8; p++)
                    if (last_issue8(p) == t) load_part8(smem + ((s + 1) % NS) * C::STAGE_BYTES, p);
#pragma unroll
                for (int v = 8; v < 16; v++) acc[i][j][v] = fmaf(S[b][v], P[b][v], acc[i][j][v]);
                asm volatile("" : "+v"(acc[i][j]));
                __builtin_amdgcn_sched_barrier(0x0004 | 0x0010);
            }
        }
    } else {
        v16f S0[2], S1[2];
        v32f P[2];
#pragma unroll
        for (int p = 0; p < PARTS; p++) load_part(smem, p);
        P[0] = mfma_p(0, 0);
        S0[0] = mfma_block(af[0], bf[0], sel0);
        S1[0] = mfma_block(af[0], bf[0], sel1);

        for (int s = 0; s < nstages; s++) {
#pragma unroll
            for (int t = 0; t < STEPS; t++) {
                const int i = t / TN, j = t % TN, b = t & 1, b1 = b ^ 1;
                if (t == BAR) {
                    // stage s + 1 has landed for this wave; after the barrier for
                    // every wave, and stage s - 1's slot is free.  (After the last
                    // stage the reads below see a reloaded stage; the MFMAs they
                    // feed are never consumed.)
                    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(C::DMA_PER_WAVE * (NS - 3)) : "memory");
                    __syncthreads();
                }
                if (t >= BAR) {  // refill stage s - 1's slot, spread over the steps
                    const int q = t - BAR;
#pragma unroll
                    for (int d = q * C::DMA_PER_WAVE / SPAN; d < (q + 1) * C::DMA_PER_WAVE / SPAN; d++)
                        issue_one(s + NS - 1, (s + NS - 1) % NS, d);
                }
                // the MFMAs of tile t + 1 (of stage s + 1 after the last step) ...
                const int t1 = (t + 1) % STEPS, i1 = t1 / TN, j1 = t1 % TN;
                P[b1] = mfma_p(i1, j1);
#pragma unroll
                for (int v = 0; v < 11; v++) acc[i][j][v] = fmaf(S0[b][v], P[b][v], acc[i][j][v]);
                __builtin_amdgcn_sched_barrier(0x0004 | 0x0010);  // scalar and global-to-LDS ops may move
                S0[b1] = mfma_block(af[i1], bf[j1], sel0);
#pragma unroll
                for (int v = 11; v < 16; v++) acc[i][j][v] = fmaf(S0[b][v], P[b][v], acc[i][j][v]);
#pragma unroll
                for (int v = 0; v < 6; v++) acc[i][j][v] = fmaf(S1[b][v], P[b][16 + v], acc[i][j][v]);
                __builtin_amdgcn_sched_barrier(0x0004 | 0x0010);
                S1[b1] = mfma_block(af[i1], bf[j1], sel1);
                // ... then the operands they were the last to take, for stage s + 1
#pragma unroll
                for (int p = 0; p < PARTS; p++)
                    if (last_issue(p) == t) load_part(smem + ((s + 1) % NS) * C::STAGE_BYTES, p);
                // ... while the multiply-adds of tile t finish
#pragma unroll
                for (int v = 6; v < 16; v++) acc[i][j][v] = fmaf(S1[b][v], P[b][16 + v], acc[i][j][v]);
                asm volatile("" : "+v"(acc[i][j]));  // materialised here, not sunk past the loop's end
                __builtin_amdgcn_sched_barrier(0x0004 | 0x0010);
            }
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
                if (r >= a.m) continue;
                if (a.splits > 1) a.partial[(z * a.m + r) * a.n + col] = acc[i][j][v];
                else a.y[r * a.ldy + col] = acc[i][j][v];
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
template <int BM_, int BN_, bool A8_ = false>
struct MxPieceCfg {
    static constexpr int BM = BM_, BN = BN_;                 // tile shape of the main kernel
    static constexpr int PIECES = (BM / 32) * (BN / 32);     // 32x32 pieces per leftover tile
    static constexpr bool A8 = A8_;
    static constexpr int AP = A8 ? 2 : 1;                    // activation planes (see MxCfg)
    static constexpr int BKB = A8 ? 1 : 2, NS = 4, NT = 256; // per wave: NS stages of BKB blocks
    static constexpr int WAVE_RING = NS * BKB * (AP + 1) * MX_REC;  // per stage: A records (each plane), then B's
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
    constexpr int AP = C::AP;
    const uint8_t *arec = uniform_ptr(a.act + min(rt, rtiles - 1) * AP * nbp * MX_REC);  // (A8: the l plane follows)
    const uint8_t *brec = uniform_ptr(a.wrec + min(ct, ctiles - 1) * nbp * MX_REC);

    // this wave's quarter of the blocks, in whole stages
    const int64_t nstages_all = nbp / BKB;
    const int64_t s_begin = nstages_all * wave / 4, s_end = nstages_all * (wave + 1) / 4;
    const int nst = (int)(s_end - s_begin);
    uint8_t *ring = smem + wave * C::WAVE_RING;
    const uint32_t ring_lds =
        __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)ring);
    const uint32_t voff = lane * 16;
    auto issue = [&](int stage, int slot) {
        // past the last stage the ring reloads the last one (never computed)
        const int64_t kb0 = (s_begin + min(stage, max(nst - 1, 0))) * BKB;
        const uint32_t lds = ring_lds + slot * BKB * (AP + 1) * MX_REC;
#pragma unroll
        for (int bb = 0; bb < BKB; bb++) {
#pragma unroll
            for (int pl = 0; pl < AP; pl++)
                dma16s(arec + (pl * nbp + kb0 + bb) * MX_REC, voff, lds + (pl * BKB + bb) * MX_REC);
            dma16s(brec + (kb0 + bb) * MX_REC, voff, lds + (AP * BKB + bb) * MX_REC);
        }
    };
    const int sel0 = g ? 0 : 127, sel1 = g ? 127 : 0;  // E8M0 lane masks of blocks 0 and 1
    const uint32_t id_sel = opaque_identity_selector();

    v16f acc;
#pragma unroll
    for (int v = 0; v < 16; v++) acc[v] = 0.0f;
    // One operand set per stage (both blocks; lane group g reads block g's
    // records).  The three MFMAs of stage s + 1 are issued around the 32
    // multiply-adds of stage s, each once the multiply-adds have read the
    // result it replaces (one tile per wave leaves nothing else to cover
    // their latency).
    v8i af, bf;
    uint2 ap;
    uint32_t bw;
    auto load = [&](const uint8_t *st) {  // (A8: lane group g reads plane g, both the weights)
        const uint8_t *pa = st + g * MX_REC, *pb = st + (AP * BKB + (C::A8 ? 0 : g)) * MX_REC;
        af = fp6_operand(lds_read<u32x2>(pa + 8 * c), lds_read<u32x2>(pa + 256 + 8 * c),
                         lds_read<u32x2>(pa + 512 + 8 * c));
        bf = fp6_operand(lds_read<u32x2>(pb + 8 * c), lds_read<u32x2>(pb + 256 + 8 * c),
                         lds_read<u32x2>(pb + 512 + 8 * c));
        const u32x2 sp = lds_read<u32x2>(pa + MX_CODE_BYTES + 8 * c);
        ap = make_uint2(sp.x, sp.y);
        bw = lds_read<uint32_t>(pb + MX_CODE_BYTES + 4 * c);
    };
    if constexpr (C::A8) {
        if (nst > 0) {
            // A8: one block per stage, one FP6 MFMA and one single-block scale
            // product per stage
            constexpr int LOADS = (AP + 1) * BKB;  // per stage
#pragma unroll
            for (int x = 0; x < NS - 1; x++) issue(x, x);
            asm volatile("s_waitcnt vmcnt(%0)" ::"n"(LOADS * (NS - 2)) : "memory");  // stage 0 has landed
            load(ring);
            v16f P = mfma_bf16_32x32x8(ap, dup_at_use(bw, id_sel)), S = mfma_block8(af, bf, g);
            for (int s = 0; s < nst; s++) {
                issue(s + NS - 1, (s + NS - 1) % NS);
                asm volatile("s_waitcnt vmcnt(%0)" ::"n"(LOADS * (NS - 2)) : "memory");
                load(ring + ((s + 1) % NS) * BKB * (AP + 1) * MX_REC);
#pragma unroll
                for (int v = 0; v < 16; v++) acc[v] = fmaf(S[v], P[v], acc[v]);
                asm volatile("" : "+v"(acc));
                __builtin_amdgcn_sched_barrier(0x0004 | 0x0010 | 0x0080);
                P = mfma_bf16_32x32x8(ap, dup_at_use(bw, id_sel));
                S = mfma_block8(af, bf, g);
                __builtin_amdgcn_sched_barrier(0x0004 | 0x0010 | 0x0080);
            }
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // no load may still be writing the ring
        }
    } else if (nst > 0) {
#pragma unroll
        for (int x = 0; x < NS - 1; x++) issue(x, x);
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * BKB * (NS - 2)) : "memory");  // stage 0 has landed
        v16f S0, S1;
        v32f P;
        load(ring);
        P = mfma_bf16_32x32x4_2blk(ap, dup_at_use(bw, id_sel));
        S0 = mfma_block(af, bf, sel0);
        S1 = mfma_block(af, bf, sel1);
        for (int s = 0; s < nst; s++) {
            // refill the slot computed last, wait for stage s + 1 and read its
            // operands (after the last stage this reads a reloaded stage;
            // unused)
            issue(s + NS - 1, (s + NS - 1) % NS);
            asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * BKB * (NS - 2)) : "memory");
            load(ring + ((s + 1) % NS) * BKB * (AP + 1) * MX_REC);
#pragma unroll
            for (int v = 0; v < 16; v++) acc[v] = fmaf(S0[v], P[v], acc[v]);
            __builtin_amdgcn_sched_barrier(0x0004 | 0x0010 | 0x0080);
            S0 = mfma_block(af, bf, sel0);
#pragma unroll
            for (int v = 0; v < 16; v++) acc[v] = fmaf(S1[v], P[16 + v], acc[v]);
            asm volatile("" : "+v"(acc));
            __builtin_amdgcn_sched_barrier(0x0004 | 0x0010 | 0x0080);
            P = mfma_bf16_32x32x4_2blk(ap, dup_at_use(bw, id_sel));
            S1 = mfma_block(af, bf, sel1);
            __builtin_amdgcn_sched_barrier(0x0004 | 0x0010 | 0x0080);
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
    using P = MxPieceCfg<C::BM, C::BN, C::A8>;
    static_assert(P::NT == C::NT, "one workgroup size for both kinds");
    constexpr int MAIN_LDS = C::NS * C::STAGE_BYTES, PIECE_LDS = 4 * P::WAVE_RING;
    __shared__ __attribute__((aligned(1024))) uint8_t smem[MAIN_LDS > PIECE_LDS ? MAIN_LDS : PIECE_LDS];
    if ((int64_t)blockIdx.x < main_wgs) mx_tile<C>(a, blockIdx.x, smem);  // uniform per workgroup
    else mx_piece<P>(a, first_piece_tile, blockIdx.x - main_wgs, smem);
}

}  // namespace w4a4
