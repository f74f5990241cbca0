// MUL_MAT_ID product that streams the experts' 4-bit weight records.
//
// 1bit-MONSTER engine docs, "The lean option: ROCmFP4, ROCmI4 and Hadamard
// Q4_0", section "MoE: W4A4 on the experts": the expert matmuls take the same
// W4A4 path as the dense ones -- int4 x int4 block dots, per-block scaling.
//
// The experts of a micro-batch get few rows each (tens, a few hundred for the
// popular ones), so the product streams the weights, as for m <= 16.  Work
// item = (expert tile of GS_ROWS routed rows, chunk of GS_WAVES column
// tiles): the workgroup stages its rows' activations in LDS straight from the
// activation rows (the routing's row permutation picks them; no gathered
// copy is written), already in the int8 MFMA's lane order and with each
// scale split into its scale-product operand; then each wave streams one
// 32-column tile's 2304-byte records (0.5625 B per weight) through a 2-deep
// register ring.  Per block and wave: one 32x32x32 int8 MFMA (all 32 rows x
// the tile's 32 columns); per two blocks one 32x32x4 bf16 MFMA forms both
// blocks' scale products s (x) d (the split operands the dense kernel uses);
// per output a convert and one fused multiply-add remain.  Codes enter as
// 16 x nibble, so d is scaled by 2^-8.  Long K is staged in chunks of
// GS_KCHUNK blocks, each chunk's loads issued while the previous chunk
// streams.  Each workgroup scatters its rows to y.  Each XCD takes a
// contiguous share of the expert-ordered items, so an expert's row tiles
// share one L2 and read its weights from HBM about once.
#pragma once

#include "common.h"
#include "k_route.h"

namespace w4a4 {

constexpr int GS_ROWS = 32;     // routed rows per item (one 32x32 MFMA tile)
constexpr int GS_WAVES = 8;     // waves per workgroup, one column tile each
constexpr int GS_KCHUNK = 32;   // blocks of activations staged per pass (a multiple of 4)
// per staged block: 32 rows x 32 int8 codes (1 KB), 32 scale operands (256 B)
constexpr int GS_STAGE_BYTES = GS_KCHUNK * (GS_ROWS * QK + GS_ROWS * 8);

// Column tiles per wave and item: two when K fits one staging pass (the
// staged activations then serve twice as many columns), else one.
__host__ inline int grouped_tiles_per_wave(int64_t n, int64_t k) {
    return k / QK <= GS_KCHUNK && padded_n(n) / TILE_N > GS_WAVES ? 2 : 1;
}
__host__ inline int64_t grouped_col_chunks(int64_t n, int64_t k) {
    const int64_t per = (int64_t)GS_WAVES * grouped_tiles_per_wave(n, k);
    return (padded_n(n) / TILE_N + per - 1) / per;
}

struct GsArgs {
    const uint8_t *codes;    // activation codes [rows][k/2]
    const float *scales;     // activation scales [rows][k/32]
    const uint8_t *packed;   // packed weights of expert 0; expert e at + e * expert_bytes
    int64_t expert_bytes;
    float *y;                // [n_tokens * top_k][n]
    int64_t ldy, n, k;
    Routing g;
    int top_k, per_slot;     // activation row of routed row i: i (per slot) or i / top_k
    int64_t n_rows;          // routed rows (tokens x slots); those past offsets[E] have invalid ids
    int64_t col_chunks;      // ceil(tiles / (GS_WAVES * tiles_per_wave))
    int tiles_per_wave = 1;  // > 1 only when K fits one staging pass
};

__global__ __launch_bounds__(64 * GS_WAVES, 4) void gemm_grouped_stream_kernel(GsArgs a) {  // 4 waves per SIMD: two workgroups per CU
    constexpr int ROW_BYTES = QK / 2;  // activation code bytes per (row, block)
    __shared__ __attribute__((aligned(16))) uint8_t smem[GS_STAGE_BYTES];
    __shared__ int64_t src_row[GS_ROWS];
    __shared__ int32_t out_row[GS_ROWS];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int64_t k = a.k, nb = k / QK, nq = sq_quads(k);
    const int64_t tiles = padded_n(a.n) / TILE_N;

    // workgroup 0 first zeroes the output rows of invalid ids (the routing put
    // them after the valid rows), whatever item it takes after
    if (blockIdx.x == 0) {
        const int64_t first = a.g.offsets[a.g.n_expert], bad = a.n_rows - first;
        for (int64_t i = tid; i < bad * a.n; i += 64 * GS_WAVES)
            a.y[(int64_t)a.g.perm[first + i / a.n] * a.ldy + i % a.n] = 0.0f;
    }

    // item: contiguous share per XCD (ids x, x + 8, ... run on XCD x).  The
    // items of one expert (row tiles x column chunks) are consecutive and
    // column-chunk-major, so a chunk's weights are read from HBM once and
    // then from the XCD's L2 by the expert's other row tiles.
    const int64_t rtiles = a.g.tile_prefix[a.g.n_expert];
    const int64_t items = rtiles * a.col_chunks, per_xcd = (items + 7) / 8;
    const int64_t j = blockIdx.x / 8, item = (blockIdx.x % 8) * per_xcd + j;
    if (j >= per_xcd || item >= items) return;  // uniform
    const int e = expert_of_tile(a.g, item / a.col_chunks);
    const int64_t t0 = a.g.tile_prefix[e], ne = a.g.tile_prefix[e + 1] - t0;
    const int64_t local = item - t0 * a.col_chunks, cc = local / ne, rt_e = local % ne;
    const int64_t cnt = a.g.offsets[e + 1] - a.g.offsets[e];
    const int64_t row_lo = rt_e * GS_ROWS;
    if (tid < GS_ROWS) {
        const int64_t lr = row_lo + tid;  // row within the expert
        int64_t src = -1;
        int32_t orow = -1;
        if (lr < cnt) {
            orow = a.g.perm[a.g.offsets[e] + lr];
            src = a.per_slot ? orow : orow / a.top_k;
        }
        src_row[tid] = src;
        out_row[tid] = orow;
    }

    const int lo16 = lane * 16, d4 = SQ_SCALE_OFF + lane * 4;
    const int g = lane >> 5, r32 = lane & 31;  // K half and row / column of this lane
    v16f acc;
    uint4 *codes16 = reinterpret_cast<uint4 *>(smem);                                  // [block][g][row]
    uint2 *sop = reinterpret_cast<uint2 *>(smem + GS_KCHUNK * GS_ROWS * QK);            // [block][row]

    // Activations of a chunk: thread t stages entries (row, block) t and
    // t + 64 GS_WAVES of the chunk's GS_KCHUNK x GS_ROWS; their loads are
    // issued one chunk ahead, into registers, so that they overlap the
    // previous chunk's stream.  Rows past the expert's count and blocks past
    // nb are zero.
    constexpr int NT = 64 * GS_WAVES, PER = GS_KCHUNK * GS_ROWS / NT;
    struct Stage {
        uint4 u[PER];
        float s[PER];
    } st;
    auto stage_load = [&](int64_t c0) {
#pragma unroll
        for (int p = 0; p < PER; p++) {
            const int i = tid + p * NT, bl = i / GS_ROWS, r = i % GS_ROWS;
            const int64_t b = c0 + bl, src = src_row[r];
            st.u[p] = make_uint4(0, 0, 0, 0);
            st.s[p] = 0.0f;
            if (src >= 0 && b < nb) {
                const uint4 *q = reinterpret_cast<const uint4 *>(a.codes + src * (k / 32 * ROW_BYTES) + b * ROW_BYTES);
                st.u[p] = q[0];
                st.s[p] = a.scales[src * nb + b];
            }
        }
    };
    // ... and written to LDS as the MFMA's two K halves of 16 int8 codes and
    // the scale operand
    auto stage_store = [&]() {
#pragma unroll
        for (int p = 0; p < PER; p++) {
            const int i = tid + p * NT, bl = i / GS_ROWS, r = i % GS_ROWS;
            const uint4 w = k8_words(st.u[p]);
            const v4i h0 = widen_k8x2(w.x, w.y), h1 = widen_k8x2(w.z, w.w);
            codes16[(bl * 2 + 0) * GS_ROWS + r] = make_uint4(h0[0], h0[1], h0[2], h0[3]);
            codes16[(bl * 2 + 1) * GS_ROWS + r] = make_uint4(h1[0], h1[1], h1[2], h1[3]);
            sop[bl * GS_ROWS + r] = act_scale_operand(st.s[p]);
        }
    };

    // This wave's records, in order, through a 2-deep ring that runs across
    // the chunks (the weights do not wait for the staging).
    struct Rec {
        v4u c0, c1;
        uint32_t d;
    };
    __amdgpu_buffer_rsrc_t wbuf;
    auto load = [&](int64_t i, Rec &R) {  // slots past the tile reload its last record (a cache hit)
        const int off = __builtin_amdgcn_readfirstlane((int)min(i, nq - 1) * SQ_REC);
        R.c0 = __builtin_amdgcn_raw_buffer_load_b128(wbuf, lo16, off, 0);
        __builtin_amdgcn_sched_barrier(0);
        R.c1 = __builtin_amdgcn_raw_buffer_load_b128(wbuf, lo16 + 1024, off, 0);
        __builtin_amdgcn_sched_barrier(0);
        R.d = __builtin_amdgcn_raw_buffer_load_b32(wbuf, d4, off, 0);
        __builtin_amdgcn_sched_barrier(0);
    };
    constexpr float UNSCALE = 1.0f / 256.0f;  // the operands' 16 x factors
    // blocks bl and bl + 1 of the chunk: (w0, w1) this lane's words of each,
    // dh its d of block bl + g
    auto pair = [&](int bl, uint32_t w00, uint32_t w01, uint32_t w10, uint32_t w11, uint16_t dh) {
        const uint32_t wop = weight_scale_operand(__half2float(__ushort_as_half(dh)) * UNSCALE);
        const v32f P = mfma_bf16_32x32x4_2blk(sop[(bl + g) * GS_ROWS + r32], make_uint2(wop, wop));
        const uint4 a0 = codes16[(bl * 2 + g) * GS_ROWS + r32];
        const v16i S0 = mfma_i8_32x32x32(v4i{(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w}, widen_k8x2(w00, w01));
        const uint4 a1 = codes16[((bl + 1) * 2 + g) * GS_ROWS + r32];
        const v16i S1 = mfma_i8_32x32x32(v4i{(int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w}, widen_k8x2(w10, w11));
#pragma unroll
        for (int v = 0; v < 16; v++) acc[v] = fmaf((float)S0[v], P[v], acc[v]);
#pragma unroll
        for (int v = 0; v < 16; v++) acc[v] = fmaf((float)S1[v], P[16 + v], acc[v]);
    };
    auto compute = [&](int rec, const Rec &R) {  // rec: record index within the chunk
        const int bl = rec * SQ_BLOCKS;
        pair(bl + 0, R.c0[0], R.c0[1], R.c0[2], R.c0[3], (uint16_t)(R.d & 0xFFFF));
        pair(bl + 2, R.c1[0], R.c1[1], R.c1[2], R.c1[3], (uint16_t)(R.d >> 16));
    };

    constexpr int RPC = GS_KCHUNK / SQ_BLOCKS;  // records per chunk (even)
    // The wave's tt-th column tile: of the item's tiles_per_wave rounds of
    // GS_WAVES (a last chunk's extra waves stream the last tile again and
    // store nothing).
    auto tile_of = [&](int tt) { return (cc * a.tiles_per_wave + tt) * GS_WAVES + wave; };
    auto set_tile = [&](int64_t tile) {
        const uint8_t *sq = a.packed + e * a.expert_bytes + sq_section_offset(a.n, k) + min(tile, tiles - 1) * nq * SQ_REC;
        wbuf = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(sq), 0, (int)(nq * SQ_REC), 0x00020000);
        acc = v16f{};
    };
    // records r0 .. r0 + cnt_r - 1 of the tile, record r0 already in q0; an
    // even count leaves record r0 + cnt_r in q0
    auto stream = [&](int64_t r0, int cnt_r, Rec &q0, Rec &q1) {
        for (int i = 0; i < cnt_r; i += 2) {
            load(r0 + i + 1, q1);
            __builtin_amdgcn_sched_barrier(0);
            compute(i, q0);
            __builtin_amdgcn_sched_barrier(0);
            if (i + 1 >= cnt_r) break;
            load(r0 + i + 2, q0);
            __builtin_amdgcn_sched_barrier(0);
            compute(i + 1, q1);
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    // scatter: output row of local row r is out_row[r]
    auto scatter = [&](int64_t tile) {
        const int64_t col = tile * TILE_N + r32;
        if (tile >= tiles || col >= a.n) return;
#pragma unroll
        for (int v = 0; v < 16; v++) {
            const int32_t orow = out_row[mfma32_row(v, lane)];
            if (orow >= 0) a.y[(int64_t)orow * a.ldy + col] = acc[v];
        }
    };

    Rec q0, q1;
    if (nq <= RPC) {
        // K fits one pass: stage once, then stream each of the wave's tiles
        set_tile(tile_of(0));
        load(0, q0);
        __syncthreads();  // the row table is written
        stage_load(0);
        stage_store();
        __syncthreads();
        for (int tt = 0; tt < a.tiles_per_wave; tt++) {
            if (tt > 0) {
                set_tile(tile_of(tt));
                load(0, q0);
            }
            stream(0, (int)nq, q0, q1);
            scatter(tile_of(tt));
        }
    } else {
        // passes of GS_KCHUNK blocks, the next pass's loads issued during
        // this one's stream; the weight ring runs across the passes
        set_tile(tile_of(0));
        load(0, q0);
        __syncthreads();  // the row table is written
        stage_load(0);
        for (int64_t r0 = 0; r0 < nq; r0 += RPC) {
            __syncthreads();  // the previous chunk's LDS reads are done
            stage_store();
            __syncthreads();
            if (r0 + RPC < nq) stage_load((r0 + RPC) * SQ_BLOCKS);
            stream(r0, (int)min((int64_t)RPC, nq - r0), q0, q1);
        }
        scatter(tile_of(0));
    }
}

}  // namespace w4a4
