// W4A4 GEMM for m <= 16 (a speculative-verify-sized batch): HBM-bound, every
// weight byte is read from HBM once per call.
//
// 1bit-MONSTER engine docs, "The lean option: ROCmFP4, ROCmI4 and Hadamard
// Q4_0", section "Hadamard-rotated Q4_0: W4A4 prompt processing": the same
// int4 x int4 block dots and per-block scaling as the large-m path; only the
// way the weights are streamed differs.
//
// Work split: a workgroup owns one 32-column weight tile and a contiguous
// range of K (split z of the tile's streaming records, 4 blocks each; narrow
// projections split K so that every CU gets workgroups).  Its waves take the
// range's records round-robin and stream them straight into registers
// through a ring SM_DEPTH records deep, each record together with its 16
// rows' activation codes and scales (one 16-byte and one 4-byte load per
// lane).  A record's activations are needed by its wave alone: the wave
// moves them through its own LDS slot into the MFMA's lane order just before
// computing the record, so no workgroup-wide staging phase or barrier
// precedes the stream.  Per block and wave: one 32x32x32 int8 MFMA (the 16
// rows, and 16 rows of don't-care lanes whose outputs are dropped, x the
// tile's 32 columns) and one single-block 32x32x8 bf16 MFMA for the scale
// products s (x) d (the split operands the dense kernel uses); per output a
// convert and one fused multiply-add remain.  Codes enter the MFMA
// as 16 x (signed nibble), so the integer sum is 256 S, and d is scaled by
// 2^-8 (exact) to match.  The waves' sums meet in LDS; the workgroup stores
// its 16 x 32 outputs, or its partial sums when K is split: then the last
// workgroup of the tile to finish (by a per-tile arrival count) adds the
// splits in ascending order, so no second launch is needed and the sum does
// not depend on which split finished last.
//
// Measured on MI355X (7 dense projections of a 27B-class layer, 16 rows):
// 8 waves per workgroup and a 2-record ring beat 4 waves or deeper rings;
// K from 5120 to 8192 runs 16 waves per workgroup over the whole of K (the o
// projection, K = 6144: 9.1 us against 9.8 us with 8 waves in 4 K splits,
// weights cold).
#pragma once

#include "common.h"
#include "k_rotq.h"

namespace w4a4 {

constexpr int SMALL_M_MAX = SMA_ROWS;
constexpr int SM_WAVES = 8;             // waves per workgroup (SM_WAVES_LONG_K for K in (5120, 8192])
constexpr int SM_WAVES_LONG_K = 16;
constexpr int SM_DEPTH = 2;             // streaming records in flight per wave
constexpr int SM_ITEM_TARGET = 512;     // workgroups wanted (two per CU on a 256-CU part)
static_assert(SM_ITEM_TARGET < (1 << 16), "a tile's K splits are counted in 16 bits");

struct SmallArgs {
    const uint8_t *codes;   // activation codes [m][k/2] (int8 activations: [m][k])
    const float *scales;    // activation scales [m][k/32]
    const uint8_t *act_rec = nullptr;  // W4A4: the record-ordered operand (common.h) instead of codes, scales
    const uint8_t *sq;      // streaming section of the packed weights
    float *y;               // [m][ldy] (splits == 1) ...
    float *partial;         // ... or [splits][m][n] partial sums
    // K split: per column tile, a count of the workgroups arrived, tagged
    // with this call's ticket (small_m_arrive); the last of the tile's
    // splits resets it to zero.
    unsigned long long *arrivals = nullptr;
    unsigned long long ticket = 0;  // 48 bits, non-zero, drawn per call
    int64_t ldy, m, n, k;
    int64_t range;          // records per split (tiles past `whole`)
    int64_t whole = 0;      // tiles 0 .. whole - 1 run whole K (no partial sums)
    // fused rotate-quantise only (gemm_small_m_fused_kernel): the
    // activations, their row stride and load mode (as the quantiser takes
    // them), where the producers write the codes and scales (= codes,
    // scales above), and the workspace's synchronisation words
    const void *x = nullptr;
    int64_t ldx = 0;
    int mode = 0;
    uint8_t *codes_out = nullptr;
    float *scales_out = nullptr;
    uint32_t *sync = nullptr;   // [0] epoch, [1] workgroups finished, [2] waits that timed out
    uint32_t *flags = nullptr;  // one per quad of blocks: the epoch that published it
    int64_t producers = 0;      // workgroups 0 .. producers - 1 quantise
};

// Launch plan of an m <= 16 product: waves per workgroup and the K splits.
// Narrow projections split K so that about a target number of workgroups
// run.  Pure function of the sizes and the kernel (the workspace size
// depends on it).
// Tiles 0 .. whole - 1 run whole K in one workgroup each; the other tiles
// split K in `splits` ranges of `range` records.
struct SmallPlan {
    int64_t tiles, splits, range;
    int waves;
    int64_t whole;
};
// CUs the plan balances over (MI355X): the leftover tiles of whole rounds of
// this many are split so that every CU gets the same number of records.
constexpr int64_t SM_REF_CUS = 256;
// a8: int8 activations (8 waves per workgroup at every K).
__host__ __device__ inline SmallPlan small_m_plan(int64_t n, int64_t k, bool a8 = false) {
    const int64_t tiles = padded_n(n) / TILE_N, nq = sq_quads(k);
    // Measured on the 16-row verify set with the splits added in-kernel.  K
    // up to 5120 aims at a quarter as many workgroups (q unsplit and k, v in
    // 4 splits beat 2 and 8 splits by 0.3 to 2 us each).  K up to 8192 (at
    // most 64 records per tile) takes 16 waves per workgroup at the same
    // quarter, so the o projection runs whole K: 9.1 us against 9.8 us for 8
    // waves in 4 splits, weights cold.  Longer K keeps 8 waves at the full
    // target (down, K = 17408: 17.9 us in 4 splits against 19.9 us whole K
    // with 16 waves, where each wave streams 8 or 9 records in turn); 16
    // waves for K up to 5120 lose 0.6 to 0.8 us on q, k and v.
    const bool long_k = !a8 && k > 5120 && nq <= 64;
    const int waves = long_k ? SM_WAVES_LONG_K : SM_WAVES;
    const int64_t target = k <= 5120 || long_k ? SM_ITEM_TARGET / 4 : SM_ITEM_TARGET;
    const int64_t want = (target + tiles - 1) / tiles;
    const int64_t splits = want < nq ? want : nq;
    const int64_t range = (nq + splits - 1) / splits;
    if ((nq + range - 1) / range > 1) return SmallPlan{tiles, (nq + range - 1) / range, range, waves, 0};
    // Unsplit: more tiles than CUs leave the L = tiles mod SM_REF_CUS tiles
    // of the last round to a few CUs (a 544-tile projection: 32 CUs hold a
    // third workgroup; 512 tiles run 1.17x faster per byte).  Those L tiles
    // split K in SM_REF_CUS / L parts instead, one piece per CU, and their
    // parts are added in the same launch as other K splits are.
    const int64_t left = tiles % SM_REF_CUS;
    if (tiles > SM_REF_CUS && left > 0 && SM_REF_CUS / left >= 2 && nq >= 2) {
        const int64_t parts = SM_REF_CUS / left < nq ? SM_REF_CUS / left : nq;
        const int64_t r = (nq + parts - 1) / parts;
        return SmallPlan{tiles, (nq + r - 1) / r, r, waves, tiles - left};
    }
    return SmallPlan{tiles, 1, nq, waves, tiles};
}
// Workgroups of a plan: the whole tiles, then the split tiles' ranges.
__host__ __device__ inline int64_t small_m_items(const SmallPlan &p) { return p.whole + (p.tiles - p.whole) * p.splits; }

// Spin limit of a consumer's wait for its activations (each round is one
// device-scope load and a short sleep): the wait always ends, and a wait that
// runs out (which in-order dispatch of the producers rules out) is counted in
// the workspace so that a caller can see it.
constexpr int FUSE_SPIN_LIMIT = 1 << 20;

// Wave 0 of the workgroup waits until the quads q0 .. q0 + nr - 1 of the
// activations carry `target`; the barrier then holds every wave's
// activation loads back until it has.  The producers store the codes and
// scales with device-scope (write-through) stores and complete them before
// their flags, and the consumers load them with device-scope loads, so no
// cache-wide write-back or invalidation is needed on either side.  Every
// wave of the workgroup must call wait_for_quads.
__device__ __forceinline__ void wait_for_quads_wave(const SmallArgs &a, int64_t q0, int nr, uint32_t target,
                                                    int lane) {
    for (int base = 0; base < nr; base += 64) {
        const int i = base + lane;
        int spins = 0;
        while (true) {
            const bool ready =
                i >= nr || __hip_atomic_load(a.flags + q0 + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == target;
            if (__all(ready)) break;
            if (++spins >= FUSE_SPIN_LIMIT) {
                if (lane == 0) atomicAdd(a.sync + 2, 1u);
                break;
            }
            __builtin_amdgcn_s_sleep(20);  // ~0.6 us between polls: hundreds of waves poll the same lines
        }
    }
}

__device__ __forceinline__ void wait_for_quads(const SmallArgs &a, int64_t q0, int nr, uint32_t target) {
    if (threadIdx.x < 64) wait_for_quads_wave(a, q0, nr, target, threadIdx.x & 63);
    __syncthreads();
}

// Bytes of the cross-wave reduction in LDS ([wave][8][64] floats); the
// word after it tells the workgroup whether it arrived last.
__host__ __device__ constexpr int sm_red_bytes(int waves) { return waves * 8 * 64 * 4; }

// Counts one arrival of a K split at its column tile's word and returns 1 to
// the last of `splits` (< 2^16) arrivals, which also resets the word to zero.
// Every arrival adds ticket << 16 | 1, so after c arrivals on a word that
// started at zero it holds (c * ticket mod 2^48) << 16 | c: one fetch-and-add
// per arrival, with no retry however many splits arrive at once, and a value
// that stale contents match only by chance (hi == lo * ticket for a 48-bit
// ticket drawn per call).  An arrival that finds another form (the
// workspace's previous contents) counts itself with compare-and-swaps into a
// word of this call's form; each swap that fails does so because another
// arrival's update succeeded, so the loop ends.
__device__ __forceinline__ int small_m_arrive(unsigned long long *word, unsigned long long ticket, int64_t splits) {
    const unsigned long long inc = ticket << 16 | 1ull, lo = 0xffffull;
    auto ours = [&](unsigned long long w) {  // a count of this call's arrivals
        const unsigned long long c = w & lo;
        return c < (unsigned long long)splits && (w >> 16) == ((c * ticket) & 0xffffffffffffull);
    };
    const unsigned long long old = __hip_atomic_fetch_add(word, inc, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    unsigned long long pos;
    if (ours(old)) {
        pos = (old & lo) + 1;
    } else {
        unsigned long long w = old + inc, next;
        do {
            next = ours(w) ? w + inc : inc;
        } while (!__hip_atomic_compare_exchange_strong(word, &w, next, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                                       __HIP_MEMORY_SCOPE_AGENT));
        pos = next & lo;
    }
    if ((int64_t)pos < splits) return 0;
    __hip_atomic_store(word, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return 1;
}

// A8: int8 activation codes (the exact int8 path on a rotated file): staged
// as they are (16 codes per K half) and fed to the MFMA; the weights still
// enter as 16 x nibble, so d is scaled by 2^-4.
// The streaming GEMM of one workgroup: column tile `tile`, K split z.  With
// FUSED, the first records' weight loads are issued, then the workgroup waits
// for the activation quads of its split (published with `target`).
// REC: W4A4 activations from the record-ordered operand a.act_rec.
template <int WAVES, int DEPTH, bool A8, bool FUSED, bool REC = false>
__device__ __forceinline__ void small_m_tile(const SmallArgs &a, int64_t tile, int64_t z, uint8_t *smem,
                                             uint32_t target) {
    static_assert(!REC || (!A8 && !FUSED), "the record-ordered operand is W4A4, written before the launch");
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar loop control
    const int64_t k = a.k, nb = k / QK, nq = sq_quads(k);
    const int m = (int)a.m;
    const int64_t q_lo = z * a.range;
    const int nr = (int)min(nq - q_lo, a.range);  // records of this split (>= 1)

    // this wave's records: local index wave, wave + WAVES, ...
    const int cnt = nr > wave ? (nr - wave + WAVES - 1) / WAVES : 0;
    // Buffer loads: record offsets are scalar or fixed per lane, so no
    // address arithmetic touches the registers that loads are still filling;
    // the hardware range-checks every load (bytes past a buffer read zero).
    constexpr int CFG = 0x00020000;
    const __amdgpu_buffer_rsrc_t wbuf = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t *>(a.sq + (tile * nq + q_lo) * SQ_REC), 0, nr * SQ_REC, CFG);
    constexpr int ROW_BYTES = A8 ? QK : QK / 2;  // activation code bytes per (row, block)
    const int lo16 = lane * 16, d4 = SQ_SCALE_OFF + lane * 4;
    const int g = lane >> 5, r16 = lane & 15;  // K half and row (mod 16) of this lane in the MFMAs
    // A record's activations are loaded by its own wave, lane l = 4 r + j
    // taking row r's code bytes of the record's block j and its scale: each
    // group of 16 lanes covers 4 rows' 64 contiguous code bytes, not 16 rows
    // (a third fewer cycles per gather on the measured part).  From the public
    // codes and scales, the range check zeroes rows past m and the bytes past
    // the matrix (the weights of blocks past nb are zero, so what those lanes
    // read inside the matrix adds nothing); from the record-ordered operand
    // (W4A4, act_rec) both loads are contiguous.  The record position is part
    // of the lane offset because the range check does not cover the scalar
    // offset.
    const int ar = lane >> 2, ab = lane & 3;
    constexpr bool rec_act = REC;
    const __amdgpu_buffer_rsrc_t cbuf =
        rec_act ? __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(a.act_rec), 0, (int)small_act_bytes(k), CFG)
                : __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(a.codes), 0, (int)(m * nb * ROW_BYTES), CFG);
    const __amdgpu_buffer_rsrc_t sbuf =
        rec_act ? cbuf : __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(a.scales), 0, (int)(m * nb * 4), CFG);
    // This lane's pieces of quad q from one index t = t0 + q * T: codes at
    // t * CM, scale at t * SM + s_off (one register per lane, not two).
    const int t0 = rec_act ? lane * 4 : ar * (int)nb + ab;
    constexpr int T = rec_act ? SMA_SCALE_BYTES : SQ_BLOCKS;
    constexpr int CM = rec_act ? 4 : ROW_BYTES, SM = rec_act ? 1 : 4;
    const int s_off = rec_act ? (int)nq * SMA_CODE_BYTES : 0;
    struct Rec {
        v4u c0, c1;
        uint32_t d;
        uint4 ac[A8 ? 2 : 1];
        float as;
    };
    // Every wave issues the same loads whatever its count (slots past it
    // reload the split's last record, a cache hit), so the number of loads in
    // flight is the same on every path into the main loop and its waits stay
    // exact.
    auto load_w = [&](int i, Rec &R) {
        const int li = min(wave + WAVES * i, nr - 1);
        const int off = __builtin_amdgcn_readfirstlane(li * SQ_REC);
        R.c0 = __builtin_amdgcn_raw_buffer_load_b128(wbuf, lo16, off, 0);
        __builtin_amdgcn_sched_barrier(0);  // one issue order everywhere
        R.c1 = __builtin_amdgcn_raw_buffer_load_b128(wbuf, lo16 + 1024, off, 0);
        __builtin_amdgcn_sched_barrier(0);
        R.d = __builtin_amdgcn_raw_buffer_load_b32(wbuf, d4, off, 0);
        __builtin_amdgcn_sched_barrier(0);
    };
    // fused: the activations were written in this launch, read them with
    // device-scope (sc1) loads
    constexpr int ACT_CPOL = FUSED ? 16 : 0;
    auto load_a = [&](int i, Rec &R) {
        const int q = (int)q_lo + min(wave + WAVES * i, nr - 1);  // quad of this record
        const int t = t0 + q * T;
#pragma unroll
        for (int h = 0; h < (A8 ? 2 : 1); h++) {
            const v4u u = __builtin_amdgcn_raw_buffer_load_b128(cbuf, t * CM + 16 * h, 0, ACT_CPOL);
            R.ac[h] = make_uint4(u[0], u[1], u[2], u[3]);
            __builtin_amdgcn_sched_barrier(0);
        }
        R.as = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(sbuf, t * SM + s_off, 0, ACT_CPOL));
        __builtin_amdgcn_sched_barrier(0);
    };
    auto load = [&](int i, Rec &R) {
        load_w(i, R);
        load_a(i, R);
    };

    // This wave's LDS slot for one record's activations, in the MFMA's lane
    // order: [block][K half][row] 16 int8 codes (16 B), then the scale
    // operands [block][row] (8 B).
    constexpr int SLOT = SQ_BLOCKS * 2 * 16 * 16 + SQ_BLOCKS * 16 * 8;
    uint8_t *slot = smem + wave * SLOT;
    uint4 *codes16 = reinterpret_cast<uint4 *>(slot);
    uint2 *sop = reinterpret_cast<uint2 *>(slot + SQ_BLOCKS * 2 * 16 * 16);
    auto put = [&](const Rec &R) {
        if constexpr (A8) {
            codes16[(ab * 2 + 0) * 16 + ar] = R.ac[0];  // codes 0..15
            codes16[(ab * 2 + 1) * 16 + ar] = R.ac[1];  // codes 16..31
        } else {
            const uint4 w = k8_words(R.ac[0]);
            const v4i h0 = widen_k8x2(w.x, w.y), h1 = widen_k8x2(w.z, w.w);
            codes16[(ab * 2 + 0) * 16 + ar] = make_uint4(h0[0], h0[1], h0[2], h0[3]);
            codes16[(ab * 2 + 1) * 16 + ar] = make_uint4(h1[0], h1[1], h1[2], h1[3]);
        }
        sop[ab * 16 + ar] = act_scale_operand(R.as);
    };

    // outputs of rows 0..15: elements 0..7 of the 32x32 layout
    float acc[8];
#pragma unroll
    for (int v = 0; v < 8; v++) acc[v] = 0.0f;
    constexpr float UNSCALE = A8 ? 1.0f / 16.0f : 1.0f / 256.0f;  // the operands' 16 x factors
    // blocks bl and bl + 1 of the record: (w0, w1) this lane's words of
    // each, dh its d of block bl + g.  Lanes of rows 16..31 read row r % 16
    // (their outputs are not used).
    // Per block the scale products come from a single-block 32x32x8 MFMA
    // (half the result registers of the two-block form, which keeps the
    // kernel at three workgroups per CU): lane group g holds block bl + g's
    // operands, and the other group's A operand is zeroed.
    auto pair = [&](int bl, uint32_t w00, uint32_t w01, uint32_t w10, uint32_t w11, uint16_t dh) {
        const uint32_t wop = weight_scale_operand(__half2float(__ushort_as_half(dh)) * UNSCALE);
        const uint2 sa = sop[(bl + g) * 16 + r16], zero = make_uint2(0, 0);
        const v16f P0 = mfma_bf16_32x32x8(g ? zero : sa, make_uint2(wop, wop));
        const uint4 a0 = codes16[(bl * 2 + g) * 16 + r16];
        const v16i S0 = mfma_i8_32x32x32(v4i{(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w}, widen_k8x2(w00, w01));
#pragma unroll
        for (int v = 0; v < 8; v++) acc[v] = fmaf((float)S0[v], P0[v], acc[v]);
        const v16f P1 = mfma_bf16_32x32x8(g ? sa : zero, make_uint2(wop, wop));
        const uint4 a1 = codes16[((bl + 1) * 2 + g) * 16 + r16];
        const v16i S1 = mfma_i8_32x32x32(v4i{(int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w}, widen_k8x2(w10, w11));
#pragma unroll
        for (int v = 0; v < 8; v++) acc[v] = fmaf((float)S1[v], P1[v], acc[v]);
    };
    auto compute = [&](const Rec &R) {
        put(R);  // the same wave reads the slot next: LDS operations of a wave stay in order
        pair(0, R.c0[0], R.c0[1], R.c0[2], R.c0[3], (uint16_t)(R.d & 0xFFFF));
        pair(2, R.c1[0], R.c1[1], R.c1[2], R.c1[3], (uint16_t)(R.d >> 16));
    };

    // Ring of DEPTH records: record i + DEPTH - 1 is loaded before record i
    // is computed.  The loop is unrolled DEPTH times so that every ring index
    // is static; the scheduling barriers keep the loads ahead of the compute
    // (the scheduler would otherwise sink them to their first use).
    Rec ring[DEPTH];
    if constexpr (FUSED) {
        // the weights do not depend on the producers: start their stream,
        // then wait for this split's activations
#pragma unroll
        for (int j = 0; j < DEPTH - 1; j++) load_w(j, ring[j]);
        wait_for_quads(a, q_lo, nr, target);
#pragma unroll
        for (int j = 0; j < DEPTH - 1; j++) load_a(j, ring[j]);
    } else {
#pragma unroll
        for (int j = 0; j < DEPTH - 1; j++) load(j, ring[j]);
    }
    for (int i = 0; i < cnt; i += DEPTH) {
#pragma unroll
        for (int j = 0; j < DEPTH; j++) {
            load(i + j + DEPTH - 1, ring[(j + DEPTH - 1) % DEPTH]);
            __builtin_amdgcn_sched_barrier(0);
            compute(ring[j]);
            __builtin_amdgcn_sched_barrier(0);
            if (i + j + 1 >= cnt) break;
        }
    }

    // the waves' sums meet in LDS (ascending wave order), then one store
    __syncthreads();  // every wave is done with its activation slot
    float *red = reinterpret_cast<float *>(smem);  // [wave][8][64]
#pragma unroll
    for (int v = 0; v < 8; v++) red[(wave * 8 + v) * 64 + lane] = acc[v];
    __syncthreads();
    uint32_t *part = reinterpret_cast<uint32_t *>(a.partial);
    for (int i = tid; i < 512; i += 64 * WAVES) {
        const int v = i >> 6, l = i & 63;
        float sum = red[i];
#pragma unroll
        for (int w = 1; w < WAVES; w++) sum += red[w * 512 + i];
        const int r = mfma32_row(v, l);  // v < 8: rows 0..15
        const int64_t col = tile * TILE_N + (l & 31);
        if (r < m && col < a.n) {
            // partial sums are stored device-scope (write-through), so the
            // tile's last workgroup reads them from any XCD
            if (part)
                __hip_atomic_store(part + (z * a.m + r) * a.n + col, __float_as_uint(sum), __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
            else a.y[(int64_t)r * a.ldy + col] = sum;
        }
    }
    if (!part) return;  // uniform

    // K split: every thread's partial stores have completed before the
    // barrier, so the arrival counted after it follows them
    const int64_t splits = (sq_quads(k) + a.range - 1) / a.range;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    int *last = reinterpret_cast<int *>(smem + sm_red_bytes(WAVES));  // after the reduction
    if (tid == 0) *last = small_m_arrive(a.arrivals + tile, a.ticket, splits);
    __syncthreads();
    if (!*last) return;  // uniform
    const int64_t mn = a.m * a.n;
    for (int i = tid; i < 512; i += 64 * WAVES) {
        const int v = i >> 6, l = i & 63;
        const int r = mfma32_row(v, l);
        const int64_t col = tile * TILE_N + (l & 31);
        if (r >= m || col >= a.n) continue;
        const uint32_t *p = part + (int64_t)r * a.n + col;
        float sum = 0.0f;
        for (int64_t z0 = 0; z0 < splits; z0 += 8) {  // eight loads in flight, then the adds in order
            float x[8];
#pragma unroll
            for (int j = 0; j < 8; j++)
                x[j] = __uint_as_float(
                    __hip_atomic_load(p + min(z0 + j, splits - 1) * mn, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
#pragma unroll
            for (int j = 0; j < 8; j++)
                if (z0 + j < splits) sum = z0 + j == 0 ? x[j] : sum + x[j];
        }
        a.y[(int64_t)r * a.ldy + col] = sum;
    }
}

// Grid (tiles, splits).  8 waves: at most 80 registers (int4 activations),
// six waves per SIMD keep three workgroups resident per CU, so the 544
// workgroups of a 17408-column projection run in one round.  16 waves (long
// K, at most a few hundred workgroups): four waves per SIMD, one workgroup
// per CU.
// Item c of a plan (small_m_items): whole tiles first, then the split
// tiles' ranges, range-major (range 0 of every split tile, then range 1, ...).
// Returns the tile and range and the arguments for that item.
__device__ __forceinline__ SmallArgs small_m_item(const SmallArgs &a, int64_t c, int64_t &tile, int64_t &z) {
    SmallArgs b = a;
    if (c < a.whole) {
        tile = c;
        z = 0;
        b.range = sq_quads(a.k);
        b.partial = nullptr;
    } else {
        const int64_t split_tiles = padded_n(a.n) / TILE_N - a.whole, p = c - a.whole;
        tile = a.whole + p % split_tiles;
        z = p / split_tiles;
    }
    return b;
}

template <int WAVES, int DEPTH, bool A8 = false, bool REC = false>
__global__ __launch_bounds__(64 * WAVES, A8 ? 1 : WAVES > 8 ? 4 : 6) void gemm_small_m_kernel(SmallArgs a) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    int64_t tile, z;
    const SmallArgs b = small_m_item(a, blockIdx.x, tile, z);
    small_m_tile<WAVES, DEPTH, A8, false, REC>(b, tile, z, smem, 0);
}

// ---------------------------------------------------------------------------
// Rotate-quantise fused into the m <= 16 product, one launch: workgroups
// 0 .. producers - 1 quantise the activations (fuse_quads(WAVES) quads of 4 blocks
// each, every row; the quantiser's own per-block code, so the codes are the
// standalone quantiser's bit for bit) into the public codes and scales and
// publish each quad by storing the call's epoch + 1 into its flag (release);
// the other workgroups are the streaming GEMM's (tile, split), in the
// unfused grid's order.  Workgroups are dispatched in index order, so every
// producer is running or done before a consumer can wait for it; the wait
// is bounded all the same.  Each call's epoch comes from the workspace: all
// workgroups read it at their start, and the last one to finish (by a
// device-scope count) advances it and clears the count, so the workspace is
// ready for the next call without a separate clearing launch.
// ---------------------------------------------------------------------------
// quads per producer workgroup: one thread per lane of a (block, row) quad,
// 4 blocks x 16 rows x 4 lanes = 256 threads per quad of blocks
__host__ __device__ constexpr int fuse_quads(int waves) { return waves * 64 / (SQ_BLOCKS * SMALL_M_MAX * 4); }

template <int QUADS, typename T>
__device__ __forceinline__ void fused_producer(const SmallArgs &a, int64_t pid, uint32_t target) {
    const int tid = threadIdx.x, L = tid & 3, g = tid >> 2;  // quad g: row g % 16, block g / 16
    const int row = g & 15;
    const int64_t nb = a.k / QK, nq = sq_quads(a.k);
    const int64_t b = pid * QUADS * SQ_BLOCKS + (g >> 4);
    const bool live = row < a.m && b < nb;  // uniform per quad
    int q[8];
    float s;
    quantise_quad<T, 7, true>(static_cast<const T *>(a.x) + row * a.ldx + b * QK + 8 * L, a.mode, live, L, q, s);
    store_codes4<true>(q, s, L, live, a.codes_out + row * (a.k / 2) + b * 16, a.scales_out + row * nb + b);
    // every thread's device-scope stores have completed before the barrier,
    // so the flags, stored after it, follow them
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (tid < QUADS) {
        const int64_t quad = pid * QUADS + tid;
        if (quad < nq) __hip_atomic_store(a.flags + quad, target, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

template <int WAVES, int DEPTH, typename T>
__global__ __launch_bounds__(64 * WAVES, WAVES > 8 ? 4 : 6) void gemm_small_m_fused_kernel(SmallArgs a, uint32_t total) {
    // (the unfused kernel's occupancy: the waiting consumers and the
    // producers are resident together)
    static_assert(64 * WAVES == fuse_quads(WAVES) * SQ_BLOCKS * SMALL_M_MAX * 4, "one producer thread per lane of a quad");
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    const uint32_t epoch = __hip_atomic_load(a.sync, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const uint32_t target = epoch + 1;
    const int64_t id = blockIdx.x;
    if (id < a.producers) {
        fused_producer<fuse_quads(WAVES), T>(a, id, target);  // uniform per workgroup
    } else {
        int64_t tile, z;
        const SmallArgs b = small_m_item(a, id - a.producers, tile, z);
        small_m_tile<WAVES, DEPTH, false, true>(b, tile, z, smem, target);
    }
    // the last workgroup to finish advances the epoch for the next call (the
    // next call reads it after this launch has ended: no fence is needed)
    __syncthreads();
    if (threadIdx.x == 0 && atomicAdd(a.sync + 1, 1u) + 1 == total) {
        __hip_atomic_store(a.sync + 1, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(a.sync, target, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

// LDS bytes of one workgroup: the waves' activation slots, or the cross-wave
// reduction and the last-arrival word if that is larger.
__host__ inline size_t small_m_lds_bytes(const SmallPlan &p) {
    const size_t slots = (size_t)p.waves * SQ_BLOCKS * (2 * 16 * 16 + 16 * 8), red = (size_t)sm_red_bytes(p.waves) + 16;
    return slots > red ? slots : red;
}

// Workspace of an m <= 16 product that splits K: the tiles' arrival words,
// then the splits' partial sums (both in whole 256-byte units); 0 without a
// split.
__host__ inline size_t small_m_arrival_bytes(const SmallPlan &p) { return (size_t)((p.tiles * 8 + 255) / 256 * 256); }
__host__ inline size_t small_m_workspace_bytes(const SmallPlan &p, int64_t m, int64_t n) {
    return p.splits > 1 ? small_m_arrival_bytes(p) + (size_t)((p.splits * m * n * 4 + 255) / 256 * 256) : 0;
}

// y = sum over the K splits of the partial sums, in ascending split order
// (the dense kernel's split K).  The loads of eight splits are issued together (clamped past the last
// split, which then adds nothing), so the latency is paid once per eight.
__global__ __launch_bounds__(256) void small_m_reduce_kernel(const float *__restrict__ partial, int64_t splits,
                                                             int64_t m, int64_t n, float *__restrict__ y,
                                                             int64_t ldy) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= m * n) return;
    const int64_t mn = m * n;
    float sum = 0.0f;
    for (int64_t z0 = 0; z0 < splits; z0 += 8) {
        float v[8];
#pragma unroll
        for (int j = 0; j < 8; j++) v[j] = partial[min(z0 + j, splits - 1) * mn + i];
#pragma unroll
        for (int j = 0; j < 8; j++)
            if (z0 + j < splits) sum = (z0 + j == 0) ? v[j] : sum + v[j];
    }
    y[(i / n) * ldy + i % n] = sum;
}

}  // namespace w4a4
