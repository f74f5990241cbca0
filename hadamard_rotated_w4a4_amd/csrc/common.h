// Device-side helpers shared by the W4A4 kernels (gfx950 / CDNA4 only).
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

namespace w4a4 {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef unsigned int v4u __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef short v4s __attribute__((ext_vector_type(4)));

constexpr int QK = 32;               // Q4_0 block length along K
constexpr int TILE_N = 32;           // columns per packed weight tile (one MFMA N)

// Packed weight layout (written by the repack kernels, read by the GEMMs).
// Np = n rounded up to 32; padding columns hold zero codes and zero scales.
// Two sections hold the same weights losslessly, one per reader.
//
// Matrix-core section (the m > 16 kernels), at offset 0: [Np/32][nbp][1 KB]
// with nbp = nb rounded up to MX_BLOCK_PAD.  One 1 KB record per (32-column
// tile, block).  Column c's 32 codes (each q - 8) form one 192-bit MFMA lane
// operand of FP6 E2M3 fields, code t at bits 6t..6t+5; its six dwords lie in
// three planes so that 32 lanes read each plane conflict-free:
//   bytes [0, 768)     dwords 2p, 2p + 1 of column c at 256 p + 8 c (p < 3);
//   bytes [768, 896)   4 B at 768 + 4 c: the bf16 pair (d_0, d_1) with
//                      64 * d = d_0 + d_1 exactly (d the column's fp16 Q4_0
//                      scale; d_0 its leading 8 bits, d_1 the remaining 3);
//   bytes [896, 1024)  zero.
// A 32x32x64 MFMA lane l takes its operand from the record of block b + l/32
// (lanes 32..63 the next block), so one operand register set carries two
// blocks; per-lane MX scales select one of them per MFMA.  The scale-product
// MFMA (32x32x4, two blocks per instruction) reads lane l's (d_0, d_1) from
// the same record as the codes.
// The activation operand built by the GEMM's pre-pass has the same record
// shape per (32-row tile, block); at 768 + 8 r it holds the bf16 quadruple
// (s_1, s_1, s_2, s_2) of row r's scale, s_1 its leading 8 bits and s_2 the
// next 8 (s_1 + s_2 is s to within 2^-16 relative).
__host__ __device__ inline int64_t padded_n(int64_t n) { return (n + TILE_N - 1) / TILE_N * TILE_N; }
constexpr int MX_REC = 1024;            // bytes per (tile, block) record
constexpr int MX_CODE_BYTES = 768;      // fp6 codes of 32 rows / columns
constexpr int MX_BLOCK_PAD = 8;         // records per tile are padded to a multiple of this
__host__ __device__ inline int64_t mx_blocks(int64_t k) { return (k / QK + MX_BLOCK_PAD - 1) / MX_BLOCK_PAD * MX_BLOCK_PAD; }
// Streaming section (the m <= 16 and grouped kernels), directly after the
// matrix-core section (a multiple of 1 KB): [Np/32][nq][2304 B] with
// nq = ceil(nb / 4), one record per (32-column tile, 4 consecutive blocks).
// Per column and block the 32 signed codes (q ^ 8) form four "K8 words", one
// per K-group w of 8 codes: byte i of word w holds code 8 w + i in its low
// nibble and code 8 w + 4 + i in its high nibble.  Lane l = 32 g + c of a
// 32x32x32 int8 MFMA takes codes 16 g .. 16 g + 15 (words 2 g and 2 g + 1)
// of column c:
//   bytes [0, 1024)     lane l's 16 B at 16 l: for blocks 0 and 1 of the
//                       record, words 2 g and 2 g + 1 of column c;
//   bytes [1024, 2048)  the same for blocks 2 and 3;
//   bytes [2048, 2304)  4 B at 2048 + 4 l: the fp16 d of column c for block g
//                       (low half) and block 2 + g (high half), the lane's
//                       operands of the two two-block scale-product MFMAs.
// Blocks past nb and padding columns hold zero codes and zero scales.  A wave
// reads a record with two 16-byte loads and one 4-byte load per lane.
constexpr int SQ_BLOCKS = 4;            // blocks per streaming record
constexpr int SQ_REC = 2304;            // bytes per (tile, 4 blocks) record
constexpr int SQ_SCALE_OFF = 2048;
__host__ __device__ inline int64_t sq_quads(int64_t k) { return (k / QK + SQ_BLOCKS - 1) / SQ_BLOCKS; }
__host__ __device__ inline int64_t sq_section_offset(int64_t n, int64_t k) {
    return padded_n(n) / TILE_N * mx_blocks(k) * MX_REC;
}
__host__ __device__ inline int64_t packed_total_bytes(int64_t n, int64_t k) {
    return sq_section_offset(n, k) + padded_n(n) / TILE_N * sq_quads(k) * SQ_REC;
}
// Record-ordered activation operand of an m <= 16 product (written by the
// quantiser, read by the streaming kernel), for nq quads of 4 blocks, in the
// order a wave loads them:
//   bytes [0, 1024 nq)            quad q's codes at 1024 q: row r's 16 code
//                                 bytes of block 4 q + j at 64 r + 16 j (the
//                                 bytes of the public int4 codes);
//   bytes [1024 nq, 1280 nq)      quad q's scales at 1024 nq + 256 q: row r's
//                                 fp32 scale of block 4 q + j at 16 r + 4 j.
// Rows m .. 15 and blocks past nb hold zero codes and zero scales.  Lane
// l = 4 r + j reads one 16 B and one 4 B piece: both loads are contiguous.
// (Codes and scales in separate runs measured ~8% faster than one 1280 B
// record per quad.)
constexpr int SMA_ROWS = 16;
constexpr int SMA_CODE_BYTES = 1024;    // per quad
constexpr int SMA_SCALE_BYTES = 256;    // per quad
__host__ __device__ inline int64_t small_act_bytes(int64_t k) { return sq_quads(k) * (SMA_CODE_BYTES + SMA_SCALE_BYTES); }
// The four K8 words of one block from its 16 Q4_0 code bytes (u.x = bytes
// 0..3, ...; byte j holds code j low and code j + 16 high).
__host__ __device__ inline uint4 k8_words(uint4 u) {
    uint4 w;
    w.x = (u.x & 0x0F0F0F0Fu) | (u.y & 0x0F0F0F0Fu) << 4;         // codes 0..7
    w.y = (u.z & 0x0F0F0F0Fu) | (u.w & 0x0F0F0F0Fu) << 4;         // codes 8..15
    w.z = (u.x >> 4 & 0x0F0F0F0Fu) | (u.y & 0xF0F0F0F0u);         // codes 16..23
    w.w = (u.z >> 4 & 0x0F0F0F0Fu) | (u.w & 0xF0F0F0F0u);         // codes 24..31
    return w;
}

// FP6 E2M3 code of the integer q in [-8, 8], read by the MFMA as q / 8: the
// five magnitude bits of E2M3 are linear in the value for magnitudes below
// 2 (subnormals m / 8, then 1 + m / 8), so |q| itself is the magnitude field.
__host__ __device__ inline uint32_t fp6_e2m3_of(int q) { return (q < 0 ? 0x20u : 0u) | (uint32_t)(q < 0 ? -q : q); }

// Pack 32 six-bit fields (element j at bits 6j..6j+5) into six dwords.
__host__ __device__ inline void pack_fp6x32(const uint32_t f[32], uint32_t w[6]) {
    for (int i = 0; i < 6; i++) w[i] = 0;
    for (int j = 0; j < 32; j++) {
        const int bit = 6 * j, dw = bit >> 5, off = bit & 31;
        w[dw] |= f[j] << off;
        if (off > 26) w[dw + 1] |= f[j] >> (32 - off);
    }
}

// Write the operand of row / column r (six dwords) into a record (layout above).
__host__ __device__ inline void put_mx_row(uint8_t *rec, int r, const uint32_t w[6]) {
    for (int p = 0; p < 3; p++) reinterpret_cast<uint2 *>(rec + 256 * p)[r] = make_uint2(w[2 * p], w[2 * p + 1]);
}

// Scale products of two blocks at once: the 32x32x4 bf16 MFMA in its
// two-block form.  Lane l supplies 4 bf16 K values of row (A) or column (B)
// l % 32 of block l / 32; the result holds block 0's 32x32 tile in elements
// 0..15 and block 1's in 16..31, each in the usual 32x32 output layout.
typedef float v32f __attribute__((ext_vector_type(32)));
__device__ __forceinline__ v32f mfma_bf16_32x32x4_2blk(uint2 a, uint2 b) {
    v32f zero = {};
    return __builtin_amdgcn_mfma_f32_32x32x4bf16_1k(__builtin_bit_cast(v4s, a), __builtin_bit_cast(v4s, b), zero, 0,
                                                   0, 0);
}

// Scale products of one block: the 32x32x8 bf16 MFMA, whose K slots 0..3
// come from lanes 0..31 and 4..7 from lanes 32..63; the caller zeroes one
// lane group's A operand so that only the other group's block contributes.
__device__ __forceinline__ v16f mfma_bf16_32x32x8(uint2 a, uint2 b) {
    return __builtin_amdgcn_mfma_f32_32x32x8bf16_1k(__builtin_bit_cast(v4s, a), __builtin_bit_cast(v4s, b), v16f{}, 0,
                                                   0, 0);
}

// Scale operands of the two-block scale-product MFMA (K slots k = 0..3 of a
// lane pair up as A_k * B_k).
// Activation row: (s_1, s_1, s_2, s_2), s_1 the leading 8 bits of s
// (truncation), s_2 the leading 8 bits of the exact remainder s - s_1.
__device__ __forceinline__ uint2 act_scale_operand(float s) {
    const uint32_t h1 = __float_as_uint(s) & 0xFFFF0000u;
    const float r1 = __fsub_rn(s, __uint_as_float(h1));
    const uint32_t h2 = __float_as_uint(r1) & 0xFFFF0000u;
    return make_uint2(h1 | (h1 >> 16), h2 | (h2 >> 16));
}
// Weight column: (d_0, d_1) with d_0 + d_1 = x exactly for x = 64 * d (d an
// fp16 value: 11 significant bits, the leading 8 in d_0, the rest in d_1);
// the MFMA reads it twice, as (d_0, d_1, d_0, d_1).
__device__ __forceinline__ uint32_t weight_scale_operand(float x) {
    const uint32_t h1 = __float_as_uint(x) & 0xFFFF0000u;
    const float r1 = __fsub_rn(x, __uint_as_float(h1));  // exact: at most 3 significant bits remain
    const uint32_t h2 = __float_as_uint(r1) & 0xFFFF0000u;
    return (h1 >> 16) | h2;
}

// A K8 word (8 signed nibbles, see the streaming section) as 8 int8 MFMA
// operand bytes, each 16 x the nibble, in K order: 3 bit operations.
__device__ __forceinline__ long widen_k8(uint32_t w) {  // 8 signed nibbles -> 8 x int8 (x 16), K order
    const uint32_t lo = (w << 4) & 0xF0F0F0F0u, hi = w & 0xF0F0F0F0u;
    return (long)((uint64_t)hi << 32 | lo);
}

typedef int v16i __attribute__((ext_vector_type(16)));
// The integer dot of one block for a 32x32 tile: lane l gives 16 int8 codes
// of row / column l % 32 (K half l / 32, the same K order on both sides);
// the result is in the usual 32x32 output layout.
__device__ __forceinline__ v16i mfma_i8_32x32x32(v4i a, v4i b) {
    return __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, v16i{}, 0, 0, 0);
}
// Two K8 words as the 16 int8 operand bytes of one lane (each 16 x the
// nibble), in K order.
__device__ __forceinline__ v4i widen_k8x2(uint32_t w0, uint32_t w1) {
    const long a = widen_k8(w0), b = widen_k8(w1);
    return v4i{(int)(uint32_t)a, (int)(uint32_t)((uint64_t)a >> 32), (int)(uint32_t)b, (int)(uint32_t)((uint64_t)b >> 32)};
}

// Materialise a value in a register so that the compiler cannot fuse the
// operation producing it with the one consuming it (e.g. a multiply folded
// into a mixed-precision conversion as fma(x, c, +0), which loses -0.0).
__device__ __forceinline__ float opaque(float x) {
    asm volatile("" : "+v"(x));
    return x;
}

// Output layout of a 32x32 MFMA tile: lane l holds column l % 32; accumulator
// register v holds row 8*(v/4) + 4*(l/32) + (v%4).
__device__ __forceinline__ int mfma32_row(int v, int lane) {
    return 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
}

}  // namespace w4a4
