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
//   bytes [768, 1024)  4 B at 768 + 4 (32 g + c) (g = 0, 1): the bf16 part d_g
//                      of 64 * d = d_0 + d_1 (exact; d the column's fp16 Q4_0
//                      scale) in both halves, so that lane 32 g + c of the
//                      scale-product MFMA reads its operand as one dword.
// A 32x32x64 MFMA lane l takes its operand from the record of block b + l/32
// (lanes 32..63 the next block), so one operand register set carries two
// blocks; per-lane MX scales select one of them per MFMA.
// The activation operand built by the GEMM's pre-pass has the same record
// shape per (32-row tile, block), with a bf16 triple per row at 768.
__host__ __device__ inline int64_t padded_n(int64_t n) { return (n + TILE_N - 1) / TILE_N * TILE_N; }
constexpr int MX_REC = 1024;            // bytes per (tile, block) record
constexpr int MX_CODE_BYTES = 768;      // fp6 codes of 32 rows / columns
constexpr int MX_BLOCK_PAD = 8;         // records per tile are padded to a multiple of this
__host__ __device__ inline int64_t mx_blocks(int64_t k) { return (k / QK + MX_BLOCK_PAD - 1) / MX_BLOCK_PAD * MX_BLOCK_PAD; }
// Streaming section (the m <= 16 kernel), directly after the matrix-core
// section (a multiple of 1 KB): [Np/32][nq][2304 B] with nq = ceil(nb / 4), one record
// per (32-column tile, 4 consecutive blocks).  Per column and block the 32
// signed codes (q ^ 8) form four "K8 words", one per K-group g of 8 codes:
// byte i of word g holds code 8 g + i in its low nibble and code 8 g + 4 + i
// in its high nibble.  Lane l = 16 g + c (c < 16) of a 16x16x32 int8 MFMA
// wants word g of columns c and 16 + c:
//   bytes [0, 1024)     lane l's 16 B at 16 l: blocks 0 and 1 of the record,
//                       each as (word of column c, word of column 16 + c);
//   bytes [1024, 2048)  the same for blocks 2 and 3;
//   bytes [2048, 2304)  16 B at 2048 + 16 c: for blocks 0..3 the fp16 pair
//                       (d of column c, d of column 16 + c).
// Blocks past nb and padding columns hold zero codes and zero scales.  A wave
// reads a record with three 16-byte loads per lane, the first two contiguous.
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

// 32x32x8 bf16 MFMA: 4 bf16 per lane, lane groups l/32 hold K 0..3 and 4..7.
__device__ __forceinline__ v16f mfma_bf16_32x32x8(uint2 a, uint2 b) {
    v16f zero = {0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};
    return __builtin_amdgcn_mfma_f32_32x32x8bf16_1k(__builtin_bit_cast(v4s, a), __builtin_bit_cast(v4s, b),
                                                   zero, 0, 0, 0);
}

// A K8 word (8 signed nibbles, see the streaming section) as 8 int8 MFMA
// operand bytes, each 16 x the nibble, in K order: 3 bit operations.
__device__ __forceinline__ long widen_k8(uint32_t w) {  // 8 signed nibbles -> 8 x int8 (x 16), K order
    const uint32_t lo = (w << 4) & 0xF0F0F0F0u, hi = w & 0xF0F0F0F0u;
    return (long)((uint64_t)hi << 32 | lo);
}

__device__ __forceinline__ v4i mfma_i8_16x16x32(long a, long b) {
    return __builtin_amdgcn_mfma_i32_16x16x32_i8(a, b, v4i{0, 0, 0, 0}, 0, 0, 0);
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
