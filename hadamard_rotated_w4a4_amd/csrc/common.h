// Device-side helpers shared by the W4A4 kernels (gfx950 / CDNA4 only).
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

namespace w4a4 {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

constexpr int QK = 32;               // Q4_0 block length along K
constexpr int TILE_N = 32;           // columns per packed weight tile (one MFMA N)
constexpr int TILE_CODE_BYTES = 512; // packed codes of one (tile, block): 32 cols x 16 B
constexpr int TILE_SCALE_HALFS = 32; // fp16 scales of one (tile, block)

// Packed weight layout (written by the repack kernel, read by the GEMMs):
//   codes  [Np/32][nb][64 lanes][8 B]; lane l = 32g + c holds bytes 8g..8g+7
//          of column c's Q4_0 block, each byte XOR 0x88 (signed nibbles).
//   scales [Np/32][nb][32] fp16, directly after the codes.
// Np = n rounded up to 32; padded columns hold zero codes and zero scales.
__host__ __device__ inline int64_t padded_n(int64_t n) { return (n + TILE_N - 1) / TILE_N * TILE_N; }
__host__ __device__ inline int64_t packed_code_bytes(int64_t n, int64_t k) {
    return padded_n(n) / TILE_N * (k / QK) * TILE_CODE_BYTES;
}
__host__ __device__ inline int64_t packed_total_bytes(int64_t n, int64_t k) {
    return padded_n(n) / TILE_N * (k / QK) * (TILE_CODE_BYTES + 2 * TILE_SCALE_HALFS);
}

// Eight packed bytes (16 signed nibbles) -> sixteen int8 lanes of an MFMA
// operand, each holding 16 * nibble: masking the high nibble keeps it in
// place (two's complement survives), shifting the low nibble up by 4 does the
// same for it.  Products therefore carry a factor 256, which the epilogue
// folds into the weight scale.  A and B go through the same permutation, so
// the dot over the 32 K positions is unchanged.
__device__ __forceinline__ v4i unpack_nibbles_x16(uint32_t lo_word, uint32_t hi_word) {
    v4i r;
    r.x = (int)((lo_word << 4) & 0xF0F0F0F0u);
    r.y = (int)((hi_word << 4) & 0xF0F0F0F0u);
    r.z = (int)(lo_word & 0xF0F0F0F0u);
    r.w = (int)(hi_word & 0xF0F0F0F0u);
    return r;
}

__device__ __forceinline__ v16i mfma_i8_32x32x32(v4i a, v4i b) {
    v16i zero = {0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};
    return __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, zero, 0, 0, 0);
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
