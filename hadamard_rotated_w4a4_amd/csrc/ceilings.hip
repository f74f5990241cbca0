// libw4a4_ceilings.so: the practical ceilings the GEMMs are measured against
// on the running part, beside the published peaks.  Not part of the W4A4
// path: the benchmark reports each kernel's rate as a fraction of the
// published peak and of these measured ceilings.
//
//   w4a4c_read_stream  HBM read bandwidth: every byte of a buffer larger than
//                      the last-level cache read once with 16-byte loads,
//                      four in flight per thread, grid-stride.
//   w4a4c_mfma_loop    matrix-core issue rate over the whole chip: each wave
//                      runs independent chains of one MFMA kind (no memory
//                      traffic), two waves per SIMD.
//
// Both are plain bounded loops with in-bounds accesses; results are folded
// into one value per thread so that nothing is optimised away.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));

__global__ __launch_bounds__(256) void read_stream_kernel(const uint4 *__restrict__ p, int64_t n16,
                                                          uint32_t *__restrict__ sink) {
    const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    uint32_t acc = 0;
    int64_t i = tid;
    for (; i + 3 * stride < n16; i += 4 * stride) {
        const uint4 a = p[i], b = p[i + stride], c = p[i + 2 * stride], d = p[i + 3 * stride];
        acc ^= a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w ^ c.x ^ c.y ^ c.z ^ c.w ^ d.x ^ d.y ^ d.z ^ d.w;
    }
    for (; i < n16; i += stride) {
        const uint4 a = p[i];
        acc ^= a.x ^ a.y ^ a.z ^ a.w;
    }
    sink[tid] = acc;
}

// KIND 0: FP6 E2M3 v_mfma_scale_f32_32x32x64_f8f6f4 (the dense W4A4 block
// dot); KIND 1: v_mfma_i32_32x32x32_i8.  Four independent accumulators per
// wave, so the rate is the issue rate, not the latency.
template <int KIND>
__global__ __launch_bounds__(256) void mfma_loop_kernel(int iters, float *__restrict__ sink) {
    const int lane = threadIdx.x & 63;
    float out = 0.0f;
    if constexpr (KIND == 0) {
        v8i a = {lane, lane * 3, lane * 5, lane * 7, lane * 11, lane * 13, 0, 0};
        v8i b = {lane * 2, lane * 4, lane * 6, lane * 8, lane * 10, lane * 12, 0, 0};
        v16f c0 = {}, c1 = {}, c2 = {}, c3 = {};
        for (int it = 0; it < iters; it++) {
            c0 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c0, 2, 2, 0, 127, 0, 127);
            c1 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c1, 2, 2, 0, 127, 0, 127);
            c2 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c2, 2, 2, 0, 127, 0, 127);
            c3 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c3, 2, 2, 0, 127, 0, 127);
        }
        for (int v = 0; v < 16; v++) out += c0[v] + c1[v] + c2[v] + c3[v];
    } else {
        v4i a = {lane, lane * 3, lane * 5, lane * 7};
        v4i b = {lane * 2, lane * 4, lane * 6, lane * 8};
        v16i c0 = {}, c1 = {}, c2 = {}, c3 = {};
        for (int it = 0; it < iters; it++) {
            c0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c0, 0, 0, 0);
            c1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c1, 0, 0, 0);
            c2 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c2, 0, 0, 0);
            c3 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c3, 0, 0, 0);
        }
        for (int v = 0; v < 16; v++) out += (float)(c0[v] ^ c1[v] ^ c2[v] ^ c3[v]);
    }
    sink[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = out;
}

}  // namespace

extern "C" {

// Reads `bytes` (a multiple of 16) of `buf` once; sink: device, one uint32
// per thread of `blocks` x 256 threads.  Returns 0, or the hipError_t of the
// launch.
int w4a4c_read_stream(const void *buf, int64_t bytes, void *sink, int blocks, void *stream) {
    if (!buf || !sink || bytes <= 0 || bytes % 16 || blocks <= 0) return (int)hipErrorInvalidValue;
    read_stream_kernel<<<blocks, 256, 0, (hipStream_t)stream>>>((const uint4 *)buf, bytes / 16, (uint32_t *)sink);
    return (int)hipGetLastError();
}

// kind 0: FP6 32x32x64 (131072 flops each), kind 1: int8 32x32x32 (65536
// ops each); every wave of `blocks` x 256 threads issues 4 x iters MFMAs.
// sink: device, one float per thread.
int w4a4c_mfma_loop(int kind, int iters, int blocks, void *sink, void *stream) {
    if (!sink || iters <= 0 || blocks <= 0 || (kind != 0 && kind != 1)) return (int)hipErrorInvalidValue;
    if (kind == 0) mfma_loop_kernel<0><<<blocks, 256, 0, (hipStream_t)stream>>>(iters, (float *)sink);
    else mfma_loop_kernel<1><<<blocks, 256, 0, (hipStream_t)stream>>>(iters, (float *)sink);
    return (int)hipGetLastError();
}

}  // extern "C"
