// libw4a4.so: host side of the C ABI declared in include/w4a4.h.
//
// Every entry point validates its arguments on the host, then enqueues its
// kernels on the caller's stream and returns; nothing here allocates, frees
// or synchronises.
#include "w4a4.h"

#include <algorithm>
#include <atomic>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "common.h"
#include "k_dense.h"
#include "k_grouped.h"
#include "k_prep.h"
#include "k_rotq.h"
#include "k_route.h"
#include "k_smallm.h"
#include "k_w16.h"

using namespace w4a4;

namespace {

thread_local char g_last_hip_error[256] = "";

w4a4_status hip_status(const char *what) {
    const hipError_t err = hipGetLastError();
    if (err == hipSuccess) return W4A4_OK;
    std::snprintf(g_last_hip_error, sizeof g_last_hip_error, "%s: %s", what, hipGetErrorString(err));
    return W4A4_ERR_HIP;
}

inline bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }
inline hipStream_t as_stream(void *s) { return reinterpret_cast<hipStream_t>(s); }
inline unsigned blocks_for(int64_t work, int per) { return (unsigned)((work + per - 1) / per); }
inline size_t up256_bytes(int64_t b) { return (size_t)((b + 255) / 256 * 256); }
// An odd 48-bit ticket per m <= 16 launch that splits K, for its tiles'
// arrival words: the top 48 bits of the call count times an odd 64-bit
// constant (a Weyl sequence), made odd, so that a word of the ticket's form
// (see small_m_arrive) looks like no small integer or float pair that a
// workspace may hold.  A captured launch keeps its ticket on every replay,
// which is sound because each launch leaves the words at zero.
std::atomic<uint64_t> g_calls{0};
unsigned long long next_ticket() {
    return (((g_calls.fetch_add(1, std::memory_order_relaxed) + 1) * 0x9E3779B97F4A7C15ull) >> 16) | 1ull;
}
// m <= 16 with a K split: the arrival words at the workspace's start, the
// partial sums after them
inline void set_small_m_split(SmallArgs &a, const SmallPlan &p, void *workspace) {
    a.whole = p.whole;
    if (p.splits <= 1) return;
    a.arrivals = static_cast<unsigned long long *>(workspace);
    a.partial = reinterpret_cast<float *>(static_cast<uint8_t *>(workspace) + small_m_arrival_bytes(p));
    a.ticket = next_ticket();
}
// y[0..m)[0..n) = 0 (row stride ldy): a grid-stride kernel on at most 2^16 workgroups
inline void launch_zero_rows(float *y, int64_t m, int64_t n, int64_t ldy, hipStream_t s) {
    zero_rows_kernel<<<(unsigned)std::min<int64_t>((m * n + 255) / 256, 1 << 16), 256, 0, s>>>(y, m, n, ldy);
}

// Dense m > 16: stages of 2 blocks, a ring of 4 stages; workgroup tiles of
// 128 x 128, 128 x 64 or 64 x 128, chosen per problem (see launch_mx).
using Mx128x128 = MxCfg<2, 4, 2, 2>;
using Mx128x64 = MxCfg<2, 4, 2, 1>;
using Mx64x128 = MxCfg<2, 4, 1, 2>;
// int8 activations (two FP6 planes in one operand set, one block per
// stage): 128 x 128 and 64 x 128 tiles (a 128 x 64 stage would not split
// into equal loads over the four waves).  Two-block stages in a 3-stage
// ring (72 KB, still two workgroups per CU) measured slower: 127 against
// 116-117 us at FFN up.
using Mx128x128A8 = MxCfg<1, 4, 2, 2, true>;
using Mx64x128A8 = MxCfg<1, 4, 1, 2, true>;

// Compute units of the current device (cached per device).
int device_cus() {
    static int cache[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (!cache[dev]) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cache[dev] = n;
    }
    return cache[dev];
}

template <class C>
int mx_occupancy() {  // resident workgroups per CU (registers and LDS decide)
    static const int occ = [] {
        int n = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, gemm_mx_kernel<C>, C::NT, 0) != hipSuccess || n < 1)
            n = 1;
        return n;
    }();
    return occ;
}

// Launch plan of one tile shape.  Whole rounds of resident workgroups take
// whole tiles; the leftover tiles either form one more (partial) round or,
// when that is cheaper, are split into pieces (a piece is 1/PIECES of a tile
// at about 1.6x the cost per output: no operand reuse across waves).  The
// modelled time counts rounds x padded work per tile (the smaller tiles reuse
// operands less: ~15% slower per output on MI355X, ~35% with int8 activations,
// whose stages are one block and twice the activation records); ties go to the
// shape that pads less.
struct MxPlan {
    int64_t main_wgs, piece_wgs, first_piece_tile;
    double time, padded;
    bool operator<=(const MxPlan &o) const { return time < o.time || (time == o.time && padded <= o.padded); }
};
template <class C>
MxPlan mx_plan(int64_t m, int64_t n) {
    using P = MxPieceCfg<C::BM, C::BN, C::A8>;
    const int64_t tm = (m + C::BM - 1) / C::BM, tn = (n + C::BN - 1) / C::BN, tiles = tm * tn;
    const int64_t slots = (int64_t)device_cus() * mx_occupancy<C>();
    const int64_t whole = tiles / slots * slots, left = tiles - whole;
    const double prounds = (double)((left * P::PIECES + slots - 1) / slots) * 1.6 / P::PIECES;
    const bool pieces = left > 0 && prounds < 1.0;
    const double rounds = (double)(whole / slots) + (left == 0 ? 0.0 : pieces ? prounds : 1.0);
    MxPlan p;
    p.main_wgs = pieces ? whole : tiles;
    p.piece_wgs = pieces ? left * P::PIECES : 0;
    p.first_piece_tile = whole;
    p.time = rounds * C::BM * C::BN * (C::TM * C::TN == 4 ? 1.0 : C::A8 ? 1.35 : 1.15);
    p.padded = (double)(tm * C::BM) * (tn * C::BN);
    return p;
}

template <class C>
void launch_mx_cfg(const MxArgs &a, const MxPlan &p, hipStream_t s) {
    gemm_mx_kernel<C><<<(unsigned)(p.main_wgs + p.piece_wgs), C::NT, 0, s>>>(a, p.main_wgs, p.first_piece_tile);
}

// Split K.  A product with fewer 128 x 128 tiles than one round of resident
// workgroups would otherwise run entirely as 32 x 32 pieces (no operand reuse
// across waves, ~1.6x the cost per output).  With a long K, S whole-tile
// workgroups per tile, each over 1/S of the stage pairs, fill the round
// instead; their partial sums are added in ascending split order by a second
// kernel.  Pure function of the sizes, modelled on a 256-CU part with two
// resident workgroups per CU (so the workspace size is one too): S =
// min(round / tiles, pairs of stages / 16), taken when its modelled time is
// under 3/4 of the pieces'.  Returns 1 for no split.
constexpr int64_t kSplitRefSlots = 512;
int64_t mx_k_splits(int64_t m, int64_t n, int64_t k) {
    if (m <= SMALL_M_MAX || k <= 0) return 1;
    const int64_t tiles = (m + 127) / 128 * ((n + 127) / 128);
    if (tiles >= kSplitRefSlots) return 1;
    const int64_t pairs = mx_blocks(k) / 4;
    const int64_t S = std::min(kSplitRefSlots / tiles, pairs / 16);
    if (S < 2) return 1;
    const double t_split = (double)((tiles * S + kSplitRefSlots - 1) / kSplitRefSlots) / S;
    const double t_pieces = (double)((tiles * 16 + kSplitRefSlots - 1) / kSplitRefSlots) * 1.6 / 16;
    return t_split < 0.75 * t_pieces ? S : 1;
}

size_t split_partial_bytes(int64_t m, int64_t n, int64_t k) {
    const int64_t S = mx_k_splits(m, n, k);
    return S > 1 ? (size_t)((S * m * n * 4 + 255) / 256 * 256) : 0;
}

// partial: S x m x n fp32 when mx_k_splits(m, n, k) = S > 1 (checked by the caller)
void launch_mx(const MxArgs &a0, float *partial, hipStream_t s) {
    const int64_t S = mx_k_splits(a0.m, a0.n, a0.k);
    if (S > 1) {
        MxArgs a = a0;
        a.splits = S;
        a.partial = partial;
        const int64_t wgs = (a.m + 127) / 128 * ((a.n + 127) / 128) * S;
        gemm_mx_kernel<Mx128x128><<<(unsigned)wgs, Mx128x128::NT, 0, s>>>(a, wgs, 0);
        small_m_reduce_kernel<<<blocks_for(a.m * a.n, 256), 256, 0, s>>>(partial, S, a.m, a.n, a.y, a.ldy);
        return;
    }
    const MxArgs &a = a0;
    const MxPlan p0 = mx_plan<Mx128x128>(a.m, a.n), p1 = mx_plan<Mx128x64>(a.m, a.n), p2 = mx_plan<Mx64x128>(a.m, a.n);
    if (p0 <= p1 && p0 <= p2) launch_mx_cfg<Mx128x128>(a, p0, s);
    else if (p1 <= p2) launch_mx_cfg<Mx128x64>(a, p1, s);
    else launch_mx_cfg<Mx64x128>(a, p2, s);
}

// int8 activations at m > 16 (act: the two-plane records of act8_operand_kernel):
// whole tiles and pieces as for W4A4, no K split.
void launch_mx_a8(const MxArgs &a, hipStream_t s) {
    const MxPlan p0 = mx_plan<Mx128x128A8>(a.m, a.n), p2 = mx_plan<Mx64x128A8>(a.m, a.n);
    if (p0 <= p2) launch_mx_cfg<Mx128x128A8>(a, p0, s);
    else launch_mx_cfg<Mx64x128A8>(a, p2, s);
}

// Size bounds, so that every launch fits the hardware's grid limits and the
// kernels' 32-bit offsets: rows (m, or routed rows) within 65535 row tiles of
// 32 (the quantisers' grid.y); K and N well past any model's.  A 1-D launch
// must stay below 2^32 threads in all.
constexpr int64_t kMaxGridY = 65535;
constexpr int64_t kMaxRows = kMaxGridY * 32;
constexpr int64_t kMaxK = int64_t{1} << 24;
constexpr int64_t kMaxN = int64_t{1} << 26;
constexpr int64_t kMaxThreads = (int64_t{1} << 32) - 1;
inline bool grid_fits(int64_t threads) { return threads <= kMaxThreads; }
// m rows, n columns, k: inside the bounds above (sizes already known >= 0)
inline bool within_bounds(int64_t m, int64_t n, int64_t k) { return m <= kMaxRows && n <= kMaxN && k <= kMaxK; }
// 128 x 128 output tiles of a dense product: each is at most one 256-thread
// workgroup, plus at most 16 pieces per leftover tile of one round
constexpr int64_t kMaxDenseTiles = int64_t{1} << 20;

w4a4_status check_gemm_common(const void *packed_w, const uint8_t *codes, const float *scales,
                              const float *y, int64_t n, int64_t k) {
    if (n < 0 || k < 0) return W4A4_ERR_INVALID_VALUE;
    if (k % QK) return W4A4_ERR_K_NOT_MULTIPLE_OF_32;
    if (!packed_w || !codes || !scales || !y) return W4A4_ERR_INVALID_VALUE;
    if (!aligned(packed_w, 16) || !aligned(codes, 16) || !aligned(scales, 4) || !aligned(y, 4))
        return W4A4_ERR_MISALIGNED;
    return W4A4_OK;
}

}  // namespace

extern "C" {

const char *w4a4_status_string(w4a4_status s) {
    switch (s) {
    case W4A4_OK: return "W4A4_OK";
    case W4A4_ERR_INVALID_VALUE: return "W4A4_ERR_INVALID_VALUE";
    case W4A4_ERR_K_NOT_MULTIPLE_OF_32: return "W4A4_ERR_K_NOT_MULTIPLE_OF_32";
    case W4A4_ERR_MISALIGNED: return "W4A4_ERR_MISALIGNED";
    case W4A4_ERR_UNSUPPORTED_DTYPE: return "W4A4_ERR_UNSUPPORTED_DTYPE";
    case W4A4_ERR_WORKSPACE_TOO_SMALL: return "W4A4_ERR_WORKSPACE_TOO_SMALL";
    case W4A4_ERR_HIP: return "W4A4_ERR_HIP";
    }
    return "W4A4_ERR_UNKNOWN";
}

const char *w4a4_last_hip_error(void) { return g_last_hip_error; }

size_t w4a4_q4_0_bytes(int64_t n, int64_t k) {
    if (n < 0 || k < 0 || k % QK) return 0;
    return (size_t)(n * (k / QK) * 18);
}

size_t w4a4_packed_weight_bytes(int64_t n, int64_t k) {
    if (n < 0 || k < 0 || k % QK) return 0;
    return (size_t)packed_total_bytes(n, k);
}

namespace {
w4a4_status quantize_q4_0(bool rotate, const float *w, int64_t n, int64_t k, int64_t ldw, void *q4_0, void *stream) {
    if (n < 0 || k < 0 || ldw < k || !within_bounds(0, n, k)) return W4A4_ERR_INVALID_VALUE;
    if (k % QK) return W4A4_ERR_K_NOT_MULTIPLE_OF_32;
    if (n == 0 || k == 0) return W4A4_OK;
    if (!w || !q4_0) return W4A4_ERR_INVALID_VALUE;
    if (!grid_fits(n * (k / QK))) return W4A4_ERR_INVALID_VALUE;
    if (!aligned(w, 4)) return W4A4_ERR_MISALIGNED;
    const int64_t blocks = n * (k / QK);
    uint8_t *q = static_cast<uint8_t *>(q4_0);
    if (rotate) quantize_q4_0_h32_kernel<true><<<blocks_for(blocks, 256), 256, 0, as_stream(stream)>>>(w, n, k, ldw, q);
    else quantize_q4_0_h32_kernel<false><<<blocks_for(blocks, 256), 256, 0, as_stream(stream)>>>(w, n, k, ldw, q);
    return hip_status("quantize_q4_0_h32_kernel");
}
}  // namespace

w4a4_status w4a4_quantize_q4_0_h32(const float *w, int64_t n, int64_t k, int64_t ldw, void *q4_0,
                                   void *stream) {
    return quantize_q4_0(true, w, n, k, ldw, q4_0, stream);
}

w4a4_status w4a4_quantize_q4_0(const float *w, int64_t n, int64_t k, int64_t ldw, void *q4_0, void *stream) {
    return quantize_q4_0(false, w, n, k, ldw, q4_0, stream);
}

w4a4_status w4a4_repack_q4_0_h32(const void *q4_0, void *packed, int64_t n, int64_t k, void *stream) {
    if (n < 0 || k < 0 || !within_bounds(0, n, k)) return W4A4_ERR_INVALID_VALUE;
    if (k % QK) return W4A4_ERR_K_NOT_MULTIPLE_OF_32;
    if (n == 0 || k == 0) return W4A4_OK;
    if (!q4_0 || !packed) return W4A4_ERR_INVALID_VALUE;
    if (!aligned(packed, 16)) return W4A4_ERR_MISALIGNED;
    const int64_t mx_threads = padded_n(n) / TILE_N * mx_blocks(k) * 32;
    if (!grid_fits(mx_threads) || !grid_fits(padded_n(n) / TILE_N * sq_quads(k) * SQ_BLOCKS * 32))
        return W4A4_ERR_INVALID_VALUE;
    repack_mx_kernel<<<blocks_for(mx_threads, 256), 256, 0, as_stream(stream)>>>(
        static_cast<const uint8_t *>(q4_0), n, k, static_cast<uint8_t *>(packed));
    const w4a4_status st2 = hip_status("repack_mx_kernel");
    if (st2 != W4A4_OK) return st2;
    const int64_t sq_threads = padded_n(n) / TILE_N * sq_quads(k) * SQ_BLOCKS * 32;
    repack_sq_kernel<<<blocks_for(sq_threads, 256), 256, 0, as_stream(stream)>>>(
        static_cast<const uint8_t *>(q4_0), n, k, static_cast<uint8_t *>(packed));
    return hip_status("repack_sq_kernel");
}

namespace {
// a8: int8 codes ([m][k] bytes) instead of int4 ([m][k/2]); rotate = false:
// no rotation (the unrotated ablation; int4 only)
// sma: the record-ordered operand of an m <= 16 product (W4A4, rotated;
// instead of `act`)
w4a4_status rotate_quantize(bool a8, const void *x, w4a4_dtype dt, int64_t m, int64_t k, int64_t ldx,
                            uint8_t *codes, float *scales, void *act, size_t act_bytes, void *stream,
                            bool rotate = true, void *sma = nullptr) {
    if (dt != W4A4_DTYPE_F32 && dt != W4A4_DTYPE_F16) return W4A4_ERR_UNSUPPORTED_DTYPE;
    if (m < 0 || k < 0 || ldx < k || !within_bounds(m, 0, k)) return W4A4_ERR_INVALID_VALUE;
    if (k % QK) return W4A4_ERR_K_NOT_MULTIPLE_OF_32;
    if (m == 0 || k == 0) return W4A4_OK;
    if (!x || !codes || !scales) return W4A4_ERR_INVALID_VALUE;
    if (!aligned(x, dt == W4A4_DTYPE_F32 ? 4 : 2) || !aligned(codes, 16) || !aligned(scales, 4))
        return W4A4_ERR_MISALIGNED;
    if (act) {
        if (!rotate) return W4A4_ERR_INVALID_VALUE;
        if (!aligned(act, 256)) return W4A4_ERR_MISALIGNED;
        if (act_bytes < (a8 ? w4a4_act8_operand_bytes(m, k) : w4a4_act_operand_bytes(m, k)))
            return W4A4_ERR_WORKSPACE_TOO_SMALL;
    }
    if (sma) {
        if (a8 || !rotate || act || m > SMALL_M_MAX) return W4A4_ERR_INVALID_VALUE;
        if (!aligned(sma, 256)) return W4A4_ERR_MISALIGNED;
        if (act_bytes < w4a4_small_act_operand_bytes(m, k)) return W4A4_ERR_WORKSPACE_TOO_SMALL;
    }
    const size_t esz = dt == W4A4_DTYPE_F32 ? 4 : 2;
    // vector loads of a block: 16-byte (every block start 16-byte aligned),
    // 4-element (every 4-element group aligned), or none
    const int vec = aligned(x, 16) && (ldx * esz) % 16 == 0 ? 2 : aligned(x, 4 * esz) && (ldx % 4) == 0 ? 1 : 0;
    const int64_t blocks = act ? mx_blocks(k) : sma ? sq_quads(k) * SQ_BLOCKS : k / QK;
    const dim3 grid((unsigned)((blocks + RQ_BLOCKS - 1) / RQ_BLOCKS), (unsigned)((m + 31) / 32));
    hipStream_t s = as_stream(stream);
    uint8_t *a = static_cast<uint8_t *>(act);
    const float *xf = static_cast<const float *>(x);
    const __half *xh = static_cast<const __half *>(x);
    const unsigned nt = 128 * RQ_BLOCKS;
    if (!rotate && dt == W4A4_DTYPE_F32) rotate_quantize_kernel<float, 7, false><<<grid, nt, 0, s>>>(xf, m, k, ldx, vec, codes, scales, a);
    else if (!rotate) rotate_quantize_kernel<__half, 7, false><<<grid, nt, 0, s>>>(xh, m, k, ldx, vec, codes, scales, a);
    else if (dt == W4A4_DTYPE_F32 && a8) rotate_quantize_kernel<float, 127><<<grid, nt, 0, s>>>(xf, m, k, ldx, vec, codes, scales, a);
    else if (dt == W4A4_DTYPE_F32) rotate_quantize_kernel<float, 7><<<grid, nt, 0, s>>>(xf, m, k, ldx, vec, codes, scales, a, static_cast<uint8_t *>(sma));
    else if (a8) rotate_quantize_kernel<__half, 127><<<grid, nt, 0, s>>>(xh, m, k, ldx, vec, codes, scales, a);
    else rotate_quantize_kernel<__half, 7><<<grid, nt, 0, s>>>(xh, m, k, ldx, vec, codes, scales, a, static_cast<uint8_t *>(sma));
    return hip_status("rotate_quantize_kernel");
}
}  // namespace

w4a4_status w4a4_rotate_quantize_act(const void *x, w4a4_dtype dt, int64_t m, int64_t k, int64_t ldx,
                                     uint8_t *codes, float *scales, void *stream) {
    return rotate_quantize(false, x, dt, m, k, ldx, codes, scales, nullptr, 0, stream);
}

w4a4_status w4a4_quantize_act(const void *x, w4a4_dtype dt, int64_t m, int64_t k, int64_t ldx, uint8_t *codes,
                              float *scales, void *stream) {
    return rotate_quantize(false, x, dt, m, k, ldx, codes, scales, nullptr, 0, stream, false);
}

w4a4_status w4a4_rotate_quantize_act8(const void *x, w4a4_dtype dt, int64_t m, int64_t k, int64_t ldx,
                                      int8_t *codes, float *scales, void *stream) {
    return rotate_quantize(true, x, dt, m, k, ldx, reinterpret_cast<uint8_t *>(codes), scales, nullptr, 0, stream);
}

w4a4_status w4a4_rotate_quantize_prepare(const void *x, w4a4_dtype dt, int64_t m, int64_t k, int64_t ldx,
                                         uint8_t *codes, float *scales, void *act, size_t act_bytes,
                                         void *stream) {
    if (!act && m > 0 && k > 0) return W4A4_ERR_INVALID_VALUE;
    return rotate_quantize(false, x, dt, m, k, ldx, codes, scales, act, act_bytes, stream);
}

size_t w4a4_small_act_operand_bytes(int64_t m, int64_t k) {
    if (m < 0 || m > SMALL_M_MAX || k < 0 || k % QK) return 0;
    return (size_t)small_act_bytes(k);
}

w4a4_status w4a4_rotate_quantize_prepare_small(const void *x, w4a4_dtype dt, int64_t m, int64_t k, int64_t ldx,
                                               uint8_t *codes, float *scales, void *act, size_t act_bytes,
                                               void *stream) {
    if (m > SMALL_M_MAX) return W4A4_ERR_INVALID_VALUE;
    if (!act && m > 0 && k > 0) return W4A4_ERR_INVALID_VALUE;
    return rotate_quantize(false, x, dt, m, k, ldx, codes, scales, nullptr, act_bytes, stream, true, act);
}

w4a4_status w4a4_rotate_quantize_prepare8(const void *x, w4a4_dtype dt, int64_t m, int64_t k, int64_t ldx,
                                          int8_t *codes, float *scales, void *act, size_t act_bytes,
                                          void *stream) {
    if (!act && m > 0 && k > 0) return W4A4_ERR_INVALID_VALUE;
    return rotate_quantize(true, x, dt, m, k, ldx, reinterpret_cast<uint8_t *>(codes), scales, act, act_bytes,
                           stream);
}

size_t w4a4_gemm_workspace_bytes(int64_t m, int64_t n, int64_t k) {
    if (m < 0 || n < 0 || k < 0 || k % QK) return 0;
    if (n == 0 || k == 0 || m == 0) return 0;
    if (m <= SMALL_M_MAX) return small_m_workspace_bytes(small_m_plan(n, k), m, n);  // the K splits' sums
    return (w4a4_act_operand_bytes(m, k) + 255) / 256 * 256 + split_partial_bytes(m, n, k);
}

size_t w4a4_gemm_prepared_workspace_bytes(int64_t m, int64_t n, int64_t k) {
    if (m < 0 || n < 0 || k < 0 || k % QK) return 0;
    if (m == 0 || n == 0 || k == 0) return 0;
    return split_partial_bytes(m, n, k);
}

}  // extern "C"

namespace {
// The m <= 16 product (sizes and buffers checked by the caller), from the
// public codes and scales or (act_rec) from the record-ordered operand.
w4a4_status launch_small_m(const void *packed_w, const uint8_t *codes, const float *scales, const void *act_rec,
                           float *y, int64_t m, int64_t n, int64_t k, int64_t ldy, void *workspace,
                           size_t workspace_bytes, hipStream_t s) {
    const SmallPlan plan = small_m_plan(n, k);
    if (plan.splits > 1) {
        if (!workspace) return W4A4_ERR_INVALID_VALUE;
        if (!aligned(workspace, 256)) return W4A4_ERR_MISALIGNED;
        if (workspace_bytes < w4a4_gemm_workspace_bytes(m, n, k)) return W4A4_ERR_WORKSPACE_TOO_SMALL;
    }
    SmallArgs a{};
    a.codes = codes;
    a.scales = scales;
    a.act_rec = static_cast<const uint8_t *>(act_rec);
    a.sq = static_cast<const uint8_t *>(packed_w) + sq_section_offset(n, k);
    a.y = y;
    a.ldy = ldy;
    a.m = m;
    a.n = n;
    a.k = k;
    a.range = plan.range;
    set_small_m_split(a, plan, workspace);
    const unsigned grid = (unsigned)small_m_items(plan);
    const bool rec = act_rec != nullptr;
    if (plan.waves == SM_WAVES_LONG_K && rec)
        gemm_small_m_kernel<SM_WAVES_LONG_K, SM_DEPTH, false, true><<<grid, 64 * SM_WAVES_LONG_K, small_m_lds_bytes(plan), s>>>(a);
    else if (plan.waves == SM_WAVES_LONG_K)
        gemm_small_m_kernel<SM_WAVES_LONG_K, SM_DEPTH><<<grid, 64 * SM_WAVES_LONG_K, small_m_lds_bytes(plan), s>>>(a);
    else if (rec)
        gemm_small_m_kernel<SM_WAVES, SM_DEPTH, false, true><<<grid, 64 * SM_WAVES, small_m_lds_bytes(plan), s>>>(a);
    else
        gemm_small_m_kernel<SM_WAVES, SM_DEPTH><<<grid, 64 * SM_WAVES, small_m_lds_bytes(plan), s>>>(a);
    return hip_status("gemm_small_m_kernel");
}
}  // namespace

extern "C" {

w4a4_status w4a4_gemm_prepared_small(const void *packed_w, const void *act, float *y, int64_t m, int64_t n,
                                     int64_t k, int64_t ldy, void *workspace, size_t workspace_bytes,
                                     void *stream) {
    if (m < 0 || m > SMALL_M_MAX || n < 0 || k < 0 || ldy < n || !within_bounds(m, n, k))
        return W4A4_ERR_INVALID_VALUE;
    if (k % QK) return W4A4_ERR_K_NOT_MULTIPLE_OF_32;
    if (m == 0 || n == 0) return W4A4_OK;
    if (!y) return W4A4_ERR_INVALID_VALUE;
    if (!aligned(y, 4)) return W4A4_ERR_MISALIGNED;
    hipStream_t s = as_stream(stream);
    if (k == 0) {  // empty sum
        launch_zero_rows(y, m, n, ldy, s);
        return hip_status("zero_rows_kernel");
    }
    if (!packed_w || !act) return W4A4_ERR_INVALID_VALUE;
    if (!aligned(packed_w, 16) || !aligned(act, 256)) return W4A4_ERR_MISALIGNED;
    return launch_small_m(packed_w, nullptr, nullptr, act, y, m, n, k, ldy, workspace, workspace_bytes, s);
}

w4a4_status w4a4_gemm(const void *packed_w, const uint8_t *codes, const float *scales, float *y,
                      int64_t m, int64_t n, int64_t k, int64_t ldy, void *workspace, size_t workspace_bytes,
                      void *stream) {
    if (m < 0 || ldy < n) return W4A4_ERR_INVALID_VALUE;
    if (m == 0 || n == 0) {
        if (n < 0 || k < 0) return W4A4_ERR_INVALID_VALUE;
        return k % QK ? W4A4_ERR_K_NOT_MULTIPLE_OF_32 : W4A4_OK;
    }
    if (n < 0 || k < 0 || !within_bounds(m, n, k)) return W4A4_ERR_INVALID_VALUE;
    const w4a4_status st = check_gemm_common(packed_w, codes, scales, y, n, k);
    if (st != W4A4_OK) return st;
    hipStream_t s = as_stream(stream);
    if (k == 0) {  // empty sum
        launch_zero_rows(y, m, n, ldy, s);
        return hip_status("zero_rows_kernel");
    }
    if (m <= SMALL_M_MAX) return launch_small_m(packed_w, codes, scales, nullptr, y, m, n, k, ldy, workspace,
                                                workspace_bytes, s);
    // workspace: the activation operand, then the split-K partial sums
    if (!workspace) return W4A4_ERR_INVALID_VALUE;
    if (!aligned(workspace, 256)) return W4A4_ERR_MISALIGNED;
    if (workspace_bytes < w4a4_gemm_workspace_bytes(m, n, k)) return W4A4_ERR_WORKSPACE_TOO_SMALL;
    const w4a4_status pst = w4a4_gemm_prepare_act(codes, scales, m, k, workspace, workspace_bytes, stream);
    if (pst != W4A4_OK) return pst;
    const size_t act_bytes = (w4a4_act_operand_bytes(m, k) + 255) / 256 * 256;
    return w4a4_gemm_prepared(packed_w, workspace, y, m, n, k, ldy, static_cast<uint8_t *>(workspace) + act_bytes,
                              workspace_bytes - act_bytes, stream);
}

}  // extern "C"

// Scratch of w4a4_gemm_noalloc: a device array of fixed size, one instance per
// GPU (each holds its copy while the library is loaded).  Host code never
// passes this name to a kernel or a copy: it stands for the array only in
// device code, and its device address is looked up per device below.
namespace {
constexpr size_t kNoAllocScratchBytes = size_t{64} << 20;
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
void *g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];
std::once_flag g_scratch_once[kMaxDevices];

// The current device's copy of `scratch`: its address is looked up once per
// device, on that device's first call, with that device current.
w4a4_status current_scratch(void **out) {
    int dev = -1;
    const hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        std::snprintf(g_last_hip_error, sizeof g_last_hip_error, "hipGetDevice: %s",
                      e != hipSuccess ? hipGetErrorString(e) : "device index out of range");
        return W4A4_ERR_HIP;
    }
    std::call_once(g_scratch_once[dev], [dev] {
        void *ptr = nullptr;
        g_scratch_err[dev] = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        g_scratch_ptr[dev] = g_scratch_err[dev] == hipSuccess ? ptr : nullptr;
    });
    if (g_scratch_err[dev] != hipSuccess || !g_scratch_ptr[dev]) {
        std::snprintf(g_last_hip_error, sizeof g_last_hip_error, "hipGetSymbolAddress(scratch): %s",
                      hipGetErrorString(g_scratch_err[dev]));
        return W4A4_ERR_HIP;
    }
    *out = g_scratch_ptr[dev];
    return W4A4_OK;
}
}  // namespace

extern "C" {

size_t w4a4_gemm_noalloc_scratch_bytes(void) { return kNoAllocScratchBytes; }

w4a4_status w4a4_gemm_noalloc(const void *packed_w, const uint8_t *codes, const float *scales, float *y,
                              int64_t m, int64_t n, int64_t k, int64_t ldy, void *stream) {
    // invalid sizes need no workspace: w4a4_gemm then reports them
    const size_t need = w4a4_gemm_workspace_bytes(m, n, k);
    if (need > kNoAllocScratchBytes) return W4A4_ERR_WORKSPACE_TOO_SMALL;
    void *ws = nullptr;
    if (need) {
        const w4a4_status st = current_scratch(&ws);
        if (st != W4A4_OK) return st;
    }
    return w4a4_gemm(packed_w, codes, scales, y, m, n, k, ldy, ws, need, stream);
}

// Fused rotate-quantise + product.  Workspace: m <= 16: 256 bytes of
// synchronisation words and one flag per quad of blocks (zero before the
// first use; every call leaves them ready for the next), then the K splits'
// arrival words and partial sums (as w4a4_gemm's); m > 16: the matrix-core operand, then the split-K partial
// sums (w4a4_gemm's workspace).
namespace {
size_t fused_sync_bytes(int64_t k) { return 256 + up256_bytes(sq_quads(k) * 4); }
}  // namespace

size_t w4a4_rotate_quantize_gemm_workspace_bytes(int64_t m, int64_t n, int64_t k) {
    if (m < 0 || n < 0 || k < 0 || k % QK) return 0;
    if (m == 0 || n == 0 || k == 0) return 0;
    if (m > SMALL_M_MAX) return w4a4_gemm_workspace_bytes(m, n, k);
    return fused_sync_bytes(k) + small_m_workspace_bytes(small_m_plan(n, k), m, n);
}

w4a4_status w4a4_rotate_quantize_gemm(const void *x, w4a4_dtype dt, int64_t m, int64_t k, int64_t ldx,
                                      const void *packed_w, int64_t n, float *y, int64_t ldy, uint8_t *codes,
                                      float *scales, void *workspace, size_t workspace_bytes, void *stream) {
    if (dt != W4A4_DTYPE_F32 && dt != W4A4_DTYPE_F16) return W4A4_ERR_UNSUPPORTED_DTYPE;
    if (m < 0 || n < 0 || k < 0 || ldx < k || ldy < n || !within_bounds(m, n, k)) return W4A4_ERR_INVALID_VALUE;
    if (k % QK) return W4A4_ERR_K_NOT_MULTIPLE_OF_32;
    if (m == 0 || n == 0) return W4A4_OK;
    if (!y) return W4A4_ERR_INVALID_VALUE;
    if (!aligned(y, 4)) return W4A4_ERR_MISALIGNED;
    hipStream_t s = as_stream(stream);
    if (k == 0) {  // empty sums (no codes to write)
        launch_zero_rows(y, m, n, ldy, s);
        return hip_status("zero_rows_kernel");
    }
    if (!x || !packed_w || !codes || !scales) return W4A4_ERR_INVALID_VALUE;
    if (!aligned(x, dt == W4A4_DTYPE_F32 ? 4 : 2) || !aligned(packed_w, 16) || !aligned(codes, 16) ||
        !aligned(scales, 4))
        return W4A4_ERR_MISALIGNED;
    const size_t need = w4a4_rotate_quantize_gemm_workspace_bytes(m, n, k);
    if (!workspace) return W4A4_ERR_INVALID_VALUE;
    if (!aligned(workspace, 256)) return W4A4_ERR_MISALIGNED;
    if (workspace_bytes < need) return W4A4_ERR_WORKSPACE_TOO_SMALL;
    if (m > SMALL_M_MAX) {
        // the quantiser writes the matrix-core operand as well; then the tiled product
        const size_t act_bytes = (w4a4_act_operand_bytes(m, k) + 255) / 256 * 256;
        const w4a4_status st = w4a4_rotate_quantize_prepare(x, dt, m, k, ldx, codes, scales, workspace,
                                                            act_bytes, stream);
        if (st != W4A4_OK) return st;
        return w4a4_gemm_prepared(packed_w, workspace, y, m, n, k, ldy, static_cast<uint8_t *>(workspace) + act_bytes,
                                  workspace_bytes - act_bytes, stream);
    }
    const SmallPlan plan = small_m_plan(n, k);  // the two-launch path's plan: the same sums in the same order
    uint8_t *ws = static_cast<uint8_t *>(workspace);
    const size_t esz = dt == W4A4_DTYPE_F32 ? 4 : 2;
    SmallArgs a{};
    a.codes = codes;
    a.scales = scales;
    a.sq = static_cast<const uint8_t *>(packed_w) + sq_section_offset(n, k);
    a.y = y;
    set_small_m_split(a, plan, ws + fused_sync_bytes(k));
    a.ldy = ldy;
    a.m = m;
    a.n = n;
    a.k = k;
    a.range = plan.range;
    a.x = x;
    a.ldx = ldx;
    a.mode = aligned(x, 16) && (ldx * esz) % 16 == 0 ? 2 : aligned(x, 4 * esz) && (ldx % 4) == 0 ? 1 : 0;
    a.codes_out = codes;
    a.scales_out = scales;
    a.sync = reinterpret_cast<uint32_t *>(ws);
    a.flags = reinterpret_cast<uint32_t *>(ws + 256);
    const int quads = fuse_quads(plan.waves);
    a.producers = (sq_quads(k) + quads - 1) / quads;
    const int64_t consumers = small_m_items(plan);
    const int64_t total = a.producers + consumers;
    if (!grid_fits(total * 64 * plan.waves)) return W4A4_ERR_INVALID_VALUE;
    const unsigned threads = 64 * plan.waves;
    const size_t lds = small_m_lds_bytes(plan);
    if (plan.waves == SM_WAVES_LONG_K && dt == W4A4_DTYPE_F32)
        gemm_small_m_fused_kernel<SM_WAVES_LONG_K, SM_DEPTH, float><<<(unsigned)total, threads, lds, s>>>(a, (uint32_t)total);
    else if (plan.waves == SM_WAVES_LONG_K)
        gemm_small_m_fused_kernel<SM_WAVES_LONG_K, SM_DEPTH, __half><<<(unsigned)total, threads, lds, s>>>(a, (uint32_t)total);
    else if (dt == W4A4_DTYPE_F32)
        gemm_small_m_fused_kernel<SM_WAVES, SM_DEPTH, float><<<(unsigned)total, threads, lds, s>>>(a, (uint32_t)total);
    else
        gemm_small_m_fused_kernel<SM_WAVES, SM_DEPTH, __half><<<(unsigned)total, threads, lds, s>>>(a, (uint32_t)total);
    return hip_status("gemm_small_m_fused_kernel");
}

size_t w4a4_gemm_a8_workspace_bytes(int64_t m, int64_t n, int64_t k) {
    if (m < 0 || n < 0 || k < 0 || k % QK) return 0;
    if (n == 0 || k == 0 || m == 0) return 0;
    if (m > SMALL_M_MAX) return up256_bytes(2 * (int64_t)w4a4_act_operand_bytes(m, k));  // the two-plane records
    return small_m_workspace_bytes(small_m_plan(n, k, true), m, n);  // the K splits' sums
}

w4a4_status w4a4_gemm_a8(const void *packed_w, const int8_t *codes, const float *scales, float *y, int64_t m,
                         int64_t n, int64_t k, int64_t ldy, void *workspace, size_t workspace_bytes,
                         void *stream) {
    if (m < 0 || ldy < n) return W4A4_ERR_INVALID_VALUE;
    if (m == 0 || n == 0) {
        if (n < 0 || k < 0) return W4A4_ERR_INVALID_VALUE;
        return k % QK ? W4A4_ERR_K_NOT_MULTIPLE_OF_32 : W4A4_OK;
    }
    if (n < 0 || k < 0 || !within_bounds(m, n, k)) return W4A4_ERR_INVALID_VALUE;
    const uint8_t *c8 = reinterpret_cast<const uint8_t *>(codes);
    const w4a4_status st = check_gemm_common(packed_w, c8, scales, y, n, k);
    if (st != W4A4_OK) return st;
    hipStream_t s = as_stream(stream);
    if (k == 0) {  // empty sum
        launch_zero_rows(y, m, n, ldy, s);
        return hip_status("zero_rows_kernel");
    }
    if (m <= SMALL_M_MAX) {
        const SmallPlan plan = small_m_plan(n, k, true);
        if (plan.splits > 1) {
            if (!workspace) return W4A4_ERR_INVALID_VALUE;
            if (!aligned(workspace, 256)) return W4A4_ERR_MISALIGNED;
            if (workspace_bytes < w4a4_gemm_a8_workspace_bytes(m, n, k)) return W4A4_ERR_WORKSPACE_TOO_SMALL;
        }
        SmallArgs a{};
        a.codes = c8;
        a.scales = scales;
        a.sq = static_cast<const uint8_t *>(packed_w) + sq_section_offset(n, k);
        a.y = y;
        a.ldy = ldy;
        a.m = m;
        a.n = n;
        a.k = k;
        a.range = plan.range;
        set_small_m_split(a, plan, workspace);
        gemm_small_m_kernel<SM_WAVES, SM_DEPTH, true>
            <<<(unsigned)small_m_items(plan), 64 * SM_WAVES, small_m_lds_bytes(plan), s>>>(a);
        return hip_status("gemm_small_m_kernel<a8>");
    }
    // m > 16: the codes as two FP6 planes, then the matrix-core kernel
    if (!workspace) return W4A4_ERR_INVALID_VALUE;
    if (!aligned(workspace, 256)) return W4A4_ERR_MISALIGNED;
    if (workspace_bytes < w4a4_gemm_a8_workspace_bytes(m, n, k)) return W4A4_ERR_WORKSPACE_TOO_SMALL;
    if ((m + 127) / 128 * ((n + 127) / 128) >= kMaxDenseTiles) return W4A4_ERR_INVALID_VALUE;
    const int64_t rows = (m + 31) / 32 * 32, threads = rows * mx_blocks(k);
    if (!grid_fits(threads)) return W4A4_ERR_INVALID_VALUE;
    act8_operand_kernel<<<blocks_for(threads, 256), 256, 0, s>>>(codes, scales, m, k,
                                                                 static_cast<uint8_t *>(workspace));
    const w4a4_status st2 = hip_status("act8_operand_kernel");
    if (st2 != W4A4_OK) return st2;
    return w4a4_gemm_a8_prepared(packed_w, workspace, y, m, n, k, ldy, stream);
}

size_t w4a4_act8_operand_bytes(int64_t m, int64_t k) {
    if (m < 0 || k < 0 || k % QK) return 0;
    return 2 * w4a4_act_operand_bytes(m, k);
}

w4a4_status w4a4_gemm_a8_prepared(const void *packed_w, const void *act, float *y, int64_t m, int64_t n,
                                  int64_t k, int64_t ldy, void *stream) {
    if (m < 0 || n < 0 || k < 0 || ldy < n || !within_bounds(m, n, k)) return W4A4_ERR_INVALID_VALUE;
    if (k % QK) return W4A4_ERR_K_NOT_MULTIPLE_OF_32;
    if (m == 0 || n == 0) return W4A4_OK;
    if (!y) return W4A4_ERR_INVALID_VALUE;
    if (!aligned(y, 4)) return W4A4_ERR_MISALIGNED;
    if ((m + 127) / 128 * ((n + 127) / 128) >= kMaxDenseTiles) return W4A4_ERR_INVALID_VALUE;
    hipStream_t s = as_stream(stream);
    if (k == 0) {  // empty sum
        launch_zero_rows(y, m, n, ldy, s);
        return hip_status("zero_rows_kernel");
    }
    if (!packed_w || !act) return W4A4_ERR_INVALID_VALUE;
    if (!aligned(packed_w, 16) || !aligned(act, 256)) return W4A4_ERR_MISALIGNED;
    MxArgs a{};
    a.act = static_cast<const uint8_t *>(act);
    a.wrec = static_cast<const uint8_t *>(packed_w);  // the matrix-core section
    a.y = y;
    a.ldy = ldy;
    a.m = m;
    a.n = n;
    a.k = k;
    launch_mx_a8(a, s);
    return hip_status("gemm_mx_kernel<a8>");
}

size_t w4a4_act_operand_bytes(int64_t m, int64_t k) {
    if (m < 0 || k < 0 || k % QK) return 0;
    return (size_t)((m + 31) / 32 * mx_blocks(k) * MX_REC);
}

w4a4_status w4a4_gemm_prepare_act(const uint8_t *codes, const float *scales, int64_t m, int64_t k,
                                  void *act, size_t act_bytes, void *stream) {
    if (m < 0 || k < 0 || !within_bounds(m, 0, k)) return W4A4_ERR_INVALID_VALUE;
    if (k % QK) return W4A4_ERR_K_NOT_MULTIPLE_OF_32;
    if (m == 0 || k == 0) return W4A4_OK;
    if (!codes || !scales || !act) return W4A4_ERR_INVALID_VALUE;
    if (!grid_fits((m + 31) / 32 * 32 * mx_blocks(k))) return W4A4_ERR_INVALID_VALUE;
    if (!aligned(codes, 16) || !aligned(scales, 4) || !aligned(act, 256)) return W4A4_ERR_MISALIGNED;
    if (act_bytes < w4a4_act_operand_bytes(m, k)) return W4A4_ERR_WORKSPACE_TOO_SMALL;
    const int64_t threads = (m + 31) / 32 * 32 * mx_blocks(k);
    act_operand_kernel<<<blocks_for(threads, 256), 256, 0, as_stream(stream)>>>(codes, scales, m, k,
                                                                               static_cast<uint8_t *>(act));
    return hip_status("act_operand_kernel");
}

w4a4_status w4a4_gemm_prepared(const void *packed_w, const void *act, float *y, int64_t m, int64_t n,
                               int64_t k, int64_t ldy, void *workspace, size_t workspace_bytes, void *stream) {
    if (m < 0 || n < 0 || k < 0 || ldy < n || !within_bounds(m, n, k)) return W4A4_ERR_INVALID_VALUE;
    if (k % QK) return W4A4_ERR_K_NOT_MULTIPLE_OF_32;
    if (m == 0 || n == 0) return W4A4_OK;
    if (!y) return W4A4_ERR_INVALID_VALUE;
    if (!aligned(y, 4)) return W4A4_ERR_MISALIGNED;
    if ((m + 127) / 128 * ((n + 127) / 128) >= kMaxDenseTiles) return W4A4_ERR_INVALID_VALUE;
    hipStream_t s = as_stream(stream);
    if (k == 0) {  // empty sum
        launch_zero_rows(y, m, n, ldy, s);
        return hip_status("zero_rows_kernel");
    }
    if (!packed_w || !act) return W4A4_ERR_INVALID_VALUE;
    if (!aligned(packed_w, 16) || !aligned(act, 256)) return W4A4_ERR_MISALIGNED;
    const size_t need = w4a4_gemm_prepared_workspace_bytes(m, n, k);
    if (need) {
        if (!workspace) return W4A4_ERR_INVALID_VALUE;
        if (!aligned(workspace, 256)) return W4A4_ERR_MISALIGNED;
        if (workspace_bytes < need) return W4A4_ERR_WORKSPACE_TOO_SMALL;
    }
    MxArgs a{};
    a.act = static_cast<const uint8_t *>(act);
    a.wrec = static_cast<const uint8_t *>(packed_w);  // the matrix-core section
    a.y = y;
    a.ldy = ldy;
    a.m = m;
    a.n = n;
    a.k = k;
    launch_mx(a, static_cast<float *>(workspace), s);
    return hip_status("gemm_mx_kernel");
}

size_t w4a4_w16_weight_bytes(int64_t n, int64_t k) {
    if (n < 0 || k < 0 || k % QK) return 0;
    return (size_t)w16_operand_bytes(n, k);
}

size_t w4a4_w16_act_bytes(int64_t m, int64_t k) {
    if (m < 0 || k < 0 || k % QK) return 0;
    return (size_t)w16_operand_bytes(m, k);
}

w4a4_status w4a4_dequantize_w16(const void *q4_0, int64_t n, int64_t k, void *w16, size_t w16_bytes,
                                void *stream) {
    if (n < 0 || k < 0 || !within_bounds(0, n, k)) return W4A4_ERR_INVALID_VALUE;
    if (k % QK) return W4A4_ERR_K_NOT_MULTIPLE_OF_32;
    if (n == 0 || k == 0) return W4A4_OK;
    if (!q4_0 || !w16) return W4A4_ERR_INVALID_VALUE;
    if (!grid_fits(padded_n(n) * mx_blocks(k))) return W4A4_ERR_INVALID_VALUE;
    if (!aligned(w16, 16)) return W4A4_ERR_MISALIGNED;
    if (w16_bytes < w4a4_w16_weight_bytes(n, k)) return W4A4_ERR_WORKSPACE_TOO_SMALL;
    const int64_t threads = padded_n(n) * mx_blocks(k);
    dequantize_w16_kernel<<<blocks_for(threads, 256), 256, 0, as_stream(stream)>>>(
        static_cast<const uint8_t *>(q4_0), n, k, static_cast<_Float16 *>(w16));
    return hip_status("dequantize_w16_kernel");
}

w4a4_status w4a4_rotate_act16(const void *x, w4a4_dtype dt, int64_t m, int64_t k, int64_t ldx, void *a16,
                              size_t a16_bytes, void *stream) {
    if (dt != W4A4_DTYPE_F32 && dt != W4A4_DTYPE_F16) return W4A4_ERR_UNSUPPORTED_DTYPE;
    if (m < 0 || k < 0 || ldx < k || !within_bounds(m, 0, k)) return W4A4_ERR_INVALID_VALUE;
    if (k % QK) return W4A4_ERR_K_NOT_MULTIPLE_OF_32;
    if (m == 0 || k == 0) return W4A4_OK;
    if (!x || !a16) return W4A4_ERR_INVALID_VALUE;
    if (!aligned(x, dt == W4A4_DTYPE_F32 ? 4 : 2) || !aligned(a16, 16)) return W4A4_ERR_MISALIGNED;
    if (a16_bytes < w4a4_w16_act_bytes(m, k)) return W4A4_ERR_WORKSPACE_TOO_SMALL;
    const size_t esz = dt == W4A4_DTYPE_F32 ? 4 : 2;
    const int vec = aligned(x, 16) && (ldx * esz) % 16 == 0 ? 2 : aligned(x, 4 * esz) && (ldx % 4) == 0 ? 1 : 0;
    const dim3 grid((unsigned)(mx_blocks(k) / 2), (unsigned)((m + 31) / 32));
    hipStream_t s = as_stream(stream);
    _Float16 *out = static_cast<_Float16 *>(a16);
    if (dt == W4A4_DTYPE_F32)
        rotate_act16_kernel<float><<<grid, 256, 0, s>>>(static_cast<const float *>(x), m, k, ldx, vec, out);
    else
        rotate_act16_kernel<__half><<<grid, 256, 0, s>>>(static_cast<const __half *>(x), m, k, ldx, vec, out);
    return hip_status("rotate_act16_kernel");
}

w4a4_status w4a4_gemm_w16(const void *w16, const void *a16, float *y, int64_t m, int64_t n, int64_t k,
                          int64_t ldy, void *stream) {
    if (m < 0 || n < 0 || k < 0 || ldy < n || !within_bounds(m, n, k)) return W4A4_ERR_INVALID_VALUE;
    if (k % QK) return W4A4_ERR_K_NOT_MULTIPLE_OF_32;
    if (m == 0 || n == 0) return W4A4_OK;
    if (!y) return W4A4_ERR_INVALID_VALUE;
    if (!aligned(y, 4)) return W4A4_ERR_MISALIGNED;
    hipStream_t s = as_stream(stream);
    if (k == 0) {  // empty sum
        launch_zero_rows(y, m, n, ldy, s);
        return hip_status("zero_rows_kernel");
    }
    if (!w16 || !a16) return W4A4_ERR_INVALID_VALUE;
    if (!aligned(w16, 16) || !aligned(a16, 16)) return W4A4_ERR_MISALIGNED;
    const int64_t tiles = (m + 127) / 128 * ((n + 127) / 128);
    if (tiles >= (int64_t{1} << 20)) return W4A4_ERR_INVALID_VALUE;  // grid of < 2^32 threads, pieces included
    W16Args a{};
    a.a16 = static_cast<const _Float16 *>(a16);
    a.w16 = static_cast<const _Float16 *>(w16);
    a.y = y;
    a.ldy = ldy;
    a.m = m;
    a.n = n;
    a.k = k;
    // whole rounds of resident workgroups take whole tiles; a partial last
    // round is split into pieces when one round of pieces (~1.6x the work
    // per output) is shorter than a round of whole tiles
    static const int occ = [] {
        int o = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&o, gemm_w16_kernel, 256, 0) != hipSuccess || o < 1) o = 1;
        return o;
    }();
    const int64_t slots = (int64_t)device_cus() * occ;
    const int64_t whole = tiles / slots * slots, left = tiles - whole;
    const double prounds = (double)((left * W16_PIECES + slots - 1) / slots) * 1.6 / W16_PIECES;
    const bool pieces = left > 0 && prounds < 1.0;
    const int64_t main_wgs = pieces ? whole : tiles, piece_wgs = pieces ? left * W16_PIECES : 0;
    gemm_w16_kernel<<<(unsigned)(main_wgs + piece_wgs), 256, 0, s>>>(a, main_wgs, whole);
    return hip_status("gemm_w16_kernel");
}

namespace {
// Routing bound: every expert adds at most one partial tile to the full ones.
int64_t grouped_row_tiles(int64_t n_expert, int64_t n_rows, int64_t tile_rows) {
    return (n_rows + tile_rows - 1) / tile_rows + n_expert;
}
size_t up256(int64_t b) { return (size_t)((b + 255) / 256 * 256); }
}  // namespace

size_t w4a4_gemm_id_workspace_bytes(int64_t n_expert, int64_t n_tokens, int64_t top_k) {
    if (n_expert < 0 || n_tokens < 0 || top_k < 0) return 0;
    return 2 * up256((n_expert + 1) * 4) + up256(n_tokens * top_k * 4);
}

w4a4_status w4a4_gemm_id_route(const int32_t *ids, int64_t n_expert, int64_t n_tokens, int64_t top_k,
                               void *workspace, size_t workspace_bytes, void *stream) {
    if (n_tokens < 0 || top_k < 0 || n_expert < 0) return W4A4_ERR_INVALID_VALUE;
    if (n_tokens == 0 || top_k == 0) return W4A4_OK;
    if (n_expert < 1 || n_expert > ROUTE_MAX_EXPERTS) return W4A4_ERR_INVALID_VALUE;
    const int64_t n_rows = n_tokens * top_k;
    if (n_rows > kMaxRows) return W4A4_ERR_INVALID_VALUE;
    if (!ids || !workspace) return W4A4_ERR_INVALID_VALUE;
    if (!aligned(ids, 4) || !aligned(workspace, 256)) return W4A4_ERR_MISALIGNED;
    if (workspace_bytes < w4a4_gemm_id_workspace_bytes(n_expert, n_tokens, top_k))
        return W4A4_ERR_WORKSPACE_TOO_SMALL;
    uint8_t *ws = static_cast<uint8_t *>(workspace);
    route_kernel<<<1, ROUTE_THREADS, 0, as_stream(stream)>>>(
        ids, (int)n_rows, (int)n_expert, GS_ROWS, reinterpret_cast<int32_t *>(ws),
        reinterpret_cast<int32_t *>(ws + up256((n_expert + 1) * 4)),
        reinterpret_cast<int32_t *>(ws + 2 * up256((n_expert + 1) * 4)));
    return hip_status("route_kernel");
}

w4a4_status w4a4_gemm_id_routed(const void *packed_w, int64_t n_expert, const uint8_t *codes,
                                const float *scales, int64_t act_rows_per_token, int64_t n_tokens, int64_t top_k,
                                float *y, int64_t n, int64_t k, const void *workspace, size_t workspace_bytes,
                                void *stream) {
    if (n_tokens < 0 || top_k < 0 || n_expert < 0 || n < 0 || k < 0) return W4A4_ERR_INVALID_VALUE;
    if (k % QK) return W4A4_ERR_K_NOT_MULTIPLE_OF_32;
    if (n_tokens == 0 || top_k == 0 || n == 0) return W4A4_OK;
    if (n_expert < 1 || n_expert > ROUTE_MAX_EXPERTS) return W4A4_ERR_INVALID_VALUE;
    if (act_rows_per_token != 1 && act_rows_per_token != top_k) return W4A4_ERR_INVALID_VALUE;
    const int64_t n_rows = n_tokens * top_k;
    const int64_t row_tiles = grouped_row_tiles(n_expert, n_rows, GS_ROWS);
    const int64_t col_chunks = grouped_col_chunks(n, k);
    if (!within_bounds(n_rows, n, k) || !grid_fits((row_tiles * col_chunks + 8) * 64 * GS_WAVES))
        return W4A4_ERR_INVALID_VALUE;
    if (!workspace) return W4A4_ERR_INVALID_VALUE;
    if (k > 0) {
        const w4a4_status st = check_gemm_common(packed_w, codes, scales, y, n, k);
        if (st != W4A4_OK) return st;
    } else if (!y) {
        return W4A4_ERR_INVALID_VALUE;
    }
    if (!aligned(workspace, 256) || !aligned(y, 4)) return W4A4_ERR_MISALIGNED;
    if (workspace_bytes < w4a4_gemm_id_workspace_bytes(n_expert, n_tokens, top_k))
        return W4A4_ERR_WORKSPACE_TOO_SMALL;

    hipStream_t s = as_stream(stream);
    if (k == 0) {  // empty sums: every row is zero
        launch_zero_rows(y, n_rows, n, n, s);
        return hip_status("zero_rows_kernel");
    }
    const uint8_t *ws = static_cast<const uint8_t *>(workspace);
    GsArgs a{};
    a.codes = codes;
    a.scales = scales;
    a.packed = static_cast<const uint8_t *>(packed_w);
    a.expert_bytes = packed_total_bytes(n, k);
    a.y = y;
    a.ldy = n;
    a.n = n;
    a.k = k;
    a.g = Routing{reinterpret_cast<const int32_t *>(ws + 2 * up256((n_expert + 1) * 4)),
                  reinterpret_cast<const int32_t *>(ws), reinterpret_cast<const int32_t *>(ws + up256((n_expert + 1) * 4)),
                  (int)n_expert};
    a.top_k = (int)top_k;
    a.per_slot = act_rows_per_token != 1 ? 1 : 0;
    a.n_rows = n_rows;
    a.col_chunks = col_chunks;
    a.tiles_per_wave = grouped_tiles_per_wave(n, k);
    // a bound on the items (row tiles x column chunks), rounded up to whole XCD rows
    gemm_grouped_stream_kernel<<<(unsigned)((row_tiles * col_chunks + 7) / 8 * 8), 64 * GS_WAVES, 0, s>>>(a);
    return hip_status("gemm_grouped_stream_kernel");
}

w4a4_status w4a4_gemm_id(const void *packed_w, int64_t n_expert, const uint8_t *codes, const float *scales,
                         int64_t act_rows_per_token, const int32_t *ids, int64_t n_tokens, int64_t top_k,
                         float *y, int64_t n, int64_t k, void *workspace, size_t workspace_bytes,
                         void *stream) {
    if (n_tokens < 0 || top_k < 0 || n_expert < 0 || n < 0 || k < 0) return W4A4_ERR_INVALID_VALUE;
    if (k % QK) return W4A4_ERR_K_NOT_MULTIPLE_OF_32;
    if (n_tokens == 0 || top_k == 0 || n == 0) return W4A4_OK;
    if (!ids) return W4A4_ERR_INVALID_VALUE;
    // validate everything before the first launch
    if (n_expert < 1 || n_expert > ROUTE_MAX_EXPERTS) return W4A4_ERR_INVALID_VALUE;
    if (act_rows_per_token != 1 && act_rows_per_token != top_k) return W4A4_ERR_INVALID_VALUE;
    const int64_t n_rows = n_tokens * top_k;
    const int64_t row_tiles = grouped_row_tiles(n_expert, n_rows, GS_ROWS);
    const int64_t col_chunks = grouped_col_chunks(n, k);
    if (!within_bounds(n_rows, n, k) || !grid_fits((row_tiles * col_chunks + 8) * 64 * GS_WAVES))
        return W4A4_ERR_INVALID_VALUE;
    if (!workspace) return W4A4_ERR_INVALID_VALUE;
    if (k > 0) {
        const w4a4_status st = check_gemm_common(packed_w, codes, scales, y, n, k);
        if (st != W4A4_OK) return st;
    } else if (!y) {
        return W4A4_ERR_INVALID_VALUE;
    }
    if (!aligned(ids, 4) || !aligned(workspace, 256) || !aligned(y, 4)) return W4A4_ERR_MISALIGNED;
    if (workspace_bytes < w4a4_gemm_id_workspace_bytes(n_expert, n_tokens, top_k))
        return W4A4_ERR_WORKSPACE_TOO_SMALL;
    if (k > 0) {
        const w4a4_status rst = w4a4_gemm_id_route(ids, n_expert, n_tokens, top_k, workspace, workspace_bytes, stream);
        if (rst != W4A4_OK) return rst;
    }
    return w4a4_gemm_id_routed(packed_w, n_expert, codes, scales, act_rows_per_token, n_tokens, top_k, y, n, k,
                               workspace, workspace_bytes, stream);
}

}  // extern "C"
