/*
 * w4a4.h -- C ABI of libw4a4.so: the Hadamard-rotated W4A4 Q4_0 matmul on
 * AMD Instinct MI355X (gfx950).
 *
 * The method (1bit-MONSTER engine docs, page "The lean option: ROCmFP4,
 * ROCmI4 and Hadamard Q4_0", section "Hadamard-rotated Q4_0: W4A4 prompt
 * processing"): weights are plain Q4_0 (blocks of 32, one fp16 scale, a code q
 * stands for q - 8), rotated once by a normalised 32-point Walsh-Hadamard
 * transform per 32-element block along K.  At run time every activation row is
 * rotated by the same transform per block and rounded to 4 bits; the 4-bit
 * activation codes are multiplied with the 4-bit weight codes in integer
 * arithmetic and each block's integer dot is scaled into an fp32 accumulator.
 * Section "MoE: W4A4 on the experts" of the same page: the expert matmuls
 * (MUL_MAT_ID) take the same path.
 *
 * Conventions for every call:
 *   - Pointers are device pointers unless stated otherwise.  The caller owns
 *     every buffer; the library keeps no per-call state, never allocates,
 *     frees or synchronises, and never writes its inputs.
 *   - `stream` is a hipStream_t (NULL for the null stream).  Work is enqueued
 *     on it and returns immediately; results are ready when the stream is.
 *   - Arguments are validated on the host before anything is launched; a
 *     failed check returns its status and touches no device memory.  m == 0
 *     (or n == 0, n_tokens == 0) returns W4A4_OK without a launch.
 *   - A failed launch returns W4A4_ERR_HIP (detail: w4a4_last_hip_error()).
 *     Faults during execution surface at the caller's next synchronisation.
 *   - No C++ exception crosses this interface.
 *   - K must be a multiple of 32 (one Q4_0 block).  Any m, n >= 1 works up
 *     to these bounds (larger sizes return W4A4_ERR_INVALID_VALUE before any
 *     launch): m, and the routed rows n_tokens * top_k, at most 65535 * 32 =
 *     2097120 (row tiles of 32 within the 65535 grid rows of the row-tiled
 *     kernels); n at most 2^26; k at most 2^24; and sizes whose one-dimensional
 *     launch would reach 2^32 threads (for a dense product m > 16: 2^20 or
 *     more output tiles of 128 x 128; for weight preparation: n * k / 32 of
 *     2^32 or more) are refused.
 */
#ifndef W4A4_H
#define W4A4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    W4A4_OK = 0,
    W4A4_ERR_INVALID_VALUE = 1,        /* null pointer with work to do, negative size, bad stride or enum */
    W4A4_ERR_K_NOT_MULTIPLE_OF_32 = 2, /* k % 32 != 0 */
    W4A4_ERR_MISALIGNED = 3,           /* a pointer below its required alignment */
    W4A4_ERR_UNSUPPORTED_DTYPE = 4,    /* activation dtype not in w4a4_dtype */
    W4A4_ERR_WORKSPACE_TOO_SMALL = 5,  /* a buffer's byte count below what its size query names */
    W4A4_ERR_HIP = 6                   /* a HIP runtime call failed */
} w4a4_status;

typedef enum { W4A4_DTYPE_F32 = 0, W4A4_DTYPE_F16 = 1 } w4a4_dtype;

/* Human-readable name of a status.  Host only; never NULL. */
const char *w4a4_status_string(w4a4_status s);

/* Detail of the last W4A4_ERR_HIP on the calling thread ("" if none).  Host only. */
const char *w4a4_last_hip_error(void);

/* Bytes of a Q4_0 matrix [n][k/32] x 18-byte blocks.  Host only, pure. */
size_t w4a4_q4_0_bytes(int64_t n, int64_t k);

/*
 * Offline weight preparation (the step the page's tools/hadamard_q4_0.py does
 * on a model file): rotate each 32-block of each row of an fp32 weight matrix
 * by H/sqrt(32) and quantise the result to Q4_0.
 *   w     fp32 [n][ldw], ldw >= k (elements); 4-byte aligned.
 *   q4_0  out, [n][k/32] blocks of 18 bytes: fp16 scale d (little endian)
 *         then 16 bytes, byte j = code of element j (low nibble) | code of
 *         element j+16 (high nibble) << 4; codes 0..15 stand for q - 8.
 * Arithmetic: per element, the sum over j of +-w_j in fp64 in ascending j,
 * times fp64(1/sqrt(32)), rounded to fp32; then d = mx / -8 with mx the
 * element of largest magnitude (first on ties), q = min(15, trunc(w/d' +
 * 8.5)) with w/d' formed as w * (1/d) in fp32, d stored as fp16 (nearest even).
 */
w4a4_status w4a4_quantize_q4_0_h32(const float *w, int64_t n, int64_t k, int64_t ldw,
                                   void *q4_0, void *stream);

/* Bytes of the packed weight buffer w4a4_repack_q4_0_h32 writes.  Host only, pure. */
size_t w4a4_packed_weight_bytes(int64_t n, int64_t k);

/*
 * One-time, lossless re-layout of H32-rotated Q4_0 weights for the GEMMs.
 *   q4_0    [n][k/32] x 18 B, as above (any alignment).  The `_h32` in the
 *           name is the caller's assertion that the weights were rotated:
 *           unrotated weights give silently wrong products.
 *   packed  out, w4a4_packed_weight_bytes(n, k) bytes, 16-byte aligned.  Its
 *           layout is private to this library.  It holds the weights twice,
 *           losslessly, once per kind of reader: the matrix-core operand of
 *           the m > 16 kernel (each q - 8 as an FP6 E2M3 code, 64 times the
 *           scale as an exact pair of bf16 parts; 1 KB per 32 columns and
 *           block), then the 4-bit codes stored as q ^ 8 (read as a signed
 *           nibble that is exactly q - 8, the page's identity) with the fp16
 *           scales, in 2304-byte records of 32 columns x 4 blocks, streamed
 *           by the m <= 16 kernel and by the MUL_MAT_ID kernel.
 * Errors: negative sizes or sizes past the bounds -> W4A4_ERR_INVALID_VALUE;
 * k % 32 -> W4A4_ERR_K_NOT_MULTIPLE_OF_32; null pointers with work to do ->
 * W4A4_ERR_INVALID_VALUE; packed below 16-byte alignment -> W4A4_ERR_MISALIGNED.
 */
w4a4_status w4a4_repack_q4_0_h32(const void *q4_0, void *packed, int64_t n, int64_t k,
                                 void *stream);

/*
 * Rotate and quantise activations, one 32-element block at a time (section
 * "Hadamard-rotated Q4_0: W4A4 prompt processing": each activation row gets
 * the weights' per-block rotation at run time and is then rounded to 4 bits;
 * the page prints no rounding rule, this is the reading taken):
 * unnormalised fast Walsh-Hadamard butterflies in fp32 (stages 1, 2, 4, 8,
 * 16), amax = max |v|, d = amax / 7, codes = clamp(round-half-away(v *
 * (1/d)), -7, 7), stored scale s = d * fp32(1/sqrt(32)).  A block with d below
 * FLT_MIN stores zero codes and s = 0.
 *   x       [m][ldx] fp32 or fp16 (dt), ldx >= k; 4-byte (fp32) or 2-byte
 *           (fp16) aligned.  Non-finite values are outside the contract.
 *   codes   out, [m][k/2] bytes, 16-byte aligned: byte 16b + j holds the
 *           code of element 32b + j in its low nibble and of element
 *           32b + j + 16 in its high nibble, two's complement.
 *   scales  out, [m][k/32] fp32, 4-byte aligned.
 * Errors: dt not a w4a4_dtype -> W4A4_ERR_UNSUPPORTED_DTYPE; negative sizes,
 * ldx < k or sizes past the bounds -> W4A4_ERR_INVALID_VALUE; k % 32 ->
 * W4A4_ERR_K_NOT_MULTIPLE_OF_32; null pointers with work to do ->
 * W4A4_ERR_INVALID_VALUE; misalignment -> W4A4_ERR_MISALIGNED.
 */
w4a4_status w4a4_rotate_quantize_act(const void *x, w4a4_dtype dt, int64_t m, int64_t k,
                                     int64_t ldx, uint8_t *codes, float *scales, void *stream);

/* Workspace bytes w4a4_gemm needs for these sizes (0 when none is needed or
 * an argument is invalid).  Host only, pure. */
size_t w4a4_gemm_workspace_bytes(int64_t m, int64_t n, int64_t k);

/* Bytes of the matrix-core operand of m activation rows of width k (0 for
 * invalid sizes).  Host only, pure. */
size_t w4a4_act_operand_bytes(int64_t m, int64_t k);

/*
 * w4a4_rotate_quantize_act, and in the same pass the matrix-core operand of
 * the rows (what w4a4_gemm_prepare_act would make of codes and scales):
 *   act   out, w4a4_act_operand_bytes(m, k) bytes, 256-byte aligned, for
 *         w4a4_gemm_prepared.  Other arguments as w4a4_rotate_quantize_act.
 */
w4a4_status w4a4_rotate_quantize_prepare(const void *x, w4a4_dtype dt, int64_t m, int64_t k,
                                         int64_t ldx, uint8_t *codes, float *scales, void *act,
                                         size_t act_bytes, void *stream);

/*
 * Dense W4A4 product (section "Hadamard-rotated Q4_0: W4A4 prompt
 * processing": the 4-bit weight and activation codes are multiplied in
 * integer arithmetic and each block's dot is scaled into fp32):
 * y[i][j] = sum_b d_w[j][b] * s[i][b] * S[i][j][b], where S = sum_t (q_w - 8)
 * * q_a is the exact integer dot of block b, accumulated in fp32 (block order
 * ascending within a thread; the scale product d_w * s is formed to within
 * 2^-16 relative for m > 16, exactly for m <= 16).
 *   packed_w  from w4a4_repack_q4_0_h32(n, k), 16-byte aligned.
 *   codes, scales  from w4a4_rotate_quantize_act (m rows).
 *   y         out, [m][ldy] fp32, ldy >= n, 4-byte aligned.
 *   workspace device scratch of w4a4_gemm_workspace_bytes(m, n, k) bytes,
 *             256-byte aligned (may be NULL when that is 0); it needs no
 *             clearing: whatever it holds on entry is overwritten or, for
 *             the arrival words below, recognised as stale by its ticket.
 *             Calls that share a workspace must not overlap.
 * m <= 16 takes a weight-streaming kernel on the 4-bit records, one launch.
 * Products with few 32-column tiles or long K split K over workgroups; the
 * workspace then holds one 8-byte arrival word per 32-column tile (rounded
 * up to 256 bytes), then the splits' partial sums.  An arrival word counts
 * the tile's workgroups in a form tagged with a 48-bit ticket that the
 * library draws per call, so stale contents pass for a count of this call
 * only by a 2^-48 chance; the last workgroup of a tile to arrive adds the
 * tile's splits in ascending split order and leaves the word at zero, so
 * later calls and replays of a captured launch start from a clean word.
 * Larger m first re-lays the activation codes and
 * scales into the matrix-core operand format at the start of the workspace
 * (w4a4_act_operand_bytes rounded up to 256), then runs the tiled
 * matrix-core kernel with the rest of the workspace as its own
 * (w4a4_gemm_prepared).
 */
w4a4_status w4a4_gemm(const void *packed_w, const uint8_t *codes, const float *scales, float *y,
                      int64_t m, int64_t n, int64_t k, int64_t ldy, void *workspace,
                      size_t workspace_bytes, void *stream);

/*
 * Rotate-quantise fused with the product (section "Hadamard-rotated Q4_0: W4A4
 * prompt processing": the activations are rotated and rounded to 4 bits just
 * before the integer product; here both happen in one launch for m <= 16).
 * Computes what w4a4_rotate_quantize_act followed by w4a4_gemm computes, with
 * the same codes, scales and outputs:
 *   x, dt, m, k, ldx   the activations, as w4a4_rotate_quantize_act.
 *   packed_w, n        as w4a4_gemm; y [m][ldy] fp32 out, ldy >= n.
 *   codes, scales      out, as w4a4_rotate_quantize_act writes them (other
 *                      products that read the same rows can reuse them).
 *   workspace          w4a4_rotate_quantize_gemm_workspace_bytes(m, n, k)
 *                      bytes, 256-byte aligned.  For m <= 16 its first
 *                      256 + 4 * ceil(k / 128) bytes (rounded up to 256) hold
 *                      synchronisation words and must be zero before the
 *                      workspace's first use; every call leaves them ready
 *                      for the next, so one workspace serves any sequence of
 *                      calls (and HIP graph replays) on one stream.  Calls that
 *                      share a workspace must not overlap.
 * m <= 16: one launch: its first workgroups rotate and quantise the rows
 * (each block once) and publish them block group by block group; the
 * weight-streaming workgroups of the product wait for the groups of their K
 * range (a bounded wait; the fourth workspace word counts waits that ran
 * out, which in-order dispatch of the workgroups rules out).  A K split adds
 * its splits in the same launch, as w4a4_gemm does.  m > 16: the quantiser (writing
 * the matrix-core operand too) and the tiled product, two launches: the tiled
 * product reads each row tile once per 128 output columns, so quantising in
 * its prologue would repeat the work that many times.
 * Errors: as w4a4_rotate_quantize_act and w4a4_gemm.
 */
size_t w4a4_rotate_quantize_gemm_workspace_bytes(int64_t m, int64_t n, int64_t k);
w4a4_status w4a4_rotate_quantize_gemm(const void *x, w4a4_dtype dt, int64_t m, int64_t k, int64_t ldx,
                                      const void *packed_w, int64_t n, float *y, int64_t ldy, uint8_t *codes,
                                      float *scales, void *workspace, size_t workspace_bytes, void *stream);

/*
 * w4a4_gemm for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same product and the same kernels, with the workspace taken from a
 * fixed-size array that the library holds on each GPU it runs on (allocated
 * when the library's code object is loaded, kept until the process ends;
 * nothing is allocated or freed per call).
 *   Arguments, results and errors as w4a4_gemm, without the workspace.
 *   Sizes whose w4a4_gemm_workspace_bytes(m, n, k) exceeds
 *   w4a4_gemm_noalloc_scratch_bytes() (64 MiB) return
 *   W4A4_ERR_WORKSPACE_TOO_SMALL before any launch.
 *   Every call on one GPU shares that GPU's array, which keeps the last
 *   call's contents (no kernel needs it cleared: every byte read is written
 *   first in the same call, except the arrival words of an m <= 16 K split,
 *   which each call leaves at zero and which carry a per-call ticket).  Calls that overlap on one GPU (several streams
 *   or threads) race on it: serialise them.  The array's device address is
 *   looked up on the first call on each device, with that device current;
 *   a failed lookup returns W4A4_ERR_HIP.
 */
size_t w4a4_gemm_noalloc_scratch_bytes(void);
w4a4_status w4a4_gemm_noalloc(const void *packed_w, const uint8_t *codes, const float *scales, float *y,
                              int64_t m, int64_t n, int64_t k, int64_t ldy, void *stream);

/*
 * The two steps of w4a4_gemm for m > 16, callable on their own (one prepared
 * activation can feed several products that read the same rows, e.g. the
 * query, key and value projections).
 *
 * w4a4_gemm_prepare_act: re-lays activation codes and scales from
 * w4a4_rotate_quantize_act into the matrix-core operand format (every code
 * as an FP6 E2M3 value, exactly q / 8; every scale as two bf16 parts whose
 * sum is the scale to within 2^-16 relative).
 *   act   out, w4a4_act_operand_bytes(m, k) bytes, 256-byte aligned; private
 *         layout.
 *
 * w4a4_gemm_prepared: the product of packed_w with a prepared activation, as
 * w4a4_gemm (any m >= 1; y [m][ldy] fp32).  A product with fewer 128 x 128
 * output tiles than one round of resident workgroups and a long K splits K
 * over whole tiles: then workspace holds w4a4_gemm_prepared_workspace_bytes
 * (m, n, k) bytes of partial sums (256-byte aligned; contents on entry
 * ignored; calls sharing it must not overlap), added in ascending split
 * order by a second kernel.  workspace may be NULL when that size is 0
 * (for instance any m <= 16, or more tiles than one round).
 *
 * w4a4_gemm_prepared_workspace_bytes: 0 when no split (or invalid sizes),
 * else splits * m * n * 4 rounded up to 256.  Host only, pure: the split
 * count is a function of the sizes alone.
 */
w4a4_status w4a4_gemm_prepare_act(const uint8_t *codes, const float *scales, int64_t m, int64_t k,
                                  void *act, size_t act_bytes, void *stream);
size_t w4a4_gemm_prepared_workspace_bytes(int64_t m, int64_t n, int64_t k);
w4a4_status w4a4_gemm_prepared(const void *packed_w, const void *act, float *y, int64_t m, int64_t n,
                               int64_t k, int64_t ldy, void *workspace, size_t workspace_bytes,
                               void *stream);

/*
 * The same two steps for m <= 16 (a speculative-verify-sized batch), where
 * the product streams the weights once and each wave reads the activations
 * of every 4-block group of K it computes: the quantiser also writes the
 * codes and scales in the order the waves load them, so those loads are
 * contiguous (section "Hadamard-rotated Q4_0: W4A4 prompt processing": the
 * rotated activations rounded to 4 bits per block, with one scale each).
 *
 * w4a4_small_act_operand_bytes: bytes of that operand for m <= 16 rows and
 * width k: 1280 per group of 4 blocks, g = ceil(k / 128) groups (0 for
 * m > 16 or invalid sizes).  Host only, pure.
 *
 * w4a4_rotate_quantize_prepare_small: w4a4_rotate_quantize_act for m <= 16
 * (m > 16: W4A4_ERR_INVALID_VALUE) that also writes
 *   act   out, w4a4_small_act_operand_bytes(m, k) bytes, 256-byte aligned:
 *         for group q of 4 blocks, row r's 16 code bytes of block 4 q + j
 *         at 1024 q + 64 r + 16 j, and its fp32 scale at 1024 g + 256 q +
 *         16 r + 4 j; rows m .. 15 and blocks past k / 32 are zero.
 * codes and scales are written as by w4a4_rotate_quantize_act, bit for bit.
 *
 * w4a4_gemm_prepared_small: the m <= 16 product of packed_w with such an
 * operand (m > 16: W4A4_ERR_INVALID_VALUE); y, workspace and its size query
 * (w4a4_gemm_workspace_bytes) as for w4a4_gemm with m <= 16, and the result
 * is w4a4_gemm's on the same codes and scales, bit for bit (the same block
 * dots, scale products and summation order).
 */
size_t w4a4_small_act_operand_bytes(int64_t m, int64_t k);
w4a4_status w4a4_rotate_quantize_prepare_small(const void *x, w4a4_dtype dt, int64_t m, int64_t k,
                                               int64_t ldx, uint8_t *codes, float *scales, void *act,
                                               size_t act_bytes, void *stream);
w4a4_status w4a4_gemm_prepared_small(const void *packed_w, const void *act, float *y, int64_t m,
                                     int64_t n, int64_t k, int64_t ldy, void *workspace,
                                     size_t workspace_bytes, void *stream);

/*
 * W4A8-H32: the exact int8 path for a rotated file (section "Hadamard-rotated
 * Q4_0: W4A4 prompt processing" names it as the alternative to W4A4 for the
 * same file).  The activations get the same rotation and are rounded to 8
 * bits per block instead of 4; the weights are the same packed buffer.
 *
 * w4a4_rotate_quantize_act8: as w4a4_rotate_quantize_act, but d = amax / 127
 * and codes clamp(round-half-away(v * (1/d)), -127, 127).
 *   codes   out, [m][k] int8 (one signed byte per element, element order),
 *           16-byte aligned.
 *   scales  out, [m][k/32] fp32, s = d * fp32(1/sqrt(32)).
 *
 * w4a4_gemm_a8: y = sum_b d_w * s * S with S the exact integer dot of the
 * Q4_0 codes (q - 8) with the int8 codes.  Arguments as w4a4_gemm, with the
 * workspace of w4a4_gemm_a8_workspace_bytes (256-byte aligned, needs no
 * clearing; may be NULL when 0): for m <= 16 non-zero only when K is split
 * (arrival words and partial sums as in w4a4_gemm); for m > 16 the codes
 * re-laid as two planes of FP6 matrix-core records (every code a = 16 h + l,
 * h = (a + 8) >> 4 and l both exact in FP6), 2 * w4a4_act_operand_bytes(m, k)
 * rounded up to 256.  m <= 16 streams the weights as w4a4_gemm does; larger
 * m runs the FP6 matrix-core kernel with two block dots per block (the h
 * plane's scaled by 2^4 through the instruction's block scale, the l plane's
 * accumulated on it), so S is exact.
 */
w4a4_status w4a4_rotate_quantize_act8(const void *x, w4a4_dtype dt, int64_t m, int64_t k, int64_t ldx,
                                      int8_t *codes, float *scales, void *stream);
size_t w4a4_gemm_a8_workspace_bytes(int64_t m, int64_t n, int64_t k);
w4a4_status w4a4_gemm_a8(const void *packed_w, const int8_t *codes, const float *scales, float *y,
                         int64_t m, int64_t n, int64_t k, int64_t ldy, void *workspace,
                         size_t workspace_bytes, void *stream);

/*
 * The W4A8 product in two steps, as w4a4_rotate_quantize_prepare and
 * w4a4_gemm_prepared are for W4A4 (same section of the pages):
 *
 * w4a4_act8_operand_bytes: bytes of the int8 matrix-core operand of m rows of
 *   width k, 2 * w4a4_act_operand_bytes(m, k) (0 for invalid sizes).  Host
 *   only, pure.
 * w4a4_rotate_quantize_prepare8: w4a4_rotate_quantize_act8, and in the same
 *   pass the operand of the rows (the two FP6 planes that w4a4_gemm_a8 lays
 *   out in its workspace for m > 16):
 *   act   out, w4a4_act8_operand_bytes(m, k) bytes, 256-byte aligned; private
 *         layout.  Other arguments and errors as w4a4_rotate_quantize_act8.
 * w4a4_gemm_a8_prepared: the product of packed_w with such an operand, as
 *   w4a4_gemm_a8 (any m >= 1; y [m][ldy] fp32; no workspace: the int8 path
 *   does not split K).  Errors as w4a4_gemm_prepared.
 */
size_t w4a4_act8_operand_bytes(int64_t m, int64_t k);
w4a4_status w4a4_rotate_quantize_prepare8(const void *x, w4a4_dtype dt, int64_t m, int64_t k, int64_t ldx,
                                          int8_t *codes, float *scales, void *act, size_t act_bytes,
                                          void *stream);
w4a4_status w4a4_gemm_a8_prepared(const void *packed_w, const void *act, float *y, int64_t m, int64_t n,
                                  int64_t k, int64_t ldy, void *stream);

/*
 * Unrotated W4A4, the ablation of section "MoE: W4A4 on the experts" (the
 * same W4A4 without the rotation costs about twice the accuracy).  Both
 * sides skip the rotation; the GEMM entry points are the same, fed with
 * weights packed from w4a4_quantize_q4_0 and codes from w4a4_quantize_act.
 * (Pairing these with rotated weights, or rotated activations with these
 * weights, computes garbage: the rotation identity needs both sides.)
 *
 * w4a4_quantize_q4_0: plain Q4_0 of the unrotated weights; arguments and
 * arithmetic as w4a4_quantize_q4_0_h32 without the rotation step (the
 * quantiser sees the fp32 weights themselves).
 *
 * w4a4_quantize_act: per-block symmetric int4 without the rotation;
 * arguments and errors as w4a4_rotate_quantize_act.  Per block: d = amax / 7,
 * codes clamp(round-half-away(x * (1/d)), -7, 7), s = d (there is no
 * normalisation to fold in); a block with d below FLT_MIN gets zero codes
 * and s = 0.
 */
w4a4_status w4a4_quantize_q4_0(const float *w, int64_t n, int64_t k, int64_t ldw, void *q4_0, void *stream);
w4a4_status w4a4_quantize_act(const void *x, w4a4_dtype dt, int64_t m, int64_t k, int64_t ldx, uint8_t *codes,
                              float *scales, void *stream);

/*
 * Rotated W4A16 (section "Hadamard-rotated Q4_0: W4A4 prompt processing":
 * the rotated Q4_0 files also run with the activations rotated and kept at
 * 16 bits, with no 4-bit activation step).  Both operands are fp16 matrices
 * in one tiled layout, the matrix cores' fragment order, shared by the three
 * calls below.  With nbp = ceil(k / 32 / 8) * 8 (the block count padded to a
 * multiple of 8), the layout is [ceil(rows / 32)][nbp][2][64][8] fp16:
 * element (r, t) sits at tile r / 32, block t / 32, half (t % 32) / 16, lane
 * (r % 32) + 32 * ((t % 16) / 8), slot t % 8.  Rows past the matrix and
 * blocks past k / 32 hold +0.  The padding lets the GEMM load whole 32-row,
 * 8-block tiles without bounds checks; it adds exact zeros to every sum.
 *
 * w4a4_w16_weight_bytes(n, k): bytes of the dequantised weights,
 *   ceil(n / 32) * nbp * 2048.  w4a4_w16_act_bytes(m, k): bytes of the
 *   rotated activations, ceil(m / 32) * nbp * 2048.  Both 0 for invalid
 *   sizes; host only, pure.
 *
 * w4a4_dequantize_w16: Q4_0 [n][k/32] blocks (as w4a4_quantize_q4_0_h32
 *   writes them) -> w16, element t of block b of row r =
 *   fp16(fl(d * (q_t - 8))) (d the block's fp16 scale as fp32; the product
 *   is exact, one rounding to nearest even).  w16: device, 16-byte aligned,
 *   at least w4a4_w16_weight_bytes(n, k) bytes (else
 *   W4A4_ERR_WORKSPACE_TOO_SMALL), fully written including the padding.
 *   Done once per weight matrix.
 *
 * w4a4_rotate_act16: x as w4a4_rotate_quantize_act (fp32 or fp16 [m][ldx],
 *   element-aligned) -> a16, element t of block b of row r =
 *   fp16(fl(v_t * c32)) with v the block's unnormalised 32-point
 *   Walsh-Hadamard butterflies in fp32 (the same sums the W4A4 quantiser
 *   forms) and c32 = fp32(1/sqrt(32)).  a16: device, 16-byte aligned, at
 *   least w4a4_w16_act_bytes(m, k) bytes, fully written including padding.
 *
 * w4a4_gemm_w16: y[i][j] = sum over t < k of a16[i][t] * w16[j][t], fp32
 *   sums of the exact fp16 products (the summation order is the matrix
 *   cores', not fixed).  a16, w16 as the two calls above write them, for
 *   the same k; y: fp32 [m][ldy], ldy >= n, 4-byte aligned; only the m x n
 *   block is written.  k == 0 writes zeros.
 *
 * Errors (all three): negative sizes, ldx < k or ldy < n ->
 * W4A4_ERR_INVALID_VALUE; k % 32 -> W4A4_ERR_K_NOT_MULTIPLE_OF_32; null
 * pointers with work to do, or sizes past the bounds (2^20 or more 128 x 128
 * output tiles for w4a4_gemm_w16) -> W4A4_ERR_INVALID_VALUE; misalignment ->
 * W4A4_ERR_MISALIGNED.  Empty sizes return W4A4_OK having done nothing.
 */
size_t w4a4_w16_weight_bytes(int64_t n, int64_t k);
size_t w4a4_w16_act_bytes(int64_t m, int64_t k);
w4a4_status w4a4_dequantize_w16(const void *q4_0, int64_t n, int64_t k, void *w16, size_t w16_bytes,
                                void *stream);
w4a4_status w4a4_rotate_act16(const void *x, w4a4_dtype dt, int64_t m, int64_t k, int64_t ldx, void *a16,
                              size_t a16_bytes, void *stream);
w4a4_status w4a4_gemm_w16(const void *w16, const void *a16, float *y, int64_t m, int64_t n, int64_t k,
                          int64_t ldy, void *stream);

/* Workspace bytes w4a4_gemm_id needs (0 for invalid sizes).  Host only, pure. */
size_t w4a4_gemm_id_workspace_bytes(int64_t n_expert, int64_t n_tokens, int64_t top_k);

/*
 * MUL_MAT_ID: expert-routed W4A4 product (section "MoE: W4A4 on the experts").
 *   packed_w  n_expert consecutive packed buffers of w4a4_packed_weight_bytes(n, k).
 *   codes, scales  activation rows: n_tokens of them when act_rows_per_token
 *             == 1 (every slot of token t reads row t), n_tokens * top_k when
 *             act_rows_per_token == top_k (slot j of token t reads row
 *             t * top_k + j).
 *   ids       [n_tokens][top_k] int32 expert indices.  An id outside
 *             [0, n_expert) yields a zero output row (defined behaviour).
 *   y         out, [n_tokens][top_k][n] fp32.
 *   workspace device scratch of w4a4_gemm_id_workspace_bytes(n_expert,
 *             n_tokens, top_k) bytes, 256-byte aligned (the routing: expert
 *             offsets, tile counts, row permutation); contents on entry are
 *             ignored.  Calls that share a workspace must not overlap.
 * One launch groups the (token, slot) rows by expert (tiles of 32 rows per
 * expert; w4a4_gemm_id_route); a second streams each expert's 4-bit weight
 * records once per row tile against the tile's activation rows (read through
 * the permutation) and scatters the rows to y (w4a4_gemm_id_routed).  Each output element depends only on its own
 * row and column: the result does not depend on how rows are grouped.
 * Supports n_expert <= 8192.
 */
w4a4_status w4a4_gemm_id(const void *packed_w, int64_t n_expert, const uint8_t *codes,
                         const float *scales, int64_t act_rows_per_token, const int32_t *ids,
                         int64_t n_tokens, int64_t top_k, float *y, int64_t n, int64_t k,
                         void *workspace, size_t workspace_bytes, void *stream);

/*
 * w4a4_gemm_id in two steps, so that one routing serves every product of a
 * layer that reads the same ids (gate, up and down of an MoE block):
 *
 * w4a4_gemm_id_route: groups the (token, slot) rows of ids by expert into
 *   workspace (w4a4_gemm_id_workspace_bytes(n_expert, n_tokens, top_k)
 *   bytes, 256-byte aligned): expert offsets, row tiles per expert, and the
 *   row permutation, with the rows of invalid ids after the valid ones.  It
 *   depends on ids, n_expert, n_tokens and top_k only.
 *
 * w4a4_gemm_id_routed: the product of w4a4_gemm_id, reading the routing that
 *   w4a4_gemm_id_route wrote into workspace for the same n_expert, n_tokens
 *   and top_k (enqueued before it; the workspace is only read, so several
 *   routed products may share one routing).  Rows of invalid ids are zeroed
 *   as in w4a4_gemm_id.  Other arguments and errors as w4a4_gemm_id.
 */
w4a4_status w4a4_gemm_id_route(const int32_t *ids, int64_t n_expert, int64_t n_tokens, int64_t top_k,
                               void *workspace, size_t workspace_bytes, void *stream);
w4a4_status w4a4_gemm_id_routed(const void *packed_w, int64_t n_expert, const uint8_t *codes,
                                const float *scales, int64_t act_rows_per_token, int64_t n_tokens, int64_t top_k,
                                float *y, int64_t n, int64_t k, const void *workspace, size_t workspace_bytes,
                                void *stream);

#ifdef __cplusplus
}
#endif

#endif /* W4A4_H */
