"""Pins of the CPU oracle to things other than itself (no GPU needed).

Every oracle function is checked against a library routine (scipy's Hadamard
matrix, numpy's float16 conversion, numpy matmul in fp64), a closed form, an
invariant of the mathematics, or a pure-Python brute force on tiny inputs.
The method: 1bit-MONSTER engine docs, page "The lean option: ROCmFP4, ROCmI4
and Hadamard Q4_0", sections "Hadamard-rotated Q4_0: W4A4 prompt processing"
and "MoE: W4A4 on the experts".
"""
import decimal
import os
import struct

import numpy as np
import pytest
import scipy.linalg

import oracle
from hadamard_rotated_w4a4_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
H_SCIPY = scipy.linalg.hadamard(32).astype(np.int64)


def f32_bits(x):
    return struct.unpack("<I", struct.pack("<f", float(np.float32(x))))[0]


def decode_act_codes(codes_row, k):
    """Pure-Python decode of one activation row: element t of block b sits in
    byte 16b + t%16, low nibble for t < 16, high for t >= 16, two's complement."""
    out = []
    for b in range(k // 32):
        for t in range(32):
            byte = int(codes_row[16 * b + (t % 16)])
            nib = (byte & 15) if t < 16 else (byte >> 4)
            out.append(nib - 16 if nib >= 8 else nib)
    return out


def decode_q4_block(blk):
    d = np.frombuffer(bytes(blk[:2]), np.float16)[0].astype(np.float64)
    q = []
    for t in range(32):
        byte = int(blk[2 + (t % 16)])
        q.append((byte & 15) if t < 16 else (byte >> 4))
    return d, q


# --------------------------------------------------------------------------
# Hadamard matrix and constants
# --------------------------------------------------------------------------

def test_h32_is_scipy_sylvester_hadamard():
    assert np.array_equal(oracle.h32().astype(np.int64), H_SCIPY)


def test_h32_orthogonal_symmetric_kronecker():
    H = oracle.h32().astype(np.int64)
    assert np.array_equal(H @ H.T, 32 * np.eye(32, dtype=np.int64))
    assert np.array_equal(H, H.T)
    H2 = np.array([[1, 1], [1, -1]], np.int64)
    K = H2
    for _ in range(4):
        K = np.kron(K, H2)
    assert np.array_equal(H, K)


def test_normalisation_constants():
    decimal.getcontext().prec = 60
    exact = decimal.Decimal(1) / decimal.Decimal(32).sqrt()
    assert oracle.c64() == float(exact)  # correctly rounded to fp64
    # fp32 constant is the fp32 nearest to 1/sqrt(32)
    assert f32_bits(oracle.c32()) == 0x3E3504F3
    c = np.float32(oracle.c32())
    lo, hi = np.nextafter(c, np.float32(0)), np.nextafter(c, np.float32(1))
    e = float(exact)
    assert abs(float(c) - e) <= abs(float(lo) - e) and abs(float(c) - e) <= abs(float(hi) - e)


# --------------------------------------------------------------------------
# fp16 conversions
# --------------------------------------------------------------------------

def test_half_to_float_all_patterns():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float32)
    got = np.array([oracle.half_to_float(int(b)) for b in bits], np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def test_float_to_half_matches_numpy_rne():
    rng = np.random.default_rng(11)
    vals = [rng.standard_normal(4000).astype(np.float32) * np.float32(s)
            for s in (1e-7, 1e-5, 1e-3, 1, 100, 3e4)]
    # exact ties between adjacent fp16 values, subnormal ties, overflow edge
    h = np.arange(0, 0x7bff, 37, dtype=np.uint16).view(np.float16).astype(np.float64)
    h2 = np.arange(1, 0x7c00, 37, dtype=np.uint16).view(np.float16).astype(np.float64)
    n = min(len(h), len(h2))
    ties = ((h[:n] + np.nextafter(h[:n].astype(np.float16), np.float16(np.inf)).astype(np.float64)) / 2)
    extra = np.array([65504, 65519.99, 65520, 70000, 2**-24, 2**-25, 3 * 2**-26, 2**-14,
                      2**-14 - 2**-25, 0.0, -0.0], np.float64)
    allv = np.concatenate(vals + [ties.astype(np.float32), extra.astype(np.float32),
                                  -ties.astype(np.float32)])
    with np.errstate(over="ignore"):
        ref = allv.astype(np.float16).view(np.uint16)
    got = np.array([oracle.float_to_half(v) for v in allv], np.uint16)
    assert np.array_equal(got, ref)


# --------------------------------------------------------------------------
# offline weight rotation and Q4_0
# --------------------------------------------------------------------------

def test_weight_rotation_matches_fp64_matmul_and_is_orthogonal():
    w = synth.weights(64, 256, np.random.default_rng(3))
    wr = oracle.rotate_weights(w)
    blocks = w.astype(np.float64).reshape(64, 8, 32)
    ref = np.einsum("ij,rbj->rbi", H_SCIPY.astype(np.float64), blocks) / np.sqrt(32.0)
    ref32 = ref.astype(np.float32).reshape(64, 256)
    diff = np.abs(wr.view(np.int32).astype(np.int64) - ref32.view(np.int32).astype(np.int64))
    assert diff.max() <= 1 and np.count_nonzero(diff) <= 2
    # Parseval: the normalised transform preserves each block's energy
    e0 = (blocks ** 2).sum(-1)
    e1 = (wr.astype(np.float64).reshape(64, 8, 32) ** 2).sum(-1)
    np.testing.assert_allclose(e1, e0, rtol=1e-6)


def test_rotation_identity_exact_on_integers_and_fp64():
    rng = np.random.default_rng(4)
    w = rng.integers(-1000, 1000, 32).astype(np.int64)
    x = rng.integers(-1000, 1000, 32).astype(np.int64)
    assert (H_SCIPY @ w) @ (H_SCIPY @ x) == 32 * (w @ x)
    # x.w = (Hn x).(Hn w) with the oracle's rotation, up to fp32 rounding
    wf = rng.standard_normal((1, 32)).astype(np.float32)
    xf = rng.standard_normal((1, 32)).astype(np.float32)
    lhs = float(wf[0].astype(np.float64) @ xf[0].astype(np.float64))
    rhs = float(oracle.rotate_weights(wf)[0].astype(np.float64) @ oracle.rotate_weights(xf)[0].astype(np.float64))
    assert abs(lhs - rhs) <= 1e-6 * (np.abs(wf).sum() * np.abs(xf).sum() / 4 + 1e-30) + 1e-7


def test_q4_0_code_identity_fixture():
    rows = [list(map(int, ln.split())) for ln in open(os.path.join(GOLDEN, "q4_0_xor8.txt"))
            if ln.strip() and not ln.startswith("#")]
    assert len(rows) == 16
    for q, val, nib in rows:
        assert val == q - 8 and nib == q ^ 8
        signed = nib - 16 if nib >= 8 else nib
        assert signed == val
    # the oracle's dequantisation follows the same rule: d * (q - 8)
    blk = np.zeros((1, 1, 18), np.uint8)
    blk[0, 0, :2] = np.frombuffer(np.float16(0.5).tobytes(), np.uint8)
    for j in range(16):
        blk[0, 0, 2 + j] = j | ((15 - j) << 4)
    deq = oracle.q4_0_dequantize(blk, 32)[0]
    want = [0.5 * (j - 8) for j in range(16)] + [0.5 * (15 - j - 8) for j in range(16)]
    assert np.array_equal(deq, np.array(want, np.float32))


def test_q4_0_on_grid_round_trip():
    rng = np.random.default_rng(5)
    n, k = 40, 256
    w = np.empty((n, k), np.float32)
    for r in range(n):
        for b in range(k // 32):
            d = np.float32(np.float16(rng.uniform(0.001, 0.05) * rng.choice([-1, 1])))
            q = rng.integers(1, 16, 32)
            q[rng.integers(0, 32)] = 0  # the extreme element sits at code 0 (value -8d)
            w[r, 32 * b:32 * b + 32] = d * (q - 8).astype(np.float32)
    q4 = oracle.q4_0_quantize(w)
    assert np.array_equal(oracle.q4_0_dequantize(q4, k), w)
    assert np.array_equal(oracle.q4_0_quantize(oracle.q4_0_dequantize(q4, k)), q4)


def test_q4_0_off_grid_error_bound():
    w = synth.weights(64, 512, np.random.default_rng(6))
    q4 = oracle.q4_0_quantize(w)
    deq = oracle.q4_0_dequantize(q4, 512).astype(np.float64)
    for r in range(64):
        for b in range(16):
            blk = w[r, 32 * b:32 * b + 32].astype(np.float64)
            d16, q = decode_q4_block(q4[r, b])
            mx = blk[np.argmax(np.abs(blk))]
            d = mx / -8.0
            assert q[int(np.argmax(np.abs(blk)))] == 0
            assert abs(d16 - d) <= abs(d) * 2 ** -11 + 2 ** -25
            err = np.abs(blk - deq[r, 32 * b:32 * b + 32])
            # the grid d*(q-8), q in 0..15, reaches -8d on the extreme element's
            # side but only 7d on the other: beyond 7.5|d| there the code clamps to 15
            t = blk / d
            inside = t <= 7.5
            assert err[inside].max() <= abs(d) / 2 + 8 * abs(d - d16) + 1e-9
            if (~inside).any():
                assert np.all(np.array(q)[~inside] == 15)
                assert np.all(err[~inside] <= (t[~inside] - 7) * abs(d) + 8 * abs(d - d16) + 1e-9)


# --------------------------------------------------------------------------
# activation rotation and quantisation
# --------------------------------------------------------------------------

def test_fwht_exact_on_integers_and_involution():
    rng = np.random.default_rng(7)
    for _ in range(200):
        v = rng.integers(-(2 ** 18), 2 ** 18, 32)
        got = oracle.fwht32_f32(v.astype(np.float32))
        assert np.array_equal(got.astype(np.int64), H_SCIPY @ v)
        back = oracle.fwht32_f32(got)
        assert np.array_equal(back.astype(np.int64), 32 * v)


def test_fwht_close_to_fp64_transform():
    rng = np.random.default_rng(8)
    v = rng.standard_normal((500, 32)).astype(np.float32) * 7
    for row in v:
        got = oracle.fwht32_f32(row).astype(np.float64)
        ref = H_SCIPY @ row.astype(np.float64)
        assert np.abs(got - ref).max() <= 5 * 2 ** -24 * np.abs(row).sum() * 2


def test_quantiser_special_blocks():
    c32 = np.float32(oracle.c32())
    H = H_SCIPY
    # zero block and a block too small to have a normal scale
    for scale in (0.0, 1e-44):
        x = np.full((1, 32), scale, np.float32)
        codes, s = oracle.rotate_quantize_act(x)
        assert not codes.any() and s[0, 0] == 0.0
    # constant block a*1 -> H x = (32a, 0, ..., 0): codes (7 sign a, 0, ..., 0)
    for a in (0.37, -2.5, 1e-3, 300.0):
        x = np.full((1, 32), a, np.float32)
        codes, s = oracle.rotate_quantize_act(x)
        q = decode_act_codes(codes[0], 32)
        assert q == [7 * int(np.sign(a))] + [0] * 31
        d = np.float32(np.float32(32 * np.float32(abs(a))) / np.float32(7))
        assert s[0, 0] == np.float32(d * c32)
    # one-hot a*e_j -> (H x)_i = a H[i, j]: every code is +-7, the outlier spread over the block
    for j in (0, 5, 31):
        for a in (20.0, -3.25):
            x = np.zeros((1, 32), np.float32)
            x[0, j] = a
            codes, s = oracle.rotate_quantize_act(x)
            q = np.array(decode_act_codes(codes[0], 32))
            assert np.array_equal(q, 7 * int(np.sign(a)) * H[:, j])
            assert s[0, 0] == np.float32(np.float32(np.float32(abs(a)) / np.float32(7)) * c32)


def test_quantiser_closed_form_recovers_codes():
    """x = H(sigma*c)/32 with sigma a power of two: the rotation returns sigma*c
    exactly, so the quantiser must return the codes c and the scale sigma*c32."""
    rng = np.random.default_rng(9)
    m, k = 8, 256
    for dtype in (np.float32, np.float16):
        c = rng.integers(-7, 8, (m, k // 32, 32))
        for r in range(m):
            for b in range(k // 32):
                c[r, b, rng.integers(0, 32)] = rng.choice([-7, 7])
        sig = 2.0 ** rng.integers(-6, 4, (m, k // 32))
        x = np.einsum("ij,rbj->rbi", H_SCIPY, c).astype(np.float64) * (sig[..., None] / 32)
        x = x.reshape(m, k).astype(dtype)
        codes, s = oracle.rotate_quantize_act(x)
        for r in range(m):
            assert decode_act_codes(codes[r], k) == list(c[r].reshape(-1))
        assert np.array_equal(s, (sig.astype(np.float32) * np.float32(oracle.c32())).astype(np.float32))


def test_quantiser_rounds_to_nearest_with_ties_away():
    # H x = v with amax 7 (d = 1, id = 1): ties at +-2.5, +-0.5, 3.5 round away from zero
    v = np.zeros(32)
    v[:8] = [7, 2.5, -2.5, 0.5, -0.5, 3.5, -1.25, 6.5]
    x = (H_SCIPY @ v / 32).astype(np.float32)[None]
    assert np.array_equal(oracle.fwht32_f32(x[0]).astype(np.float64), v.astype(np.float32))
    codes, s = oracle.rotate_quantize_act(x)
    assert decode_act_codes(codes[0], 32)[:8] == [7, 3, -3, 1, -1, 4, -1, 7]


def test_quantiser_nearest_grid_point_on_random_data():
    d = synth.ffn_up(m=4)
    x = d.x[:, :1024]
    codes, s = oracle.rotate_quantize_act(x)
    c32 = float(np.float32(oracle.c32()))
    for r in range(4):
        q = np.array(decode_act_codes(codes[r], 1024)).reshape(32, 32)
        v = (x[r].astype(np.float64).reshape(32, 32) @ H_SCIPY.T)  # exact H x per block
        for b in range(32):
            dd = float(s[r, b]) / c32
            assert np.abs(q[b]).max() == 7
            assert np.abs(v[b] / dd - q[b]).max() <= 0.5 + 1e-5
            assert abs(dd - np.abs(v[b]).max() / 7) <= 1e-6 * dd


def test_quantiser_respects_row_stride():
    rng = np.random.default_rng(10)
    x = rng.standard_normal((5, 96)).astype(np.float16)
    c1, s1 = oracle.rotate_quantize_act(x, k=64)
    c2, s2 = oracle.rotate_quantize_act(np.ascontiguousarray(x[:, :64]))
    assert np.array_equal(c1, c2) and np.array_equal(s1, s2)


# --------------------------------------------------------------------------
# integer block dots and the fp32 output
# --------------------------------------------------------------------------

def _tiny_problem(seed, m=3, n=4, k=64):
    rng = np.random.default_rng(seed)
    w = synth.weights(n, k, rng)
    x = rng.standard_normal((m, k)).astype(np.float32) * 3
    q4 = oracle.prepare_weights(w)
    codes, s = oracle.rotate_quantize_act(x)
    return q4, codes, s, k


def test_block_sums_brute_force():
    q4, codes, s, k = _tiny_problem(12)
    S = oracle.block_sums(q4, codes, k)
    for i in range(codes.shape[0]):
        qa = decode_act_codes(codes[i], k)
        for j in range(q4.shape[0]):
            for b in range(k // 32):
                _, qw = decode_q4_block(q4[j, b])
                assert S[i, j, b] == sum((qw[t] - 8) * qa[32 * b + t] for t in range(32))


def test_block_sum_extremes():
    blk_w = np.zeros((1, 1, 18), np.uint8)
    blk_w[0, 0, :2] = np.frombuffer(np.float16(1).tobytes(), np.uint8)  # all codes 0 -> -8
    act = np.full((1, 16), 0x99, np.uint8)  # every nibble 9 = -7
    assert oracle.block_sums(blk_w, act, 32)[0, 0, 0] == 32 * 56
    blk_w[0, 0, 2:] = 0xff  # codes 15 -> +7
    assert oracle.block_sums(blk_w, act, 32)[0, 0, 0] == -32 * 49


def test_gemm_brute_force_tiny():
    q4, codes, s, k = _tiny_problem(13)
    y = oracle.gemm(q4, codes, s, k, threads=2)
    for i in range(codes.shape[0]):
        qa = decode_act_codes(codes[i], k)
        for j in range(q4.shape[0]):
            acc = 0.0
            for b in range(k // 32):
                d, qw = decode_q4_block(q4[j, b])
                S = sum((qw[t] - 8) * qa[32 * b + t] for t in range(32))
                acc += d * float(s[i, b]) * S
            assert y[i, j] == np.float32(acc)


def test_gemm_closed_form_matches_fp64_matmul():
    """Activations on the quantiser grid: the W4A4 product must equal the fp64
    product of the dequantised rotated weights with the rotated activations."""
    rng = np.random.default_rng(14)
    m, n, k = 6, 10, 256
    c = rng.integers(-7, 8, (m, k // 32, 32))
    c[:, :, 0] = 7
    sig = 2.0 ** rng.integers(-3, 3, (m, k // 32))
    x = (np.einsum("ij,rbj->rbi", H_SCIPY, c) * (sig[..., None] / 32)).reshape(m, k).astype(np.float32)
    w = synth.weights(n, k, rng)
    q4 = oracle.prepare_weights(w)
    codes, s = oracle.rotate_quantize_act(x)
    y = oracle.gemm(q4, codes, s, k).astype(np.float64)
    wdeq = oracle.q4_0_dequantize(q4, k).astype(np.float64)
    hx = (sig[..., None] * c).reshape(m, k) / np.sqrt(32.0)  # H/sqrt(32) applied to x, exact
    ref = hx @ wdeq.T
    np.testing.assert_allclose(y, ref, rtol=1e-6, atol=1e-9 * np.abs(ref).max())


def test_gemm_approximates_unrotated_product():
    """End to end with the offline rotation: y ~ W x up to 4-bit noise."""
    d = synth.tiny()
    q4 = oracle.prepare_weights(d.w)
    codes, s = oracle.rotate_quantize_act(d.x)
    y = oracle.gemm(q4, codes, s, d.k).astype(np.float64)
    ref = d.x.astype(np.float64) @ d.w.astype(np.float64).T
    rel = np.abs(y - ref).max(1) / np.abs(ref).max(1)
    assert rel.max() < 0.35 and np.median(rel) < 0.2
    # rotating only one side breaks the identity: error jumps
    q4_plain = oracle.q4_0_quantize(d.w)
    y_bad = oracle.gemm(q4_plain, codes, s, d.k).astype(np.float64)
    assert (np.abs(y_bad - ref).max(1) / np.abs(ref).max(1)).min() > 0.5


def test_rotation_lowers_w4a4_error_on_outliers():
    """Direction only: W4A4 with H32 beats W4A4 without it on outlier data."""
    d = synth.tiny()
    ref = d.x.astype(np.float64) @ d.w.astype(np.float64).T
    q4 = oracle.prepare_weights(d.w)
    codes, s = oracle.rotate_quantize_act(d.x)
    err_rot = np.abs(oracle.gemm(q4, codes, s, d.k) - ref).mean()
    # no rotation: quantise x itself (feed H x/32, which the transform maps back to x)
    pre = (d.x.astype(np.float64).reshape(64, 8, 32) @ H_SCIPY.T / 32).reshape(64, 256).astype(np.float32)
    codes_p, s_p = oracle.rotate_quantize_act(pre)
    # without rotation the stored scale is d * c32; undo c32 on the activation side
    s_p = (s_p.astype(np.float64) / float(np.float32(oracle.c32()))).astype(np.float32)
    err_plain = np.abs(oracle.gemm(oracle.q4_0_quantize(d.w), codes_p, s_p, d.k) - ref).mean()
    assert err_rot < err_plain


# --------------------------------------------------------------------------
# W4A8-H32 (reading R8): int8 activation codes, the same rotation
# --------------------------------------------------------------------------

def test_quantiser8_special_blocks():
    c32 = np.float32(oracle.c32())
    for scale in (0.0, 1e-44):
        codes, s = oracle.rotate_quantize_act8(np.full((1, 32), scale, np.float32))
        assert not codes.any() and s[0, 0] == 0.0
    # constant block: H x = (32a, 0, ..., 0) -> codes (127 sign a, 0, ...)
    for a in (0.37, -2.5, 300.0):
        codes, s = oracle.rotate_quantize_act8(np.full((1, 32), a, np.float32))
        assert list(codes[0]) == [127 * int(np.sign(a))] + [0] * 31
        d = np.float32(np.float32(32 * np.float32(abs(a))) / np.float32(127))
        assert s[0, 0] == np.float32(d * c32)
    # one-hot: every rotated value is +-a, so every code is +-127
    for j in (0, 17):
        x = np.zeros((1, 32), np.float32)
        x[0, j] = -4.0
        codes, s = oracle.rotate_quantize_act8(x)
        assert np.array_equal(codes[0].astype(int), -127 * H_SCIPY[:, j])


def test_quantiser8_closed_form_recovers_codes():
    """x = H(sigma*c)/32, c in [-127, 127] with 127 in every block, sigma a
    power of two: the quantiser returns c and sigma*c32."""
    rng = np.random.default_rng(19)
    m, k = 6, 256
    c = rng.integers(-127, 128, (m, k // 32, 32))
    for r in range(m):
        for b in range(k // 32):
            c[r, b, rng.integers(0, 32)] = rng.choice([-127, 127])
    sig = 2.0 ** rng.integers(-8, -2, (m, k // 32))
    x = (np.einsum("ij,rbj->rbi", H_SCIPY, c) * (sig[..., None] / 32)).reshape(m, k).astype(np.float32)
    codes, s = oracle.rotate_quantize_act8(x)
    assert np.array_equal(codes.astype(int).reshape(m, k // 32, 32), c)
    assert np.array_equal(s, (sig.astype(np.float32) * np.float32(oracle.c32())).astype(np.float32))


def test_quantiser8_ties_away_and_nearest():
    v = np.zeros(32)
    v[:6] = [127, 2.5, -2.5, 0.5, -100.5, 3.25]  # amax 127: d = 1, ties round away from zero
    x = (H_SCIPY @ v / 32).astype(np.float32)[None]
    codes, _ = oracle.rotate_quantize_act8(x)
    assert list(codes[0, :6]) == [127, 3, -3, 1, -101, 3]
    d = synth.ffn_up(m=2)
    x = d.x[:, :512]
    codes, s = oracle.rotate_quantize_act8(x)
    c32 = float(np.float32(oracle.c32()))
    v = x.astype(np.float64).reshape(2, 16, 32) @ H_SCIPY.T
    dd = s.astype(np.float64) / c32
    assert np.abs(v / dd[..., None] - codes.reshape(2, 16, 32)).max() <= 0.5 + 1e-4
    assert (np.abs(codes.reshape(2, 16, 32)).max(axis=2) == 127).all()


def test_block_sums8_brute_force_and_extremes():
    rng = np.random.default_rng(20)
    w = synth.weights(3, 64, rng)
    x = rng.standard_normal((2, 64)).astype(np.float32) * 3
    q4 = oracle.prepare_weights(w)
    codes, _ = oracle.rotate_quantize_act8(x)
    S = oracle.block_sums_a8(q4, codes, 64)
    for i in range(2):
        for j in range(3):
            for b in range(2):
                _, qw = decode_q4_block(q4[j, b])
                assert S[i, j, b] == sum((qw[t] - 8) * int(codes[i, 32 * b + t]) for t in range(32))
    blk_w = np.zeros((1, 1, 18), np.uint8)  # codes 0 -> -8
    act = np.full((1, 32), -127, np.int8)
    assert oracle.block_sums_a8(blk_w, act, 32)[0, 0, 0] == 32 * 8 * 127


def test_gemm8_brute_force_tiny():
    rng = np.random.default_rng(21)
    w = synth.weights(4, 96, rng)
    x = rng.standard_normal((3, 96)).astype(np.float32)
    q4 = oracle.prepare_weights(w)
    codes, s = oracle.rotate_quantize_act8(x)
    y = oracle.gemm_a8(q4, codes, s, 96, threads=2)
    for i in range(3):
        for j in range(4):
            acc = 0.0
            for b in range(3):
                d, qw = decode_q4_block(q4[j, b])
                S = sum((qw[t] - 8) * int(codes[i, 32 * b + t]) for t in range(32))
                acc += d * float(s[i, b]) * S
            assert y[i, j] == np.float32(acc)


def test_w4a8_error_far_below_w4a4():
    """Both against the fp64 product of the dequantised rotated weights with the
    exactly rotated activations: 8-bit codes leave ~16x less activation noise."""
    d = synth.tiny()
    q4 = oracle.prepare_weights(d.w)
    wdeq = oracle.q4_0_dequantize(q4, d.k).astype(np.float64)
    hx = (d.x.astype(np.float64).reshape(64, 8, 32) @ H_SCIPY.T / np.sqrt(32.0)).reshape(64, 256)
    ref = hx @ wdeq.T
    c4, s4 = oracle.rotate_quantize_act(d.x)
    c8, s8 = oracle.rotate_quantize_act8(d.x)
    e4 = np.abs(oracle.gemm(q4, c4, s4, d.k) - ref).mean()
    e8 = np.abs(oracle.gemm_a8(q4, c8, s8, d.k) - ref).mean()
    assert e8 < e4 / 8


# --------------------------------------------------------------------------
# MUL_MAT_ID
# --------------------------------------------------------------------------

def test_gemm_id_single_expert_reduces_to_gemm():
    q4, codes, s, k = _tiny_problem(15, m=5, n=6)
    ids = np.zeros((5, 1), np.int32)
    y = oracle.gemm_id(q4[None], codes, s, 1, ids, 6, k)
    assert np.array_equal(y[:, 0, :], oracle.gemm(q4, codes, s, k))


def test_gemm_id_is_gather_then_dense():
    rng = np.random.default_rng(16)
    E, T, top_k, n, k = 5, 7, 3, 8, 64
    q4e = np.stack([oracle.prepare_weights(synth.weights(n, k, rng)) for _ in range(E)])
    ids = np.stack([rng.choice(E, top_k, replace=False) for _ in range(T)]).astype(np.int32)
    ids[2, 1] = E + 3   # out of range -> zero row
    ids[4, 0] = -1
    for rows_per_token in (1, top_k):
        x = rng.standard_normal((T * rows_per_token, k)).astype(np.float16)
        codes, s = oracle.rotate_quantize_act(x)
        y = oracle.gemm_id(q4e, codes, s, rows_per_token, ids, n, k)
        for t in range(T):
            for j in range(top_k):
                e = ids[t, j]
                if not 0 <= e < E:
                    assert not y[t, j].any()
                    continue
                r = t if rows_per_token == 1 else t * top_k + j
                ref = oracle.gemm(q4e[e], codes[r:r + 1], s[r:r + 1], k)[0]
                assert np.array_equal(y[t, j], ref)


# --------------------------------------------------------------------------
# regression anchor: the tiny workload's oracle outputs
# --------------------------------------------------------------------------

def test_tiny_workload_golden_digests():
    import hashlib
    import json
    path = os.path.join(GOLDEN, "tiny_m64_k256_n256.json")
    if not os.path.exists(path):
        pytest.skip("golden file not generated")
    ref = json.load(open(path))
    d = synth.tiny()
    q4 = oracle.prepare_weights(d.w)
    codes, s = oracle.rotate_quantize_act(d.x)
    y = oracle.gemm(q4, codes, s, d.k)
    got = {"q4_0": q4, "codes": codes, "scales": s, "y": y}
    for key, arr in got.items():
        assert hashlib.sha256(arr.tobytes()).hexdigest() == ref[key + "_sha256"], key


# --------------------------------------------------------------------------
# Unrotated W4A4 ablation (reading R9): no rotation on either side
# --------------------------------------------------------------------------

def test_plain_quantiser_special_blocks():
    """Closed forms: zero and subnormal blocks give zeros; a constant block a
    gives all codes 7 sign(a) with s = fl(|a| / 7); a one-hot block a e_j gives
    7 sign(a) at j only (no rotation spreads it)."""
    for scale in (0.0, 1e-44):
        codes, s = oracle.quantize_act_plain(np.full((1, 32), scale, np.float32))
        assert not codes.any() and s[0, 0] == 0.0
    for a in (0.37, -2.5, 1e-3, 300.0):
        codes, s = oracle.quantize_act_plain(np.full((1, 32), a, np.float32))
        assert decode_act_codes(codes[0], 32) == [7 * int(np.sign(a))] * 32
        assert s[0, 0] == np.float32(np.float32(abs(a)) / np.float32(7))
    for j in (0, 5, 16, 31):
        for a in (20.0, -3.25):
            x = np.zeros((1, 32), np.float32)
            x[0, j] = a
            codes, s = oracle.quantize_act_plain(x)
            q = [0] * 32
            q[j] = 7 * int(np.sign(a))
            assert decode_act_codes(codes[0], 32) == q
            assert s[0, 0] == np.float32(np.float32(abs(a)) / np.float32(7))


def test_plain_quantiser_power_of_two_invariance():
    """Scaling a block by 2^e leaves its codes and scales its scale by 2^e
    exactly (every step is a correctly rounded fp32 operation)."""
    rng = np.random.default_rng(41)
    x = synth.activations(6, 256, rng, 3)
    c0, s0 = oracle.quantize_act_plain(x)
    for e in (-5, 3, 12):
        c1, s1 = oracle.quantize_act_plain((x * np.float32(2.0 ** e)).astype(np.float32))
        assert np.array_equal(c0, c1)
        assert np.array_equal(s1, (s0 * np.float32(2.0 ** e)).astype(np.float32))


def test_plain_quantiser_is_the_rotated_rule_before_the_rotation():
    """The rotated quantiser (R5, pinned above) is this one applied to the
    FWHT of each block, with the scale times c32: codes equal, and
    s_R5 = fl(s_plain * c32)."""
    rng = np.random.default_rng(43)
    x = synth.activations(8, 256, rng, 3)
    c_rot, s_rot = oracle.rotate_quantize_act(x)
    xh = np.stack([oracle.fwht32_f32(blk) for blk in x.reshape(-1, 32)]).reshape(x.shape).astype(np.float32)
    c_pl, s_pl = oracle.quantize_act_plain(xh)
    assert np.array_equal(c_rot, c_pl)
    assert np.array_equal(s_rot, (s_pl * np.float32(oracle.c32())).astype(np.float32))


def test_ablation_without_rotation_costs_more():
    """Direction of the ablation (section "MoE: W4A4 on the experts"): on
    outlier data, plain Q4_0 weights with unrotated int4 activations land
    further from the exact fp64 product than the rotated pair does."""
    d = synth.tiny()
    ref = d.x.astype(np.float64) @ d.w.astype(np.float64).T
    y_rot = oracle.gemm(oracle.prepare_weights(d.w), *oracle.rotate_quantize_act(d.x), d.k)
    y_plain = oracle.gemm(oracle.prepare_weights_plain(d.w), *oracle.quantize_act_plain(d.x), d.k)
    err_rot = np.abs(y_rot - ref).mean()
    err_plain = np.abs(y_plain - ref).mean()
    assert err_plain > 1.3 * err_rot


# --------------------------------------------------------------------------
# Rotated W4A16 (reading R10): rotated fp16 activations, fp16-dequantised Q4_0
# --------------------------------------------------------------------------

def test_act16_is_the_rounded_fwht():
    """x16 = fp16(fl(FWHT(x) * c32)): the pinned butterflies, then numpy's own
    fp16 rounding (nearest even) of the fp32 product."""
    rng = np.random.default_rng(51)
    for dtype in (np.float32, np.float16):
        x = synth.activations(5, 160, rng, 2).astype(dtype)
        got = oracle.rotate_act16(x)
        c32 = np.float32(oracle.c32())
        want = np.stack([(oracle.fwht32_f32(blk.astype(np.float32)) * c32).astype(np.float16)
                         for blk in x.reshape(-1, 32)]).reshape(5, 160)
        assert np.array_equal(got.view(np.uint16), want.view(np.uint16))


def test_act16_closed_forms():
    """Constant block a: (32 a c32, 0, ..., 0); one-hot a e_j: a c32 H[:, j],
    each rounded to fp16."""
    c32 = np.float32(oracle.c32())
    for a in (0.5, -3.0, 1e-3):
        got = oracle.rotate_act16(np.full((1, 32), a, np.float32))[0]
        assert got[0] == np.float16(np.float32(np.float32(32 * np.float32(a)) * c32)) and not got[1:].any()
    for j in (0, 9, 31):
        x = np.zeros((1, 32), np.float32)
        x[0, j] = -7.5
        got = oracle.rotate_act16(x)[0].astype(np.float64)
        assert np.array_equal(got, float(np.float16(np.float32(np.float32(7.5) * c32))) * -H_SCIPY[:, j])


def test_w16_dequantisation_from_the_bytes():
    """w16 = fp16(fl(d * (q - 8))) decoded straight from the Q4_0 bytes with
    numpy: d from the little-endian fp16, codes from the nibbles."""
    rng = np.random.default_rng(53)
    w = synth.weights(7, 96, rng)
    q4 = oracle.prepare_weights(w)
    got = oracle.dequantize_w16(q4, 96)
    d = q4[..., 0:2].copy().view(np.float16)[..., 0].astype(np.float32)          # [n, nb]
    lo, hi = q4[..., 2:] & 0xF, q4[..., 2:] >> 4                                  # codes j, j + 16
    q = np.concatenate([lo, hi], axis=-1).astype(np.float32) - 8.0               # [n, nb, 32]
    want = (d[..., None] * q).astype(np.float16).reshape(7, 96)
    assert np.array_equal(got.view(np.uint16), want.view(np.uint16))


def test_gemm_w16_is_the_fp64_product_of_the_operands():
    rng = np.random.default_rng(55)
    w16 = oracle.dequantize_w16(oracle.prepare_weights(synth.weights(24, 128, rng)), 128)
    x16 = oracle.rotate_act16(synth.activations(9, 128, rng, 2))
    y = oracle.gemm_w16(w16, x16).astype(np.float64)
    ref = x16.astype(np.float64) @ w16.astype(np.float64).T
    # fp64 sums in another order differ far below half an fp32 ulp of the result
    assert np.array_equal(y.astype(np.float32), ref.astype(np.float32)) or \
        (np.abs(y - ref) <= np.abs(ref) * 2.0 ** -23).all()


def test_w4a16_error_below_w4a4():
    """Keeping the rotated activations at 16 bits lands closer to the exact
    product than rounding them to 4 bits (same rotated Q4_0 weights)."""
    d = synth.tiny()
    ref = d.x.astype(np.float64) @ d.w.astype(np.float64).T
    q4 = oracle.prepare_weights(d.w)
    y16 = oracle.gemm_w16(oracle.dequantize_w16(q4, d.k), oracle.rotate_act16(d.x))
    y4 = oracle.gemm(q4, *oracle.rotate_quantize_act(d.x), d.k)
    assert np.abs(y16 - ref).mean() < 0.9 * np.abs(y4 - ref).mean()
