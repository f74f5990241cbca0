"""The C oracle's activation quantisers against a second implementation
(tests/quant_twin.py, numpy float32, whole arrays at once): codes, scales and
fp16 values must agree bit for bit.

The pages print no rounding rule for the activations (1bit-MONSTER engine
docs, page "The lean option: ROCmFP4, ROCmI4 and Hadamard Q4_0", section
"Hadamard-rotated Q4_0: W4A4 prompt processing"), so these pins fix the
readings R4/R5 (W4A4), R8 (W4A8), R9 (unrotated ablation) and R10 (rotated
W4A16) as stated in oracle/oracle.c, on 2^20 random blocks per rule and input
type and on blocks built to sit on the decisions that an implementation slip
would flip:
  * ties and near-ties: rotated values v with v * id = k + 1/2 up to the one
    rounding of id = fl(1 / fl(amax / q)) (exact ties and values one ulp to
    either side, both counted), built exactly in the rotated domain;
  * fp16 subnormal inputs; fp32 inputs whose d falls just above and below the
    smallest normal float32 (zero block or not);
  * several elements at +-amax; a single x20 outlier per block; constant and
    one-hot blocks; huge and tiny magnitudes.
"""
import numpy as np
import pytest

import oracle
import quant_twin as tw

H = np.array([[(-1) ** bin(i & j).count("1") for j in range(32)] for i in range(32)], np.int64)
N_RANDOM = 1 << 20  # blocks per rule and input type


def random_inputs(dtype, seed, nblocks=N_RANDOM, rows=256):
    """Blocks of N(0,1) at a per-block scale 10^U(-4, 4) (fp16: 10^U(-3, 2.5),
    clipped to stay finite), a quarter of them with one x20 outlier."""
    rng = np.random.default_rng(seed)
    k = nblocks // rows * 32
    x = rng.standard_normal((rows, k)).astype(np.float32)
    lo, hi = (-3.0, 2.5) if dtype == np.float16 else (-4.0, 4.0)
    scale = 10.0 ** rng.uniform(lo, hi, (rows, k // 32, 1))
    x = (x.reshape(rows, k // 32, 32) * scale)
    hit = rng.random((rows, k // 32)) < 0.25
    pos = rng.integers(0, 32, (rows, k // 32))
    r, b = np.nonzero(hit)
    x[r, b, pos[r, b]] *= 20.0
    if dtype == np.float16:
        x = np.clip(x, -65000.0, 65000.0)
    return x.reshape(rows, k).astype(dtype)


def check_all_rules(x):
    c, s = oracle.rotate_quantize_act(x)
    tc, ts = tw.rotate_quantize_act(x)
    assert np.array_equal(c, tc), "R5 codes differ"
    assert np.array_equal(s.view(np.uint32), ts.view(np.uint32)), "R5 scales differ"
    c8, s8 = oracle.rotate_quantize_act8(x)
    tc8, ts8 = tw.rotate_quantize_act8(x)
    assert np.array_equal(c8, tc8), "R8 codes differ"
    assert np.array_equal(s8.view(np.uint32), ts8.view(np.uint32)), "R8 scales differ"
    cp, sp = oracle.quantize_act_plain(x)
    tcp, tsp = tw.quantize_act_plain(x)
    assert np.array_equal(cp, tcp), "R9 codes differ"
    assert np.array_equal(sp.view(np.uint32), tsp.view(np.uint32)), "R9 scales differ"
    a16 = oracle.rotate_act16(x)
    t16 = tw.rotate_act16(x)
    assert np.array_equal(a16.view(np.uint16), t16.view(np.uint16)), "R10 values differ"


def test_twin_constant_is_the_oracle_constant():
    assert tw.C32.view(np.uint32) == np.float32(oracle.c32()).view(np.uint32) == 0x3E3504F3


def test_twin_butterflies_are_the_hadamard_product_on_integers():
    """The twin itself is pinned: on integer blocks its fp32 butterflies are
    exact and equal H v."""
    rng = np.random.default_rng(3)
    v = rng.integers(-2 ** 18, 2 ** 18, (1000, 32))
    assert np.array_equal(tw.butterflies(v.astype(np.float32)).astype(np.int64), v @ H.T)


@pytest.mark.parametrize("dtype,seed", [(np.float16, 101), (np.float32, 102)])
def test_random_blocks_bit_exact(dtype, seed):
    check_all_rules(random_inputs(dtype, seed))


def _from_rotated(y):
    """Inputs whose R4 butterflies are exactly y (integer rows, |H y| small):
    x = H y / 32, exact in fp32 (and fp16 when |H y| <= 2048)."""
    return (y @ H.T).astype(np.float64) / 32.0


def near_tie_blocks(rng, nblocks, jmax, sparse):
    """Rotated blocks y with amax A = 14 j (j not a power of two) and the
    other entries (2 k + 1) j, so that y * (7 / A) = k + 1/2 exactly in the
    reals: with id = fl(1 / fl(A / 7)) = fl(1 / (2 j)) rounded, fl(y * id)
    lands on k + 1/2 or one ulp to either side."""
    js = rng.integers(3, jmax + 1, nblocks)
    js = js[(js & (js - 1)) != 0]
    y = np.zeros((js.size, 32), np.int64)
    for r, j in enumerate(js):
        cols = rng.choice(32, 4 if sparse else 32, replace=False)
        ks = rng.integers(0, 7, cols.size)
        y[r, cols] = (2 * ks + 1) * j * rng.choice([-1, 1], cols.size)
        y[r, cols[0]] = 14 * j * rng.choice([-1, 1])
    return y, js


def _count_ties(y, js, qmax=7):
    """How many elements of the rotated blocks land exactly on, and one ulp
    beside, a half-integer after the scaling (as the readings compute it)."""
    A = np.abs(y).max(axis=1).astype(np.float32)
    inv = np.float32(1) / (A / np.float32(qmax))
    r = y.astype(np.float32) * inv[:, None]
    f = np.abs(r.astype(np.float64))
    frac = f - np.floor(f)
    exact = int(np.sum((frac == 0.5)))
    near = int(np.sum((frac != 0.5) & (np.abs(frac - 0.5) <= 2.0 * np.spacing(r.astype(np.float32)).astype(np.float64))))
    return exact, near


@pytest.mark.parametrize("dtype", [np.float32, np.float16])
def test_ties_and_near_ties(dtype):
    rng = np.random.default_rng(7 if dtype == np.float32 else 8)
    if dtype == np.float32:
        y, js = near_tie_blocks(rng, 20000, 4000, sparse=False)
    else:
        y, js = near_tie_blocks(rng, 20000, 36, sparse=True)
    x = _from_rotated(y)
    xd = x.astype(dtype)
    assert np.array_equal(xd.astype(np.float64), x), "construction not exact in the input type"
    assert np.array_equal(tw.butterflies(xd.astype(np.float32)), y.astype(np.float32))
    exact, near = _count_ties(y, js)
    assert exact > 1000 and near > 1000, (exact, near)
    rows = xd.reshape(-1, 32 * 8) if xd.shape[0] % 8 == 0 else xd.reshape(-1, 32)
    check_all_rules(np.ascontiguousarray(rows))


def test_fp16_subnormal_inputs():
    rng = np.random.default_rng(11)
    bits = rng.integers(-1023, 1024, (64, 32 * 256)).astype(np.int32)
    x = (bits.astype(np.float64) * 2.0 ** -24).astype(np.float16)  # every fp16 subnormal (and 0)
    assert np.all(np.abs(x.astype(np.float64)) < 2.0 ** -14)
    check_all_rules(x)


def test_scale_at_the_smallest_normal():
    """d = amax / q just below, at and above FLT_MIN: zero blocks below."""
    tiny = np.float64(np.finfo(np.float32).tiny)
    rows = []
    for q in (7.0, 127.0):
        for f in (0.5, 0.999, 0.9999999, 1.0, 1.0000001, 1.001, 2.0, 1.0e3):
            for pos in (0, 5, 31):
                blk = np.zeros(32)
                blk[pos] = q * tiny * f
                rows.append(blk)
                blk2 = np.full(32, q * tiny * f / 32.0)  # rotates to (q tiny f, 0, ..., 0)
                rows.append(blk2)
    x = np.array(rows, np.float32)
    pad = (-x.shape[0]) % 8
    x = np.concatenate([x, np.zeros((pad, 32), np.float32)]).reshape(-1, 32 * 8)
    check_all_rules(x)


def test_amax_ties_outliers_constants_and_extremes():
    rng = np.random.default_rng(13)
    blocks = []
    for _ in range(4096):  # several elements at +-amax in the rotated domain
        y = rng.integers(-50, 51, 32)
        cols = rng.choice(32, rng.integers(2, 6), replace=False)
        y[cols] = 64 * rng.choice([-1, 1], cols.size)
        blocks.append(_from_rotated(y))
    for _ in range(4096):  # a single x20 outlier in the input
        b = rng.standard_normal(32)
        b[rng.integers(32)] *= 20.0
        blocks.append(b * 10.0 ** rng.uniform(-3, 3))
    for a in (1.0, -3.25, 1e-3, 7e5):  # constant and one-hot blocks
        blocks.append(np.full(32, a))
        for j in (0, 13, 31):
            e = np.zeros(32)
            e[j] = a
            blocks.append(e)
    for mag in (1e30, 1e36, 1e-30, 1e-37):  # huge and tiny magnitudes (no overflow in the sums)
        blocks.append(rng.standard_normal(32) * mag)
    x = np.array(blocks)
    pad = (-x.shape[0]) % 8
    x = np.concatenate([x, np.zeros((pad, 32))]).reshape(-1, 32 * 8)
    check_all_rules(x.astype(np.float32))
    x16 = np.clip(x, -6e4, 6e4).astype(np.float16)
    check_all_rules(x16)


def test_a_planted_slip_is_caught():
    """The comparison has teeth: the twin with division in place of the
    multiply by the reciprocal, or with ties to even, disagrees with the oracle
    on the tie blocks."""
    rng = np.random.default_rng(7)
    y, _ = near_tie_blocks(rng, 4000, 4000, sparse=False)
    x = _from_rotated(y).astype(np.float32).reshape(-1, 32 * 4)
    c, _ = oracle.rotate_quantize_act(x)
    v = tw.butterflies(tw.blocks_of(x))
    d = np.max(np.abs(v), axis=1) / np.float32(7)
    by_division = np.clip(tw.round_half_away(v / d[:, None]), -7, 7).astype(np.int8)
    to_even = np.clip(np.rint((v * (np.float32(1) / d)[:, None]).astype(np.float64)), -7, 7).astype(np.int8)
    m, k = x.shape
    assert not np.array_equal(tw.pack_nibbles(by_division, m, k), c)
    assert not np.array_equal(tw.pack_nibbles(to_even, m, k), c)
