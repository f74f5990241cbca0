"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Bars: bit-exact for the Q4_0 bytes, activation codes and scales, and for the
integer block sums (checked through the public ABI with unit and one-hot block
scales, where every fp32 partial sum is an exact integer); fp32 outputs within
max|err| <= 2e-3 * max|ref| per row.
"""
import numpy as np
import pytest

import oracle
from hadamard_rotated_w4a4_amd import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

TOL = 2e-3


@pytest.fixture(scope="module")
def ops():
    from hadamard_rotated_w4a4_amd import _lib
    _lib.lib()
    return _lib


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def say(msg):
    print(f"[gpu] {msg}", flush=True)


def assert_rows_close(y, ref, what=""):
    err = np.abs(y.astype(np.float64) - ref.astype(np.float64)).max(axis=-1)
    bound = TOL * np.abs(ref.astype(np.float64)).max(axis=-1)
    bad = np.nonzero(err > bound)
    assert bad[0].size == 0, (f"{what}: {bad[0].size} rows outside tolerance; worst err "
                              f"{err.max():.3e} vs bound {bound[np.argmax(err - bound)]:.3e}")


def with_unit_scales(q4):
    """Same codes, every weight scale fp16 1.0."""
    q = q4.copy()
    q[..., 0:2] = np.frombuffer(np.float16(1.0).tobytes(), np.uint8)
    return q


def with_one_hot_scales(q4, b0):
    q = q4.copy()
    q[..., 0:2] = 0
    q[..., b0, 0:2] = np.frombuffer(np.float16(1.0).tobytes(), np.uint8)
    return q


# --------------------------------------------------------------------------
# offline weight preparation: rotated Q4_0 bytes, bit-exact
# --------------------------------------------------------------------------

@pytest.mark.parametrize("n,k,pad", [(256, 256, 0), (33, 96, 0), (7, 32, 5), (1, 288, 32)])
def test_quantize_q4_0_h32_bit_exact(ops, n, k, pad):
    say(f"quantize_q4_0_h32 n={n} k={k} pad={pad}")
    w = synth.weights(n, k + pad, np.random.default_rng(n * 1000 + k))
    q4 = host(ops.quantize_q4_0_h32(dev(w)[:, :k]))
    assert np.array_equal(q4, oracle.prepare_weights(np.ascontiguousarray(w[:, :k])))


def test_quantize_q4_0_h32_ffn_up_full(ops):
    d = synth.ffn_up(m=1)
    say(f"quantize_q4_0_h32 full {d.n}x{d.k}")
    q4 = host(ops.quantize_q4_0_h32(dev(d.w)))
    assert np.array_equal(q4, oracle.prepare_weights(d.w))


def test_quantize_special_blocks(ops):
    w = np.zeros((6, 64), np.float32)
    w[1, :32] = 0.5            # constant block -> one nonzero rotated value
    w[2, 3] = -7.0             # one-hot
    w[3, :] = 1e-30            # tiny
    w[4, :] = np.linspace(-1, 1, 64)
    w[5, 32:] = 3e4
    say("quantize_q4_0_h32 special blocks")
    assert np.array_equal(host(ops.quantize_q4_0_h32(dev(w))), oracle.prepare_weights(w))


# --------------------------------------------------------------------------
# activation rotate + quantise: codes and scales bit-exact
# --------------------------------------------------------------------------

def test_rotate_quantize_tiny_fp32(ops):
    d = synth.tiny()
    say("rotate_quantize tiny fp32")
    c, s = ops.rotate_quantize_act(dev(d.x))
    rc, rs = oracle.rotate_quantize_act(d.x)
    assert np.array_equal(host(c), rc) and np.array_equal(host(s), rs)


def test_rotate_quantize_ffn_up_fp16(ops):
    d = synth.ffn_up()
    say("rotate_quantize 512x5120 fp16")
    c, s = ops.rotate_quantize_act(dev(d.x))
    rc, rs = oracle.rotate_quantize_act(d.x)
    assert np.array_equal(host(c), rc) and np.array_equal(host(s), rs)


@pytest.mark.parametrize("dtype", [np.float16, np.float32])
def test_rotate_quantize_strided_and_ragged(ops, dtype):
    rng = np.random.default_rng(21)
    x = (rng.standard_normal((7, 160)) * 3).astype(dtype)
    say(f"rotate_quantize strided {dtype.__name__}")
    c, s = ops.rotate_quantize_act(dev(x), k=96)
    rc, rs = oracle.rotate_quantize_act(x, k=96)
    assert np.array_equal(host(c), rc) and np.array_equal(host(s), rs)


def test_rotate_quantize_edge_blocks(ops):
    rng = np.random.default_rng(22)
    x = np.zeros((8, 128), np.float32)
    x[1] = 1e-44                                     # subnormal: zero block
    x[2, :32] = 0.37                                 # constant block
    x[3, 5] = -20.0                                  # one-hot outlier
    x[4] = rng.standard_normal(128) * 1e-30
    x[5] = rng.standard_normal(128) * 1e30
    v = np.zeros(32); v[:8] = [7, 2.5, -2.5, 0.5, -0.5, 3.5, -1.25, 6.5]  # exact ties
    import scipy.linalg
    x[6, :32] = (scipy.linalg.hadamard(32) @ v / 32).astype(np.float32)
    x[7] = rng.integers(-3, 4, 128).astype(np.float32) * 0.25  # many ties after scaling
    say("rotate_quantize edge blocks")
    c, s = ops.rotate_quantize_act(dev(x))
    rc, rs = oracle.rotate_quantize_act(x)
    assert np.array_equal(host(c), rc) and np.array_equal(host(s), rs)


def test_rotate_quantize_many_random_blocks(ops):
    rng = np.random.default_rng(23)
    x = (rng.standard_normal((256, 4096)) * rng.uniform(0.01, 100, (256, 1))).astype(np.float16)
    x[:, rng.choice(4096, 41, replace=False)] *= np.float16(20)
    say("rotate_quantize 1M elements fp16")
    c, s = ops.rotate_quantize_act(dev(x))
    rc, rs = oracle.rotate_quantize_act(x)
    assert np.array_equal(host(c), rc) and np.array_equal(host(s), rs)


@pytest.mark.parametrize("m,k,dtype", [(512, 5120, np.float16), (45, 288, np.float32), (33, 96, np.float16)])
def test_rotate_quantize_prepare_operand(ops, m, k, dtype):
    """The fused pass: codes and scales as the oracle's, and an operand equal
    byte for byte to the one prepare_act builds from the oracle's codes."""
    rng = np.random.default_rng(m + k)
    x = synth.activations(m, k, rng, max(1, k // 100), dtype=dtype)
    say(f"rotate_quantize_prepare m={m} k={k} {dtype.__name__}")
    act = torch.empty(ops.act_operand_bytes(m, k), dtype=torch.uint8, device="cuda")
    c, s = ops.rotate_quantize_prepare(dev(x), act)
    rc, rs = oracle.rotate_quantize_act(x)
    assert np.array_equal(host(c), rc) and np.array_equal(host(s), rs)
    ref = ops.prepare_act(dev(rc), dev(rs), k)
    assert np.array_equal(host(act), host(ref))


# --------------------------------------------------------------------------
# GEMM: integer block sums exact (fed the oracle's codes), fp32 within tolerance
# --------------------------------------------------------------------------

SHAPES = [(64, 256, 256), (1, 32, 32), (5, 33, 96), (16, 100, 288), (17, 64, 64),
          (33, 257, 160), (130, 96, 320), (300, 200, 128), (16, 1024, 5120),
          (7, 1024, 6176)]  # K past 5120 at m <= 16: 16 waves, 4 K splits, a ragged last record


def _problem(m, n, k, seed):
    rng = np.random.default_rng(seed)
    w = synth.weights(n, k, rng)
    x = synth.activations(m, k, rng, max(1, k // 100))
    return w, x


@pytest.mark.parametrize("m,n,k", SHAPES)
def test_gemm_integer_unit_scales(ops, m, n, k):
    w, x = _problem(m, n, k, m + n + k)
    q4 = with_unit_scales(oracle.prepare_weights(w))
    rc, _ = oracle.rotate_quantize_act(x)
    ones = np.ones((m, k // 32), np.float32)
    say(f"gemm integer unit scales m={m} n={n} k={k}")
    packed = ops.repack_q4_0_h32(dev(q4), n, k)
    y = host(ops.gemm(packed, dev(rc), dev(ones), n, k))
    ref = oracle.gemm(q4, rc, ones, k)  # = sum_b S, an exact integer
    assert np.array_equal(y, ref)


@pytest.mark.parametrize("m,n,k", [(64, 256, 256), (16, 100, 288), (130, 96, 320)])
def test_gemm_integer_one_hot_block(ops, m, n, k):
    w, x = _problem(m, n, k, 7 * m + n)
    q4 = oracle.prepare_weights(w)
    rc, _ = oracle.rotate_quantize_act(x)
    ones = np.ones((m, k // 32), np.float32)
    S = oracle.block_sums(q4, rc, k)
    for b0 in range(k // 32):
        say(f"gemm one-hot block {b0} m={m} n={n} k={k}")
        q = with_one_hot_scales(q4, b0)
        y = host(ops.gemm(ops.repack_q4_0_h32(dev(q), n, k), dev(rc), dev(ones), n, k))
        assert np.array_equal(y, S[:, :, b0].astype(np.float32))


@pytest.mark.parametrize("m,n,k", SHAPES)
def test_gemm_end_to_end(ops, m, n, k):
    w, x = _problem(m, n, k, 3 * m + n + k)
    say(f"gemm end-to-end m={m} n={n} k={k}")
    packed = ops.prepare_weights(dev(w))
    c, s = ops.rotate_quantize_act(dev(x))
    y = host(ops.gemm(packed, c, s, n, k))
    q4 = oracle.prepare_weights(w)
    rc, rs = oracle.rotate_quantize_act(x)
    assert np.array_equal(host(c), rc) and np.array_equal(host(s), rs)
    assert_rows_close(y, oracle.gemm(q4, rc, rs, k), f"m={m} n={n} k={k}")


@pytest.mark.parametrize("m,n,k", [(512, 17408, 256), (512, 16384, 256), (64, 4096, 160), (100, 600, 96)])
def test_gemm_tile_shapes_integer(ops, m, n, k):
    """Shapes that pick each workgroup tile (128x128, 128x64, 64x128): integer sums exact."""
    w, x = _problem(m, n, k, m + 3 * n)
    q4 = with_unit_scales(oracle.prepare_weights(w))
    rc, _ = oracle.rotate_quantize_act(x)
    ones = np.ones((m, k // 32), np.float32)
    say(f"gemm tile shapes, integer unit scales m={m} n={n} k={k}")
    y = host(ops.gemm(ops.repack_q4_0_h32(dev(q4), n, k), dev(rc), dev(ones), n, k))
    rows = np.unique(np.linspace(0, m - 1, 9).astype(int))
    assert np.array_equal(y[rows], oracle.gemm(q4, rc[rows], ones[rows], k))


def test_gemm_prepared_matches_gemm(ops):
    """One prepared activation feeding two products equals the one-call path bit for bit."""
    m, k = 200, 320
    rng = np.random.default_rng(31)
    x = synth.activations(m, k, rng, 3)
    w1, w2 = synth.weights(96, k, rng), synth.weights(160, k, rng)
    say("gemm_prepared vs gemm")
    c, s = ops.rotate_quantize_act(dev(x))
    p1, p2 = ops.prepare_weights(dev(w1)), ops.prepare_weights(dev(w2))
    act = ops.prepare_act(c, s, k)
    y1, y2 = host(ops.gemm_prepared(p1, act, m, 96, k)), host(ops.gemm_prepared(p2, act, m, 160, k))
    assert np.array_equal(y1, host(ops.gemm(p1, c, s, 96, k)))
    assert np.array_equal(y2, host(ops.gemm(p2, c, s, 160, k)))
    q4 = oracle.prepare_weights(w2)
    assert_rows_close(y2, oracle.gemm(q4, *oracle.rotate_quantize_act(x), k), "prepared")


def test_gemm_output_stride_and_determinism(ops):
    m, n, k = 40, 70, 128
    w, x = _problem(m, n, k, 5)
    packed = ops.prepare_weights(dev(w))
    c, s = ops.rotate_quantize_act(dev(x))
    say("gemm ldy > n, twice")
    ybig = torch.full((m, 100), 7.0, device="cuda")
    ops.gemm(packed, c, s, n, k, y=ybig[:, :n])
    y1 = host(ybig)
    assert np.all(y1[:, n:] == 7.0)  # columns past n untouched
    y2 = host(ops.gemm(packed, c, s, n, k))
    assert np.array_equal(y1[:, :n], y2)


def test_gemm_degenerate(ops):
    say("gemm m=0 and k=0")
    packed = torch.zeros(16, dtype=torch.uint8, device="cuda")
    codes = torch.zeros((0, 16), dtype=torch.uint8, device="cuda")
    scales = torch.zeros((0, 1), dtype=torch.float32, device="cuda")
    y = ops.gemm(packed, codes, scales, 8, 32)
    assert y.shape == (0, 8)
    codes = torch.zeros((3, 1), dtype=torch.uint8, device="cuda")
    scales = torch.zeros((3, 1), dtype=torch.float32, device="cuda")
    y = torch.full((3, 8), 5.0, device="cuda")
    ops.gemm(packed, codes, scales, 8, 0, y=y)
    assert not host(y).any()


# --------------------------------------------------------------------------
# full-size workloads, in the launch configuration the benchmark times
# --------------------------------------------------------------------------

def test_ffn_up_full_size_sampled_rows(ops):
    d = synth.ffn_up()
    say(f"{d.name}: full GEMM, sampled rows vs oracle")
    packed = ops.prepare_weights(dev(d.w))
    c, s = ops.rotate_quantize_act(dev(d.x))
    y = host(ops.gemm(packed, c, s, d.n, d.k))
    rc, rs = oracle.rotate_quantize_act(d.x)
    assert np.array_equal(host(c), rc) and np.array_equal(host(s), rs)
    q4 = oracle.prepare_weights(d.w)
    rows = np.array([0, 1, 127, 128, 255, 300, 383, 511])
    ref = oracle.gemm(q4, rc[rows], rs[rows], d.k)
    assert_rows_close(y[rows], ref, d.name)
    # integer sums of the same rows, fed the oracle's codes with unit scales
    q1 = with_unit_scales(q4)
    ones = np.ones_like(rs)
    yi = host(ops.gemm(ops.repack_q4_0_h32(dev(q1), d.n, d.k), dev(rc), dev(ones), d.n, d.k))
    assert np.array_equal(yi[rows], oracle.gemm(q1, rc[rows], ones[rows], d.k))


@pytest.mark.parametrize("name,k,n", synth.DENSE_PROJECTIONS)
def test_verify_block_m16_projection(ops, name, k, n):
    """16-token verify batch, each projection of the dense layer, all outputs."""
    w = synth.weights(n, k, synth.rng_for(0, 4, k + n))
    x = synth.activations(16, k, synth.rng_for(0, 4, 7 * k + n), synth.outlier_count(k))
    say(f"m=16 projection {name} {k}->{n}")
    packed = ops.prepare_weights(dev(w))
    c, s = ops.rotate_quantize_act(dev(x))
    y = host(ops.gemm(packed, c, s, n, k))
    q4 = oracle.prepare_weights(w)
    rc, rs = oracle.rotate_quantize_act(x)
    assert_rows_close(y, oracle.gemm(q4, rc, rs, k), name)


@pytest.mark.parametrize("m", [1, 2, 3, 8, 15, 16])
def test_small_m_ragged_rows(ops, m):
    k, n = 1024, 300
    w, x = _problem(m, n, k, 100 + m)
    say(f"small-m m={m}")
    packed = ops.prepare_weights(dev(w))
    c, s = ops.rotate_quantize_act(dev(x))
    y = host(ops.gemm(packed, c, s, n, k))
    assert_rows_close(y, oracle.gemm(oracle.prepare_weights(w), *oracle.rotate_quantize_act(x), k))


def test_small_m_split_k_shared_workspace(ops):
    """K-split small-m products on one workspace sized for the largest shape,
    shapes interleaved and repeated: every call equals a call on a fresh
    workspace bit for bit (the partial sums are added in a fixed order)."""
    import torch
    shapes = [(16, 1024, 5120), (7, 160, 2048), (16, 96, 17408), (3, 1024, 5120)]  # (m, n, k), all split
    need = max(ops.gemm_workspace_bytes(m, n, k) for m, n, k in shapes)
    ws = torch.full((need,), 0x7F, dtype=torch.uint8, device="cuda:0")  # stale contents are ignored
    probs = []
    for i, (m, n, k) in enumerate(shapes):
        w, x = _problem(m, n, k, 300 + i)
        packed = ops.prepare_weights(dev(w))
        c, s = ops.rotate_quantize_act(dev(x))
        fresh = host(ops.gemm(packed, c, s, n, k))
        assert_rows_close(fresh, oracle.gemm(oracle.prepare_weights(w), *oracle.rotate_quantize_act(x), k))
        probs.append((packed, c, s, n, k, fresh))
    for rep in range(2):
        for packed, c, s, n, k, fresh in probs:
            say(f"shared workspace rep {rep} m={c.shape[0]} n={n} k={k}")
            y = host(ops.gemm(packed, c, s, n, k, workspace=ws))
            assert np.array_equal(y, fresh)


def test_small_m_split_k_random_workspace(ops):
    """The tiles' arrival words of a K split start from whatever the workspace
    holds: random bytes there give the same outputs as a fresh workspace, bit
    for bit, on this call and on the next ones (each call leaves the words at
    zero and tags them with its own ticket)."""
    import torch
    gen = torch.Generator(device="cpu").manual_seed(11)
    for i, (m, n, k) in enumerate([(16, 1024, 5120), (5, 5120, 17408), (6, 1024, 6144)]):  # 8, 8, 16 waves
        need = ops.gemm_workspace_bytes(m, n, k)
        assert need > 0
        w, x = _problem(m, n, k, 400 + i)
        packed = ops.prepare_weights(dev(w))
        c, s = ops.rotate_quantize_act(dev(x))
        fresh = host(ops.gemm(packed, c, s, n, k))
        ws = torch.randint(0, 256, (need,), dtype=torch.uint8, generator=gen).to("cuda:0")
        for rep in range(3):
            say(f"random workspace m={m} n={n} k={k} rep {rep}")
            y = host(ops.gemm(packed, c, s, n, k, workspace=ws))
            assert np.array_equal(y, fresh)
        # the arrival words are back at zero after every call
        words = ws[: (n + 31) // 32 * 8].cpu().numpy()
        assert not words.any()


def test_last_microbatch_302_rows(ops):
    k, n = 6144, 5120  # the output projection
    w = synth.weights(n, k, synth.rng_for(0, 3, 3))
    x = synth.layer_inputs(302, microbatch=3)["attn_out"]
    say("m=302 o-proj 6144->5120, sampled rows")
    packed = ops.prepare_weights(dev(w))
    c, s = ops.rotate_quantize_act(dev(x))
    y = host(ops.gemm(packed, c, s, n, k))
    rows = np.array([0, 31, 32, 150, 255, 256, 290, 301])
    rc, rs = oracle.rotate_quantize_act(x)
    assert_rows_close(y[rows], oracle.gemm(oracle.prepare_weights(w), rc[rows], rs[rows], k))


def test_down_projection_m512_k17408_sampled_rows(ops):
    """The longest K of the layer (17408 = 544 blocks) at M = 512 on the
    matrix-core path, rows sampled across all four row tiles."""
    k, n = 17408, 5120
    w = synth.weights(n, k, synth.rng_for(0, 3, 6))
    x = synth.layer_inputs(512, microbatch=0)["ffn_act"]
    say("m=512 down 17408->5120, sampled rows")
    packed = ops.prepare_weights(dev(w))
    c, s = ops.rotate_quantize_act(dev(x))
    y = host(ops.gemm(packed, c, s, n, k))
    rows = np.array([0, 127, 128, 300, 383, 511])
    rc, rs = oracle.rotate_quantize_act(x)
    assert_rows_close(y[rows], oracle.gemm(oracle.prepare_weights(w), rc[rows], rs[rows], k), "down m512")


@pytest.mark.parametrize("m,k,name", [(512, 6144, "o"), (512, 17408, "down"), (302, 17408, "down302")])
def test_split_k_whole_tiles_sampled_rows(ops, m, k, name):
    """Products with few 128 x 128 tiles and a long K (the layer's o and down
    projections, N = 5120) split K over whole tiles; the partial sums are
    added in ascending split order, so repeated calls agree bit for bit."""
    n = 5120
    assert ops.gemm_prepared_workspace_bytes(m, n, k) > 0
    rng = np.random.default_rng(m + k)
    w = synth.weights(n, k, rng)
    x = synth.activations(m, k, rng, k // 100)
    say(f"split K {name} m={m} n={n} k={k}, sampled rows")
    packed = ops.prepare_weights(dev(w))
    c, s = ops.rotate_quantize_act(dev(x))
    ws = torch.empty(ops.gemm_workspace_bytes(m, n, k), dtype=torch.uint8, device="cuda")
    y = host(ops.gemm(packed, c, s, n, k, workspace=ws))
    assert np.array_equal(y, host(ops.gemm(packed, c, s, n, k, workspace=ws)))
    rows = np.array([0, 127, 128, m // 2, m - 1])
    rc, rs = oracle.rotate_quantize_act(x[rows])
    assert_rows_close(y[rows], oracle.gemm(oracle.prepare_weights(w), rc, rs, k), name)


def test_split_k_whole_tiles_random_workspace(ops):
    """Split K over whole tiles (the o projection, M = 512: 40 tiles) on a
    workspace of random bytes: every call equals one on a fresh workspace bit
    for bit."""
    import torch
    m, n, k = 512, 5120, 6144
    need = ops.gemm_workspace_bytes(m, n, k)
    assert ops.gemm_prepared_workspace_bytes(m, n, k) > 0
    rng = np.random.default_rng(21)
    w = synth.weights(n, k, rng)
    x = synth.activations(m, k, rng, k // 100)
    packed = ops.prepare_weights(dev(w))
    c, s = ops.rotate_quantize_act(dev(x))
    fresh = host(ops.gemm(packed, c, s, n, k))
    gen = torch.Generator(device="cpu").manual_seed(12)
    ws = torch.randint(0, 256, (need,), dtype=torch.uint8, generator=gen).to("cuda:0")
    for rep in range(3):
        say(f"split K random workspace m={m} n={n} k={k} rep {rep}")
        assert np.array_equal(host(ops.gemm(packed, c, s, n, k, workspace=ws)), fresh)


def test_split_k_many_splits_small_m(ops):
    """m = 100, n = 1000 (8 tiles), K = 32768: 16 splits of 16 stage pairs;
    sampled rows against the oracle, and exact integer sums with unit scales."""
    m, n, k = 100, 1000, 32768
    assert ops.gemm_prepared_workspace_bytes(m, n, k) == 16 * m * n * 4
    w, x = _problem(m, n, k, 5)
    say(f"split K x16 m={m} n={n} k={k}")
    q4 = oracle.prepare_weights(w)
    c, s = ops.rotate_quantize_act(dev(x))
    y = host(ops.gemm(ops.repack_q4_0_h32(dev(q4), n, k), c, s, n, k))
    rows = np.array([0, 31, 32, 99])
    rc, rs = oracle.rotate_quantize_act(x[rows])
    assert_rows_close(y[rows], oracle.gemm(q4, rc, rs, k), "split x16")
    qu = with_unit_scales(q4)
    ones = np.ones((m, k // 32), np.float32)
    yu = host(ops.gemm(ops.repack_q4_0_h32(dev(qu), n, k), c, dev(ones), n, k))
    assert np.array_equal(yu[rows], oracle.gemm(qu, host(c)[rows], ones[rows], k))


def test_split_k_integer_unit_scales(ops):
    """Split K with unit scales: every partial sum is an exact integer, so
    the product equals the oracle's integer sums exactly."""
    m, n, k = 512, 5120, 17408
    w, x = _problem(m, n, k, 99)
    q4 = with_unit_scales(oracle.prepare_weights(w))
    rc, _ = oracle.rotate_quantize_act(x)
    ones = np.ones((m, k // 32), np.float32)
    say(f"split K integer unit scales m={m} n={n} k={k}")
    y = host(ops.gemm(ops.repack_q4_0_h32(dev(q4), n, k), dev(rc), dev(ones), n, k))
    rows = np.array([0, 200, 511])
    assert np.array_equal(y[rows], oracle.gemm(q4, rc[rows], ones[rows], k))


def test_gate_up_packed_side_by_side_sampled_rows(ops):
    """Gate and up packed as one 34816-column matrix (the layout the
    benchmark's fused figures use): more than two rounds of 128 x 128 tiles,
    the rest as pieces; each half equals the oracle on its own weights."""
    k, n = 5120, 17408
    wg = synth.weights(n, k, synth.rng_for(0, 3, 4))
    wu = synth.weights(n, k, synth.rng_for(0, 3, 5))
    x = synth.layer_inputs(512, microbatch=1)["ffn_in"]
    say("m=512 gate|up 5120->34816, sampled rows")
    packed = ops.prepare_weights(dev(np.concatenate([wg, wu])))
    c, s = ops.rotate_quantize_act(dev(x))
    y = host(ops.gemm(packed, c, s, 2 * n, k))
    rows = np.array([0, 200, 511])
    rc, rs = oracle.rotate_quantize_act(x)
    assert_rows_close(y[rows, :n], oracle.gemm(oracle.prepare_weights(wg), rc[rows], rs[rows], k), "gate half")
    assert_rows_close(y[rows, n:], oracle.gemm(oracle.prepare_weights(wu), rc[rows], rs[rows], k), "up half")


# --------------------------------------------------------------------------
# MUL_MAT_ID
# --------------------------------------------------------------------------

def _moe_small(seed, E=6, T=11, top_k=3, n=70, k=96, bad_ids=True):
    rng = np.random.default_rng(seed)
    we = [synth.weights(n, k, rng) for _ in range(E)]
    ids = np.stack([rng.choice(E, top_k, replace=False) for _ in range(T)]).astype(np.int32)
    if bad_ids:
        ids[2, 1] = E + 1
        ids[5, 0] = -3
    return we, ids, rng


@pytest.mark.parametrize("rows_per_token", [1, 3])
def test_gemm_id_small_end_to_end(ops, rows_per_token):
    E, T, top_k, n, k = 6, 11, 3, 70, 96
    we, ids, rng = _moe_small(1 + rows_per_token)
    x = synth.activations(T * rows_per_token, k, rng, 2)
    say(f"gemm_id small rows_per_token={rows_per_token}")
    packed = torch.cat([ops.prepare_weights(dev(w)) for w in we])
    c, s = ops.rotate_quantize_act(dev(x))
    y = host(ops.gemm_id(packed, E, c, s, rows_per_token, dev(ids), n, k))
    q4e = np.stack([oracle.prepare_weights(w) for w in we])
    rc, rs = oracle.rotate_quantize_act(x)
    ref = oracle.gemm_id(q4e, rc, rs, rows_per_token, ids, n, k)
    assert not y[2, 1].any() and not y[5, 0].any()
    assert_rows_close(y.reshape(-1, n), ref.reshape(-1, n), "gemm_id")


def test_gemm_id_route_once_for_several_products(ops):
    """One routing (w4a4_gemm_id_route) serves a gate-like product (one
    activation row per token) and a down-like one (one per slot); each equals
    w4a4_gemm_id bit for bit, invalid ids' rows included."""
    E, T, top_k, n, k = 6, 11, 3, 70, 96
    we, ids, rng = _moe_small(21)
    x1 = synth.activations(T, k, rng, 2)
    x3 = synth.activations(T * top_k, k, rng, 2)
    say("gemm_id route once, two products")
    packed = torch.cat([ops.prepare_weights(dev(w)) for w in we])
    c1, s1 = ops.rotate_quantize_act(dev(x1))
    c3, s3 = ops.rotate_quantize_act(dev(x3))
    idsd = dev(ids)
    ws = ops.gemm_id_route(idsd, E)
    y1 = torch.full((T, top_k, n), float("nan"), device="cuda")
    y3 = torch.full((T, top_k, n), float("nan"), device="cuda")
    ops.gemm_id_routed(packed, E, c1, s1, 1, T, top_k, n, k, ws, y=y1)
    ops.gemm_id_routed(packed, E, c3, s3, top_k, T, top_k, n, k, ws, y=y3)
    assert np.array_equal(host(y1), host(ops.gemm_id(packed, E, c1, s1, 1, idsd, n, k)))
    assert np.array_equal(host(y3), host(ops.gemm_id(packed, E, c3, s3, top_k, idsd, n, k)))
    assert not host(y1)[2, 1].any() and not host(y3)[5, 0].any()


def test_gemm_id_all_ids_invalid(ops):
    """No valid id at all: no work item, every output row zero."""
    E, T, top_k, n, k = 6, 5, 2, 70, 96
    we, _, rng = _moe_small(22)
    ids = np.full((T, top_k), E + 3, np.int32)
    ids[1, 0] = -1
    x = synth.activations(T, k, rng, 2)
    packed = torch.cat([ops.prepare_weights(dev(w)) for w in we])
    c, s = ops.rotate_quantize_act(dev(x))
    y = torch.full((T, top_k, n), float("nan"), device="cuda")
    ops.gemm_id(packed, E, c, s, 1, dev(ids), n, k, y=y)
    assert not host(y).any()


def test_gemm_id_integer_unit_scales(ops):
    E, T, top_k, n, k = 6, 11, 3, 70, 96
    we, ids, rng = _moe_small(9)
    x = synth.activations(T, k, rng, 2)
    q4e = np.stack([with_unit_scales(oracle.prepare_weights(w)) for w in we])
    rc, _ = oracle.rotate_quantize_act(x)
    ones = np.ones((T, k // 32), np.float32)
    say("gemm_id integer unit scales")
    packed = torch.cat([ops.repack_q4_0_h32(dev(q), n, k) for q in q4e])
    y = host(ops.gemm_id(packed, E, dev(rc), dev(ones), 1, dev(ids), n, k))
    assert np.array_equal(y, oracle.gemm_id(q4e, rc, ones, 1, ids, n, k))


def test_gemm_id_single_expert_equals_gemm(ops):
    """E = 1, top_k = 1 is the dense product: both paths meet the oracle's bar
    and give the same exact integer sums with unit scales (their fp32
    accumulation orders differ, so real scales are compared by tolerance)."""
    m, n, k = 50, 64, 128
    w, x = _problem(m, n, k, 77)
    say("gemm_id E=1 top_k=1 == gemm")
    packed = ops.prepare_weights(dev(w))
    c, s = ops.rotate_quantize_act(dev(x))
    ids = torch.zeros((m, 1), dtype=torch.int32, device="cuda")
    y1 = host(ops.gemm_id(packed, 1, c, s, 1, ids, n, k))[:, 0, :]
    y0 = host(ops.gemm(packed, c, s, n, k))
    ref = oracle.gemm(oracle.prepare_weights(w), *oracle.rotate_quantize_act(x), k)
    assert_rows_close(y0, ref, "gemm")
    assert_rows_close(y1, ref, "gemm_id")
    q1 = with_unit_scales(oracle.prepare_weights(w))
    rc, _ = oracle.rotate_quantize_act(x)
    ones = dev(np.ones((m, k // 32), np.float32))
    p1 = ops.repack_q4_0_h32(dev(q1), n, k)
    yi0 = host(ops.gemm(p1, dev(rc), ones, n, k))
    yi1 = host(ops.gemm_id(p1, 1, dev(rc), ones, 1, ids, n, k))[:, 0, :]
    assert np.array_equal(yi0, yi1)


@pytest.mark.parametrize("rows_per_token", [1, 2])
def test_gemm_id_long_k_ragged_tiles(ops, rows_per_token):
    """K over two staging chunks with a ragged last record (nb = 69), n over
    two column chunks with a ragged last tile (n = 300), an expert with
    several row tiles, one with none, and invalid ids."""
    E, T, top_k, n, k = 5, 40, 2, 300, 2208
    rng = np.random.default_rng(2208 + rows_per_token)
    we = [synth.weights(n, k, rng) for _ in range(E)]
    ids = np.where(rng.random((T, top_k)) < 0.7, 0, rng.integers(1, 4, (T, top_k))).astype(np.int32)
    ids[:, 1] = np.where(ids[:, 0] == ids[:, 1], (ids[:, 1] + 1) % 4, ids[:, 1])  # distinct per token; expert 4 unused
    ids[3, 0] = E
    x = synth.activations(T * rows_per_token, k, rng, synth.outlier_count(k))
    say(f"gemm_id long k rows_per_token={rows_per_token}: counts {np.bincount(ids[ids < E], minlength=E)}")
    packed = torch.cat([ops.prepare_weights(dev(w)) for w in we])
    c, s = ops.rotate_quantize_act(dev(x))
    y = host(ops.gemm_id(packed, E, c, s, rows_per_token, dev(ids), n, k))
    q4e = np.stack([oracle.prepare_weights(w) for w in we])
    rc, rs = oracle.rotate_quantize_act(x)
    ref = oracle.gemm_id(q4e, rc, rs, rows_per_token, ids, n, k)
    assert not y[3, 0].any()
    assert_rows_close(y.reshape(-1, n), ref.reshape(-1, n), "gemm_id long k")


def _heavy_ids(T, E):
    """Slot 0: expert 0 for tokens 0..199 (200 rows), expert 2 after; slot 1:
    expert 1 for tokens 0..129 (129 rows after one invalid id), expert 4 for
    127 tokens, expert 3 after.  No token repeats an expert."""
    ids = np.zeros((T, 2), np.int32)
    ids[200:, 0] = 2
    ids[:130, 1] = 1
    ids[130:257, 1] = 4
    ids[257:, 1] = 3
    ids[5, 1] = E  # invalid
    return ids


@pytest.mark.parametrize("rows_per_token", [1, 2])
def test_gemm_id_popular_experts_ragged(ops, rows_per_token):
    """Experts with hundreds of rows (200 and 129: whole 32-row tiles plus a
    ragged one, over one column chunk and two staging passes of K) beside
    experts with fewer, one invalid id among a popular expert's tokens:
    against the oracle, and exact integer sums with unit scales."""
    E, T, top_k, n, k = 5, 300, 2, 200, 1344
    rng = np.random.default_rng(1344 + rows_per_token)
    we = [synth.weights(n, k, rng) for _ in range(E)]
    ids = _heavy_ids(T, E)
    counts = np.bincount(ids[ids < E], minlength=E)
    assert counts[0] == 200 and counts[1] == 129 and counts[4] == 127
    x = synth.activations(T * rows_per_token, k, rng, synth.outlier_count(k))
    say(f"gemm_id popular experts rows_per_token={rows_per_token}: counts {counts}")
    packed = torch.cat([ops.prepare_weights(dev(w)) for w in we])
    c, s = ops.rotate_quantize_act(dev(x))
    idsd = dev(ids)
    y = host(ops.gemm_id(packed, E, c, s, rows_per_token, idsd, n, k))
    q4e = np.stack([oracle.prepare_weights(w) for w in we])
    rc, rs = oracle.rotate_quantize_act(x)
    ref = oracle.gemm_id(q4e, rc, rs, rows_per_token, ids, n, k)
    assert not y[5, 1].any()
    assert_rows_close(y.reshape(-1, n), ref.reshape(-1, n), "popular experts")
    q1 = np.stack([with_unit_scales(q) for q in q4e])
    p1 = torch.cat([ops.repack_q4_0_h32(dev(q), n, k) for q in q1])
    ones = np.ones_like(rs)
    yi = host(ops.gemm_id(p1, E, dev(rc), dev(ones), rows_per_token, idsd, n, k))
    assert np.array_equal(yi, oracle.gemm_id(q1, rc, ones, rows_per_token, ids, n, k))


@pytest.mark.parametrize("which", ["gate", "down"])
def test_gemm_id_moe_full_size_sampled(ops, which):
    mo = synth.moe()
    T, top_k, E = mo.ids.shape[0], mo.ids.shape[1], mo.w_gate.shape[0]
    if which == "gate":
        w, x, rpt, n, k = mo.w_gate, mo.x, 1, synth.MOE_D_FF, synth.MOE_D_MODEL
    else:
        w, x, rpt, n, k = mo.w_down, mo.h, top_k, synth.MOE_D_MODEL, synth.MOE_D_FF
    say(f"gemm_id MoE {which}: {E} experts, {T} tokens, top-{top_k}, {k}->{n}")
    packed = torch.cat([ops.prepare_weights(dev(w[e])) for e in range(E)])
    c, s = ops.rotate_quantize_act(dev(x))
    y = host(ops.gemm_id(packed, E, c, s, rpt, dev(mo.ids), n, k))
    toks = np.array([0, 1, 100, 511, 777, 1023])
    q4e = np.stack([oracle.prepare_weights(w[e]) for e in range(E)])
    rc, rs = oracle.rotate_quantize_act(x)
    if rpt == 1:
        ref = oracle.gemm_id(q4e, rc[toks], rs[toks], 1, mo.ids[toks], n, k)
    else:
        rows = (toks[:, None] * top_k + np.arange(top_k)[None]).reshape(-1)
        ref = oracle.gemm_id(q4e, rc[rows], rs[rows], top_k, mo.ids[toks], n, k)
    assert_rows_close(y[toks].reshape(-1, n), ref.reshape(-1, n), f"moe {which}")
