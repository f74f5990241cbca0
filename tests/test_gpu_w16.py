"""GPU parity of rotated W4A16 (reading R10) against the CPU oracle: the
rotated fp16 activations and the fp16-dequantised weights bit-exact in the
documented tiled layout (with its zero padding), the fp16 matrix-core GEMM on them within max|err| <=
2e-3 * max|ref| per row, and its place between W4A4 and the exact product."""
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
    print(f"[gpu w16] {msg}", flush=True)


def nbp(k):
    return (k // 32 + 7) // 8 * 8


def untile(buf, rows, k):
    """The documented tiled layout, [tile][block][half][lane group][row][8],
    back to a padded row-major [ceil(rows/32)*32, nbp*32] array."""
    tiles = (rows + 31) // 32
    a = np.asarray(buf).reshape(tiles, nbp(k), 2, 2, 32, 8).transpose(0, 4, 1, 2, 3, 5)
    return a.reshape(tiles * 32, nbp(k) * 32)


def bits(a):
    return np.ascontiguousarray(a).view(np.uint16)


def assert_rows_close(y, ref, what):
    ref = ref.astype(np.float64)
    err = np.abs(y.astype(np.float64) - ref).max(axis=1)
    bound = TOL * np.abs(ref).max(axis=1)
    assert (err <= bound).all(), f"{what}: worst row err {err.max():.3e}"


@pytest.mark.parametrize("m,k,dtype,pad", [(64, 256, np.float32, 0), (512, 5120, np.float16, 0),
                                           (33, 96, np.float16, 8), (7, 2208, np.float32, 32),
                                           (1, 32, np.float16, 0), (45, 320, np.float16, 1)])
def test_rotate_act16_bit_exact_and_padded(ops, m, k, dtype, pad):
    rng = np.random.default_rng(7 * m + k + pad)
    x = synth.activations(m, k + pad, rng, max(1, k // 100)).astype(dtype)
    say(f"rotate_act16 m={m} k={k} {np.dtype(dtype).name} ldx={k + pad}")
    a16 = untile(host(ops.rotate_act16(dev(x), k=k)), m, k)
    assert np.array_equal(bits(a16[:m, :k]), bits(oracle.rotate_act16(x, k=k)))
    assert not bits(a16[:, k:]).any() and not bits(a16[m:]).any()


def test_rotate_act16_special_blocks(ops):
    x = np.zeros((4, 128), np.float32)
    x[1, :32] = 1e-44            # subnormal input
    x[2, 32:64] = -3.0           # constant block: one non-zero output
    x[3, 70] = 4.0e5             # beyond fp16 after the rotation: +-inf on both sides
    a16 = untile(host(ops.rotate_act16(dev(x))), 4, 128)
    assert np.array_equal(bits(a16[:4, :128]), bits(oracle.rotate_act16(x)))


@pytest.mark.parametrize("n,k", [(64, 256), (33, 96), (300, 2208), (1, 32)])
def test_dequantize_w16_bit_exact_and_padded(ops, n, k):
    rng = np.random.default_rng(n + 3 * k)
    q4 = oracle.prepare_weights(synth.weights(n, k, rng))
    say(f"dequantize_w16 n={n} k={k}")
    w16 = untile(host(ops.dequantize_w16(dev(q4), n, k)), n, k)
    assert np.array_equal(bits(w16[:n, :k]), bits(oracle.dequantize_w16(q4, k)))
    assert not bits(w16[:, k:]).any() and not bits(w16[n:]).any()


def _problem(m, n, k, seed):
    rng = np.random.default_rng(seed)
    return synth.weights(n, k, rng), synth.activations(m, k, rng, max(1, k // 100))


@pytest.mark.parametrize("m,n,k", [(1, 1, 32), (33, 65, 96), (130, 300, 320), (257, 129, 2208),
                                   (128, 128, 256), (64, 1100, 512), (17, 4096, 5120)])
def test_gemm_w16_matches_oracle(ops, m, n, k):
    w, x = _problem(m, n, k, 11 * m + n + k)
    say(f"gemm_w16 m={m} n={n} k={k}")
    q4 = oracle.prepare_weights(w)
    w16 = ops.dequantize_w16(dev(q4), n, k)
    a16 = ops.rotate_act16(dev(x))
    y = host(ops.gemm_w16(w16, a16, m, n, k))
    ref = oracle.gemm_w16(oracle.dequantize_w16(q4, k), oracle.rotate_act16(x))
    assert_rows_close(y, ref, "gemm_w16")


@pytest.mark.parametrize("m,n,k", [(128, 65600, 256), (200, 33000, 320)])
def test_gemm_w16_leftover_pieces(ops, m, n, k):
    """Slightly more than one round of 128 x 128 tiles on a 256-CU part (513
    and 516 tiles for 512 resident workgroups): the leftover tiles run as
    32 x 32 pieces, the last of them ragged in both directions."""
    w, x = _problem(m, n, k, m + n)
    say(f"gemm_w16 leftover pieces m={m} n={n} k={k}")
    q4 = oracle.prepare_weights(w)
    y = host(ops.gemm_w16(ops.dequantize_w16(dev(q4), n, k), ops.rotate_act16(dev(x)), m, n, k))
    ref = oracle.gemm_w16(oracle.dequantize_w16(q4, k), oracle.rotate_act16(x))
    assert_rows_close(y, ref, "gemm_w16 pieces")


def test_gemm_w16_weights_from_gpu_quantiser(ops):
    """The whole chain on the GPU: fp32 weights -> rotated Q4_0 -> fp16."""
    w, x = _problem(40, 96, 640, 5)
    q4 = ops.quantize_q4_0_h32(dev(w))
    w16 = untile(host(ops.dequantize_w16(q4, 96, 640)), 96, 640)
    assert np.array_equal(bits(w16[:96, :640]), bits(oracle.dequantize_w16(oracle.prepare_weights(w), 640)))


def test_gemm_w16_ffn_up_sampled_rows_and_accuracy(ops):
    """The FFN-up workload at full size, sampled rows; W4A16 sits closer to
    the unquantised product than W4A4 on the same weights."""
    d = synth.ffn_up()
    say("gemm_w16 ffn_up 512x5120x17408, sampled rows")
    q4 = oracle.prepare_weights(d.w)
    w16 = ops.dequantize_w16(dev(q4), d.n, d.k)
    a16 = ops.rotate_act16(dev(d.x))
    y = host(ops.gemm_w16(w16, a16, d.m, d.n, d.k))
    rows = np.array([0, 1, 77, 255, 256, 511])
    ref = oracle.gemm_w16(oracle.dequantize_w16(q4, d.k), oracle.rotate_act16(d.x[rows]))
    assert_rows_close(y[rows], ref, "ffn_up w16")
    packed = ops.repack_q4_0_h32(dev(q4), d.n, d.k)
    c4, s4 = ops.rotate_quantize_act(dev(d.x[rows]))
    y4 = host(ops.gemm(packed, c4, s4, d.n, d.k))
    exact = d.x[rows].astype(np.float64) @ d.w.astype(np.float64).T
    assert np.abs(y[rows] - exact).mean() < np.abs(y4 - exact).mean()


def test_gemm_w16_output_stride_and_degenerate(ops):
    w, x = _problem(20, 70, 64, 5)
    w16 = ops.dequantize_w16(dev(oracle.prepare_weights(w)), 70, 64)
    a16 = ops.rotate_act16(dev(x))
    ybig = torch.full((20, 100), 7.0, device="cuda")
    ops.gemm_w16(w16, a16, 20, 70, 64, y=ybig[:, :70])
    yb = host(ybig)
    assert (yb[:, 70:] == 7.0).all()
    assert np.array_equal(yb[:, :70], host(ops.gemm_w16(w16, a16, 20, 70, 64)))
    y0 = torch.full((3, 8), 5.0, device="cuda")
    ops.gemm_w16(w16, a16, 3, 8, 0, y=y0)  # k = 0: an empty sum
    assert not host(y0).any()
