"""GPU parity of the W4A8-H32 path (int8 activation codes on a rotated file)
against the CPU oracle (reading R8).

Bars as for W4A4: activation codes and scales bit-exact; integer block sums
bit-exact through the public ABI with unit weight and activation scales;
fp32 outputs within max|err| <= 2e-3 * max|ref| per row.
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
    print(f"[gpu a8] {msg}", flush=True)


def assert_rows_close(y, ref, what=""):
    err = np.abs(y.astype(np.float64) - ref.astype(np.float64)).max(axis=-1)
    bound = TOL * np.abs(ref.astype(np.float64)).max(axis=-1)
    bad = np.nonzero(err > bound)
    assert bad[0].size == 0, f"{what}: {bad[0].size} rows outside tolerance; worst {err.max():.3e}"


def _problem(m, n, k, seed):
    rng = np.random.default_rng(seed)
    return synth.weights(n, k, rng), synth.activations(m, k, rng, max(1, k // 100))


@pytest.mark.parametrize("m,k,dtype,pad", [(64, 256, np.float32, 0), (512, 5120, np.float16, 0),
                                           (33, 96, np.float16, 8), (7, 2208, np.float32, 32)])
def test_rotate_quantize_act8_bit_exact(ops, m, k, dtype, pad):
    rng = np.random.default_rng(m + k)
    x = (synth.activations(m, k + pad, rng, max(1, k // 100))).astype(dtype)
    say(f"quantise8 m={m} k={k} {np.dtype(dtype).name} ldx={k + pad}")
    c, s = ops.rotate_quantize_act8(dev(x), k=k)
    rc, rs = oracle.rotate_quantize_act8(x, k=k)
    assert np.array_equal(host(c), rc)
    assert np.array_equal(host(s), rs)


def test_rotate_quantize_act8_special_blocks(ops):
    x = np.zeros((4, 128), np.float32)
    x[1, :32] = 1e-44          # subnormal block: zeros
    x[2, 32:64] = -3.0         # constant block
    x[3, 70] = 11.0            # one-hot block
    c, s = ops.rotate_quantize_act8(dev(x))
    rc, rs = oracle.rotate_quantize_act8(x)
    assert np.array_equal(host(c), rc) and np.array_equal(host(s), rs)


SHAPES = [(1, 32, 32), (5, 33, 96), (16, 100, 288), (16, 1024, 5120), (17, 64, 64),
          (40, 300, 2208), (130, 96, 320), (512, 256, 1024)]


@pytest.mark.parametrize("m,n,k", SHAPES)
def test_gemm_a8_integer_unit_scales(ops, m, n, k):
    """Unit weight and activation scales: every output is an exact integer sum
    of exact block sums, so the GPU must match the oracle bit for bit."""
    w, x = _problem(m, n, k, 7 * m + n)
    q4 = oracle.prepare_weights(w)
    q4[..., 0:2] = np.frombuffer(np.float16(1.0).tobytes(), np.uint8)
    rc, _ = oracle.rotate_quantize_act8(x)
    ones = np.ones((m, k // 32), np.float32)
    say(f"gemm_a8 unit scales m={m} n={n} k={k}")
    y = host(ops.gemm_a8(ops.repack_q4_0_h32(dev(q4), n, k), dev(rc), dev(ones), n, k))
    assert np.array_equal(y, oracle.gemm_a8(q4, rc, ones, k))


@pytest.mark.parametrize("m,n,k", SHAPES)
def test_gemm_a8_end_to_end(ops, m, n, k):
    w, x = _problem(m, n, k, 11 * m + n)
    say(f"gemm_a8 m={m} n={n} k={k}")
    packed = ops.prepare_weights(dev(w))
    c, s = ops.rotate_quantize_act8(dev(x))
    y = host(ops.gemm_a8(packed, c, s, n, k))
    ref = oracle.gemm_a8(oracle.prepare_weights(w), *oracle.rotate_quantize_act8(x), k)
    assert_rows_close(y, ref, "gemm_a8")


def test_gemm_a8_ffn_up_sampled_rows_and_accuracy(ops):
    """The FFN-up workload at full size, sampled rows; W4A8 sits much closer
    to the unquantised product than W4A4 does."""
    d = synth.ffn_up()
    say("gemm_a8 ffn_up 512x5120x17408, sampled rows")
    packed = ops.prepare_weights(dev(d.w))
    c, s = ops.rotate_quantize_act8(dev(d.x))
    y = host(ops.gemm_a8(packed, c, s, d.n, d.k))
    rows = np.array([0, 1, 77, 255, 256, 511])
    q4 = oracle.prepare_weights(d.w)
    rc, rs = oracle.rotate_quantize_act8(d.x[rows])
    ref = oracle.gemm_a8(q4, rc, rs, d.k)
    assert_rows_close(y[rows], ref, "ffn_up a8")
    c4, s4 = ops.rotate_quantize_act(dev(d.x[rows]))
    y4 = host(ops.gemm(packed, c4, s4, d.n, d.k))
    exact = d.x[rows].astype(np.float64) @ d.w.astype(np.float64).T
    assert np.abs(y[rows] - exact).mean() < np.abs(y4 - exact).mean()


def test_gemm_a8_output_stride_and_degenerate(ops):
    w, x = _problem(20, 70, 64, 5)
    packed = ops.prepare_weights(dev(w))
    c, s = ops.rotate_quantize_act8(dev(x))
    ybig = torch.full((20, 100), 7.0, device="cuda")
    ops.gemm_a8(packed, c, s, 70, 64, y=ybig[:, :70])
    yb = host(ybig)
    assert (yb[:, 70:] == 7.0).all()
    assert np.array_equal(yb[:, :70], host(ops.gemm_a8(packed, c, s, 70, 64)))
    y0 = torch.full((3, 8), 5.0, device="cuda")
    ops.gemm_a8(packed, c[:3], s[:3], 8, 0, y=y0)  # k = 0: an empty sum
    assert not host(y0).any()


@pytest.mark.parametrize("m,k,dtype,pad", [(5, 320, np.float32, 0), (17, 96, np.float32, 0),
                                           (130, 2208, np.float16, 0), (512, 5120, np.float16, 0),
                                           (33, 96, np.float16, 8), (40, 288, np.float32, 32)])
def test_rotate_quantize_prepare8_operand(ops, m, k, dtype, pad):
    """The fused quantiser's codes and scales equal the oracle's bit for bit
    (also from rows with a stride past k), and the operand it writes equals
    byte for byte the one gemm_a8's pre-pass builds in its workspace from
    those codes (over stale buffer contents)."""
    rng = np.random.default_rng(3 * m + k)
    x = synth.activations(m, k + pad, rng, max(1, k // 100)).astype(dtype)
    say(f"rotate_quantize_prepare8 m={m} k={k} {np.dtype(dtype).name} ldx={k + pad}")
    act = torch.full((ops.act8_operand_bytes(m, k),), 0xA5, dtype=torch.uint8, device="cuda")
    c, s = ops.rotate_quantize_prepare8(dev(x), act, k=k)
    rc, rs = oracle.rotate_quantize_act8(x, k=k)
    assert np.array_equal(host(c), rc) and np.array_equal(host(s), rs)
    if m > 16:
        n = 64
        packed = ops.prepare_weights(dev(synth.weights(n, k, rng)))
        ws = torch.full((int(ops.lib().w4a4_gemm_a8_workspace_bytes(m, n, k)),), 0x5A, dtype=torch.uint8,
                        device="cuda")
        ops.gemm_a8(packed, c, s, n, k, workspace=ws)
        torch.cuda.synchronize()
        assert ws.numel() >= act.numel() and torch.equal(ws[:act.numel()], act)


@pytest.mark.parametrize("m,n,k", SHAPES)
def test_gemm_a8_prepared(ops, m, n, k):
    """Above 16 rows gemm_a8 is the pre-pass plus this product, so the two
    agree bit for bit; at any m the result meets the oracle's bar."""
    w, x = _problem(m, n, k, 13 * m + n)
    say(f"gemm_a8_prepared m={m} n={n} k={k}")
    packed = ops.prepare_weights(dev(w))
    act = torch.empty(ops.act8_operand_bytes(m, k), dtype=torch.uint8, device="cuda")
    c, s = ops.rotate_quantize_prepare8(dev(x), act)
    y = host(ops.gemm_a8_prepared(packed, act, m, n, k))
    if m > 16:
        assert np.array_equal(y, host(ops.gemm_a8(packed, c, s, n, k)))
    ref = oracle.gemm_a8(oracle.prepare_weights(w), *oracle.rotate_quantize_act8(x), k)
    assert_rows_close(y, ref, "gemm_a8_prepared")


def test_gemm_a8_prepared_ffn_up_matches_gemm_a8(ops):
    d = synth.ffn_up()
    say("gemm_a8_prepared ffn_up 512x5120x17408 vs gemm_a8")
    packed = ops.prepare_weights(dev(d.w))
    xd = dev(d.x)
    act = torch.empty(ops.act8_operand_bytes(d.m, d.k), dtype=torch.uint8, device="cuda")
    c, s = ops.rotate_quantize_prepare8(xd, act)
    y = ops.gemm_a8_prepared(packed, act, d.m, d.n, d.k)
    assert torch.equal(y, ops.gemm_a8(packed, c, s, d.n, d.k))
    ybig = torch.full((d.m, d.n + 8), 3.0, device="cuda")
    ops.gemm_a8_prepared(packed, act, d.m, d.n, d.k, y=ybig[:, :d.n])
    assert torch.equal(ybig[:, :d.n], y) and bool((ybig[:, d.n:] == 3.0).all())
