"""GPU parity of the unrotated W4A4 ablation (reading R9) against the CPU
oracle: plain Q4_0 weights and unrotated int4 activation codes bit-exact, the
GEMM on them within max|err| <= 2e-3 * max|ref| per row, and the ablation's
direction (without the rotation the product lands further from the exact
fp64 product)."""
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
    print(f"[gpu ablation] {msg}", flush=True)


@pytest.mark.parametrize("m,k,dtype,pad", [(64, 256, np.float32, 0), (512, 5120, np.float16, 0),
                                           (33, 96, np.float16, 8), (7, 2208, np.float32, 32)])
def test_quantize_act_plain_bit_exact(ops, m, k, dtype, pad):
    rng = np.random.default_rng(3 * m + k)
    x = synth.activations(m, k + pad, rng, max(1, k // 100)).astype(dtype)
    say(f"quantize_act m={m} k={k} {np.dtype(dtype).name} ldx={k + pad}")
    c, s = ops.quantize_act(dev(x), k=k)
    rc, rs = oracle.quantize_act_plain(x, k=k)
    assert np.array_equal(host(c), rc)
    assert np.array_equal(host(s), rs)


def test_quantize_act_plain_special_blocks(ops):
    x = np.zeros((4, 128), np.float32)
    x[1, :32] = 1e-44          # subnormal block: zeros
    x[2, 32:64] = -3.0         # constant block: all -7
    x[3, 70] = 11.0            # one-hot block: one 7
    c, s = ops.quantize_act(dev(x))
    rc, rs = oracle.quantize_act_plain(x)
    assert np.array_equal(host(c), rc) and np.array_equal(host(s), rs)


@pytest.mark.parametrize("n,k,pad", [(64, 256, 0), (33, 96, 32), (300, 2208, 0)])
def test_quantize_q4_0_plain_bit_exact(ops, n, k, pad):
    rng = np.random.default_rng(n + k)
    w = synth.weights(n, k + pad, rng)
    say(f"quantize_q4_0 n={n} k={k} ldw={k + pad}")
    q = host(ops.quantize_q4_0(dev(w)[:, :k]))
    assert np.array_equal(q, oracle.q4_0_quantize(np.ascontiguousarray(w[:, :k])))


@pytest.mark.parametrize("m,n,k", [(16, 300, 2208), (5, 33, 96), (64, 256, 256), (130, 96, 320)])
def test_ablation_gemm_matches_oracle(ops, m, n, k):
    rng = np.random.default_rng(5 * m + n)
    w = synth.weights(n, k, rng)
    x = synth.activations(m, k, rng, max(1, k // 100))
    say(f"ablation gemm m={m} n={n} k={k}")
    packed = ops.prepare_weights_plain(dev(w))
    c, s = ops.quantize_act(dev(x))
    y = host(ops.gemm(packed, c, s, n, k))
    ref = oracle.gemm(oracle.prepare_weights_plain(w), *oracle.quantize_act_plain(x), k).astype(np.float64)
    err = np.abs(y.astype(np.float64) - ref).max(axis=1)
    assert (err <= TOL * np.abs(ref).max(axis=1)).all(), f"worst {err.max():.3e}"


def test_ablation_direction_on_the_gpu(ops):
    """Outlier data: the unrotated pair is further from the exact product."""
    d = synth.tiny()
    ref = d.x.astype(np.float64) @ d.w.astype(np.float64).T
    say("ablation direction, tiny workload")
    y_rot = host(ops.gemm(ops.prepare_weights(dev(d.w)), *ops.rotate_quantize_act(dev(d.x)), d.n, d.k))
    y_plain = host(ops.gemm(ops.prepare_weights_plain(dev(d.w)), *ops.quantize_act(dev(d.x)), d.n, d.k))
    assert np.abs(y_plain - ref).mean() > 1.3 * np.abs(y_rot - ref).mean()
