"""w4a4_gemm_noalloc (the library's fixed scratch instead of a caller
workspace) against w4a4_gemm on the same inputs, through the C ABI: identical
outputs on consecutive calls of decreasing size (the second call reuses the
scratch the first left behind), and within the tolerance of the CPU oracle on
sampled rows; a size whose workspace exceeds the scratch is refused."""
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


def say(msg):
    print(f"[gpu] {msg}", flush=True)


def problem(m, n, k, seed):
    rng = np.random.default_rng(seed)
    return synth.weights(n, k, rng), synth.activations(m, k, rng, max(1, k // 100))


def run_pair(ops, m, n, k, seed, rows):
    w, x = problem(m, n, k, seed)
    dev = torch.device("cuda")
    packed = ops.prepare_weights(torch.from_numpy(w).to(dev))
    codes, scales = ops.rotate_quantize_act(torch.from_numpy(x).to(dev))
    need = ops.gemm_workspace_bytes(m, n, k)
    say(f"noalloc m={m} n={n} k={k} (workspace {need} bytes of {ops.lib().w4a4_gemm_noalloc_scratch_bytes()})")
    y_ref = ops.gemm(packed, codes, scales, n, k)
    y = ops.gemm_noalloc(packed, codes, scales, n, k)
    torch.cuda.synchronize()
    y, y_ref = y.cpu().numpy(), y_ref.cpu().numpy()
    assert np.array_equal(y, y_ref), "w4a4_gemm_noalloc differs from w4a4_gemm"
    q4 = oracle.prepare_weights(w)
    rc, rs = oracle.rotate_quantize_act(x[rows])
    ref = oracle.gemm(q4, rc, rs, k).astype(np.float64)
    err = np.abs(y[rows].astype(np.float64) - ref).max(axis=1)
    assert np.all(err <= TOL * np.abs(ref).max(axis=1))


def test_noalloc_matches_gemm_on_consecutive_calls(ops):
    # first call: m > 16 with the activation operand and split-K partial sums
    # in the scratch (down projection, 3 K splits); second: a smaller m > 16
    # product; third: m <= 16 with K split (partial sums in the scratch)
    run_pair(ops, 512, 5120, 17408, 1, rows=[0, 1, 255, 511])
    run_pair(ops, 100, 1000, 2048, 2, rows=list(range(0, 100, 9)))
    run_pair(ops, 16, 1024, 5120, 3, rows=list(range(16)))
    run_pair(ops, 5, 96, 64, 4, rows=list(range(5)))


def test_noalloc_refuses_a_workspace_past_the_scratch(ops):
    m, n, k = 16384, 32, 5120  # the activation operand alone is 80 MiB
    assert ops.gemm_workspace_bytes(m, n, k) > ops.lib().w4a4_gemm_noalloc_scratch_bytes()
    dev = torch.device("cuda")
    packed = torch.zeros(ops.packed_weight_bytes(n, k), dtype=torch.uint8, device=dev)
    codes = torch.zeros((m, k // 2), dtype=torch.uint8, device=dev)
    scales = torch.zeros((m, k // 32), dtype=torch.float32, device=dev)
    with pytest.raises(ops.W4A4Error, match="WORKSPACE_TOO_SMALL"):
        ops.gemm_noalloc(packed, codes, scales, n, k)
