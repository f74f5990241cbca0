"""HIP graph capture of the hot path.  Every entry point only enqueues
kernels on the caller's stream (no allocation, memset or synchronisation),
so a captured step replays.  Each test captures one step, then replays it
several times on new inputs, with eager work and synchronisations between
the replays, and requires every replay to equal the eager result bit for
bit (the kernels sum in a fixed order)."""
import numpy as np
import pytest

from hadamard_rotated_w4a4_amd import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ops():
    from hadamard_rotated_w4a4_amd import _lib
    _lib.lib()
    return _lib


def say(msg):
    print(f"[gpu graph] {msg}", flush=True)


def replay_matches_eager(step, x, inputs, outs):
    """Eager results of `step` for each input, then one captured step
    replayed on the same inputs; every replay equals its eager result."""
    eager = []
    for xi in inputs:
        x.copy_(xi)
        step()
        torch.cuda.synchronize()
        eager.append([o.clone() for o in outs])
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        step()
    torch.cuda.synchronize()
    for rep in range(2):
        for i, xi in enumerate(inputs):
            for o in outs:
                o.fill_(float("nan")) if o.is_floating_point() else o.fill_(0)
            x.copy_(xi)                              # eager work between replays
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            for o, e in zip(outs, eager[i]):
                assert torch.equal(o, e), f"replay {rep} input {i}"


def _inputs(m, k, seed, count=3):
    rng = np.random.default_rng(seed)
    return [torch.from_numpy(synth.activations(m, k, rng, max(1, k // 100))).cuda() for _ in range(count)]


def test_dense_step_replays(ops):
    m, n, k = 200, 1000, 1024
    say(f"graph: rotate-quantise-prepare + gemm_prepared m={m} n={n} k={k}")
    rng = np.random.default_rng(1)
    packed = ops.prepare_weights(torch.from_numpy(synth.weights(n, k, rng)).cuda())
    inputs = _inputs(m, k, 2)
    x = torch.empty_like(inputs[0])
    codes = torch.empty((m, k // 2), dtype=torch.uint8, device="cuda")
    scales = torch.empty((m, k // 32), dtype=torch.float32, device="cuda")
    act = torch.empty(ops.act_operand_bytes(m, k), dtype=torch.uint8, device="cuda")
    y = torch.empty((m, n), dtype=torch.float32, device="cuda")

    def step():
        ops.rotate_quantize_prepare(x, act, codes=codes, scales=scales)
        ops.gemm_prepared(packed, act, m, n, k, y=y)
    replay_matches_eager(step, x, inputs, [codes, scales, y])


def test_dense_split_k_step_replays(ops):
    m, n, k = 512, 5120, 6144                   # few tiles, long K: split K and the reduction
    say(f"graph: rotate-quantise-prepare + split-K gemm_prepared m={m} n={n} k={k}")
    assert ops.gemm_prepared_workspace_bytes(m, n, k) > 0
    rng = np.random.default_rng(9)
    packed = ops.prepare_weights(torch.from_numpy(synth.weights(n, k, rng)).cuda())
    inputs = _inputs(m, k, 10, count=2)
    x = torch.empty_like(inputs[0])
    act = torch.empty(ops.act_operand_bytes(m, k), dtype=torch.uint8, device="cuda")
    ws = torch.empty(ops.gemm_prepared_workspace_bytes(m, n, k), dtype=torch.uint8, device="cuda")
    y = torch.empty((m, n), dtype=torch.float32, device="cuda")

    def step():
        ops.rotate_quantize_prepare(x, act)
        ops.gemm_prepared(packed, act, m, n, k, y=y, workspace=ws)
    replay_matches_eager(step, x, inputs, [y])


def test_small_m_split_k_step_replays(ops):
    m, n, k = 16, 1024, 5120                     # K split over many workgroups, then the reduction
    say(f"graph: rotate-quantise + small-M gemm (split K) m={m} n={n} k={k}")
    rng = np.random.default_rng(3)
    packed = ops.prepare_weights(torch.from_numpy(synth.weights(n, k, rng)).cuda())
    inputs = _inputs(m, k, 4)
    x = torch.empty_like(inputs[0])
    codes = torch.empty((m, k // 2), dtype=torch.uint8, device="cuda")
    scales = torch.empty((m, k // 32), dtype=torch.float32, device="cuda")
    ws = torch.empty(max(1, ops.gemm_workspace_bytes(m, n, k)), dtype=torch.uint8, device="cuda")
    assert ops.gemm_workspace_bytes(m, n, k) > 0
    y = torch.empty((m, n), dtype=torch.float32, device="cuda")

    def step():
        ops.rotate_quantize_act(x, codes=codes, scales=scales)
        ops.gemm(packed, codes, scales, n, k, y=y, workspace=ws)
    replay_matches_eager(step, x, inputs, [codes, scales, y])


def test_small_m_prepared_step_replays(ops):
    """The m <= 16 prepared path: the quantiser writes codes, scales and the
    record-ordered operand, then two products read the operand (one whole-K,
    one with K splits summed in the same launch)."""
    m, k = 13, 5120
    shapes = ((17408, "whole K"), (1024, "K split"))
    say(f"graph: rotate_quantize_prepare_small + gemm_prepared_small m={m} k={k}")
    rng = np.random.default_rng(5)
    packed = [ops.prepare_weights(torch.from_numpy(synth.weights(n, k, rng)).cuda()) for n, _ in shapes]
    inputs = _inputs(m, k, 6)
    x = torch.empty_like(inputs[0])
    codes = torch.empty((m, k // 2), dtype=torch.uint8, device="cuda")
    scales = torch.empty((m, k // 32), dtype=torch.float32, device="cuda")
    act = torch.empty(ops.small_act_operand_bytes(m, k), dtype=torch.uint8, device="cuda")
    ws = torch.empty(max(1, max(ops.gemm_workspace_bytes(m, n, k) for n, _ in shapes)), dtype=torch.uint8,
                     device="cuda")
    ys = [torch.empty((m, n), dtype=torch.float32, device="cuda") for n, _ in shapes]

    def step():
        ops.rotate_quantize_prepare_small(x, act, codes=codes, scales=scales)
        for (n, _), p, y in zip(shapes, packed, ys):
            ops.gemm_prepared_small(p, act, m, n, k, y=y, workspace=ws)
    replay_matches_eager(step, x, inputs, [codes, scales, act] + ys)


def test_mul_mat_id_step_replays(ops):
    e, t, top_k, n, k = 16, 64, 4, 256, 512
    say(f"graph: rotate-quantise + gemm_id E={e} T={t} top_k={top_k} n={n} k={k}")
    rng = np.random.default_rng(5)
    packed = torch.cat([ops.prepare_weights(torch.from_numpy(synth.weights(n, k, rng)).cuda()) for _ in range(e)])
    ids = torch.from_numpy(synth.zipf_ids(t, e, top_k, rng)).cuda()
    inputs = _inputs(t, k, 6)
    x = torch.empty_like(inputs[0])
    codes = torch.empty((t, k // 2), dtype=torch.uint8, device="cuda")
    scales = torch.empty((t, k // 32), dtype=torch.float32, device="cuda")
    ws = torch.empty(ops.gemm_id_workspace_bytes(e, t, top_k), dtype=torch.uint8, device="cuda")
    y = torch.empty((t, top_k, n), dtype=torch.float32, device="cuda")

    def step():
        ops.rotate_quantize_act(x, codes=codes, scales=scales)
        ops.gemm_id(packed, e, codes, scales, 1, ids, n, k, y=y, workspace=ws)
    replay_matches_eager(step, x, inputs, [codes, scales, y])


def test_w4a16_step_replays(ops):
    m, n, k = 130, 300, 640
    say(f"graph: rotate_act16 + gemm_w16 m={m} n={n} k={k}")
    rng = np.random.default_rng(7)
    w16 = ops.dequantize_w16(ops.quantize_q4_0_h32(torch.from_numpy(synth.weights(n, k, rng)).cuda()), n, k)
    inputs = _inputs(m, k, 8)
    x = torch.empty_like(inputs[0])
    a16 = ops.rotate_act16(inputs[0])
    y = torch.empty((m, n), dtype=torch.float32, device="cuda")

    def step():
        ops.rotate_act16(x, out=a16)
        ops.gemm_w16(w16, a16, m, n, k, y=y)
    replay_matches_eager(step, x, inputs, [a16, y])
