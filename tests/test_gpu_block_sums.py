"""GPU integer parity at the full sizes, through every launch kind.

With every activation scale 1 and the weight scales one-hot (fp16 1.0 on
block b0, 0 elsewhere), each output is exactly the integer block dot
S[:, :, b0] (every partial sum is an integer below 2^24, in any order or
split), so the GPU's block dots are checked bit for bit, block by block, on
all rows and columns: swapped, dropped or misplaced blocks fail.  The kinds:
whole tiles plus K pieces of the leftover tiles (FFN up, M = 512), split K
over whole tiles (down projection, M = 512, K = 17408), the M <= 16
streaming kernel with and without K splits, and MUL_MAT_ID at 128 experts
with unit scales.  Also the q, k and v projections at M = 512 against the
oracle on sampled rows, in the launch plan the benchmark's layer set uses.
The method: 1bit-MONSTER engine docs, page "The lean option: ROCmFP4, ROCmI4
and Hadamard Q4_0", sections "Hadamard-rotated Q4_0: W4A4 prompt processing"
and "MoE: W4A4 on the experts".
"""
import numpy as np
import pytest

import oracle
from hadamard_rotated_w4a4_amd import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

TOL = 2e-3
F16_ONE = np.frombuffer(np.float16(1.0).tobytes(), np.uint8)


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


def one_hot(q4, b0):
    q = q4.copy()
    q[..., 0:2] = 0
    q[..., b0, 0:2] = F16_ONE
    return q


def block_dot(q4, codes, b):
    """S[:, :, b] from the oracle: the block-b slice as a K = 32 problem."""
    return oracle.block_sums(np.ascontiguousarray(q4[:, b:b + 1]),
                             np.ascontiguousarray(codes[:, 16 * b:16 * b + 16]), 32)[:, :, 0]


def sampled_blocks(nb):
    """Ends, middle, and both sides of the block boundaries where a product
    split three ways over pairs of 2-block stages changes split."""
    edges = {4 * ((nb // 4) * z // 3) for z in (1, 2)}
    return sorted({0, 1, nb // 2, nb - 2, nb - 1} | edges | {e - 1 for e in edges})


KINDS = [  # (name, m, n, k): each takes a different launch plan
    ("whole tiles + K pieces (FFN up)", 512, 17408, 5120),
    ("split K over whole tiles (down)", 512, 5120, 17408),
    ("m16 streaming, K split (down)", 16, 5120, 17408),
    ("m16 streaming, whole K (gate)", 16, 17408, 5120),
]


@pytest.mark.parametrize("name,m,n,k", KINDS, ids=[kd[0].split(" (")[0].replace(" ", "_") for kd in KINDS])
def test_one_hot_block_scales_every_output(ops, name, m, n, k):
    rng = np.random.default_rng(m + n + k)
    w = synth.weights(n, k, rng)
    x = synth.activations(m, k, rng, k // 100)
    q4 = oracle.prepare_weights(w)
    rc, _ = oracle.rotate_quantize_act(x)
    ones = dev(np.ones((m, k // 32), np.float32))
    codes = dev(rc)
    y = torch.empty((m, n), dtype=torch.float32, device="cuda")
    ws = torch.empty(max(1, ops.gemm_workspace_bytes(m, n, k)), dtype=torch.uint8, device="cuda")
    for b0 in sampled_blocks(k // 32):
        say(f"{name}: m={m} n={n} k={k}, one-hot block {b0}")
        packed = ops.repack_q4_0_h32(dev(one_hot(q4, b0)), n, k)
        ops.gemm(packed, codes, ones, n, k, y=y, workspace=ws)
        assert np.array_equal(host(y), block_dot(q4, rc, b0).astype(np.float32)), f"block {b0}"


@pytest.mark.parametrize("name", ["q", "k", "v"])
def test_qkv_m512_full_size(ops, name):
    """The attention-input projections at M = 512 (q: 192 tiles of 128 x 128,
    k and v: 32 tiles each, so whole tiles, pieces or split K as the plan
    picks): sampled rows against the oracle, and exact integer sums of the
    same rows with unit scales."""
    k, n = {nm: (kk, nn) for nm, kk, nn in synth.DENSE_PROJECTIONS}[name]
    idx = [nm for nm, _, _ in synth.DENSE_PROJECTIONS].index(name)
    w = synth.weights(n, k, synth.rng_for(0, 3, idx))
    x = synth.layer_inputs(512, microbatch=0)["attn_in"]
    say(f"m=512 {name} {k}->{n}, sampled rows")
    packed = ops.prepare_weights(dev(w))
    c, s = ops.rotate_quantize_act(dev(x))
    y = host(ops.gemm(packed, c, s, n, k))
    rows = np.array([0, 1, 127, 128, 255, 300, 383, 511])
    rc, rs = oracle.rotate_quantize_act(x)
    q4 = oracle.prepare_weights(w)
    ref = oracle.gemm(q4, rc[rows], rs[rows], k).astype(np.float64)
    err = np.abs(y[rows].astype(np.float64) - ref).max(axis=1)
    assert np.all(err <= TOL * np.abs(ref).max(axis=1)), name
    q1 = q4.copy()
    q1[..., 0:2] = F16_ONE
    ones = np.ones_like(rs)
    yi = host(ops.gemm(ops.repack_q4_0_h32(dev(q1), n, k), dev(rc), dev(ones), n, k))
    assert np.array_equal(yi[rows], oracle.gemm(q1, rc[rows], ones[rows], k))


@pytest.mark.parametrize("which", ["gate", "down"])
def test_gemm_id_128_experts_unit_scales(ops, which):
    """MUL_MAT_ID on the full MoE layer (1024 tokens, top-8 of 128 experts,
    Zipf-skewed routing) with unit scales: every output of the sampled tokens
    is the exact integer sum over blocks of the routed expert's block dots."""
    mo = synth.moe()
    T, top_k, E = mo.ids.shape[0], mo.ids.shape[1], mo.w_gate.shape[0]
    if which == "gate":
        w, x, rpt, n, k = mo.w_gate, mo.x, 1, synth.MOE_D_FF, synth.MOE_D_MODEL
    else:
        w, x, rpt, n, k = mo.w_down, mo.h, top_k, synth.MOE_D_MODEL, synth.MOE_D_FF
    say(f"gemm_id unit scales {which}: {E} experts, {T} tokens, top-{top_k}, {k}->{n}")
    q4e = np.stack([oracle.prepare_weights(w[e]) for e in range(E)])
    q4e[..., 0:2] = F16_ONE
    packed = torch.cat([ops.repack_q4_0_h32(dev(q4e[e]), n, k) for e in range(E)])
    rc, rs = oracle.rotate_quantize_act(x)
    ones = np.ones_like(rs)
    y = host(ops.gemm_id(packed, E, dev(rc), dev(ones), rpt, dev(mo.ids), n, k))
    toks = np.array([0, 1, 2, 100, 511, 512, 777, 1022, 1023])
    if rpt == 1:
        ref = oracle.gemm_id(q4e, rc[toks], ones[toks], 1, mo.ids[toks], n, k)
    else:
        rows = (toks[:, None] * top_k + np.arange(top_k)[None]).reshape(-1)
        ref = oracle.gemm_id(q4e, rc[rows], ones[rows], top_k, mo.ids[toks], n, k)
    assert np.array_equal(y[toks], ref)
