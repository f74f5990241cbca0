"""Seeded synthetic inputs for the W4A4 Q4_0-H32 matmul.

This module draws random numbers and nothing else: it holds none of the
method's arithmetic (no rotation, no quantisation).  Tests, the smoke check and
the benchmark all take their inputs from here, so the HIP path and the CPU
oracle always see the same numbers.

Recipe (one ``numpy.random.Generator`` per tensor, seeded with
``[seed, workload_id, tensor_index]``):

* weights: ``standard_normal(float32) * 0.02``, shape [n, k] (fp32, unrotated;
  the offline rotation and Q4_0 quantisation are the method's, not this
  module's);
* activations: ``standard_normal(float32)`` of shape [m, k]; a fixed set of
  outlier channels (columns, the same for every row, drawn without
  replacement) is multiplied by 20; then cast to fp16 (or kept fp32);
* MoE routing: expert popularity follows a Zipf(1.1) law over a seeded random
  ranking of the experts; each token picks ``top_k`` distinct experts with
  those probabilities.

Workload shapes: the dense 27B-class projection set (Q 5120->6144,
K/V 5120->1024, O 6144->5120, gate/up 5120->17408, down 17408->5120) at
micro-batches of 512 tokens (a 1,838-token prompt is 512+512+512+302), the
16-token speculative-verify block, and an MoE layer with 128 experts, top-8,
gate/up 2048->768 and down 768->2048 at a 1024-token micro-batch.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

WEIGHT_STD = 0.02
OUTLIER_GAIN = 20.0

# (name, k, n) of the dense decoder-layer projections
DENSE_PROJECTIONS = (
    ("q", 5120, 6144),
    ("k", 5120, 1024),
    ("v", 5120, 1024),
    ("o", 6144, 5120),
    ("gate", 5120, 17408),
    ("up", 5120, 17408),
    ("down", 17408, 5120),
)
# projections that read the same activation rows share one quantised input
DENSE_INPUT_OF = {"q": "attn_in", "k": "attn_in", "v": "attn_in", "o": "attn_out",
                  "gate": "ffn_in", "up": "ffn_in", "down": "ffn_act"}
PROMPT_MICROBATCHES = (512, 512, 512, 302)  # a 1,838-token prompt
VERIFY_ROWS = 16

MOE_EXPERTS = 128
MOE_TOP_K = 8
MOE_TOKENS = 1024
MOE_D_MODEL = 2048
MOE_D_FF = 768
MOE_ZIPF_S = 1.1


def rng_for(seed: int, workload: int, tensor: int) -> np.random.Generator:
    return np.random.default_rng([seed, workload, tensor])


def weights(n: int, k: int, rng: np.random.Generator) -> np.ndarray:
    """fp32 [n, k] ~ N(0, 0.02^2), unrotated."""
    w = rng.standard_normal((n, k), dtype=np.float32)
    w *= np.float32(WEIGHT_STD)
    return w


def outlier_count(k: int, tiny: bool = False) -> int:
    return 2 if tiny else int(round(0.01 * k))


def activations(m: int, k: int, rng: np.random.Generator, n_outliers: int,
                dtype=np.float16) -> np.ndarray:
    """[m, k] ~ N(0, 1) with n_outliers channels scaled by 20, cast to dtype."""
    x = rng.standard_normal((m, k), dtype=np.float32)
    if n_outliers:
        cols = rng.choice(k, size=n_outliers, replace=False)
        x[:, cols] *= np.float32(OUTLIER_GAIN)
    return x.astype(dtype)


def zipf_ids(n_tokens: int, n_expert: int, top_k: int, rng: np.random.Generator,
             s: float = MOE_ZIPF_S) -> np.ndarray:
    """int32 [n_tokens, top_k]: distinct experts per token, Zipf(s)-skewed."""
    ranks = rng.permutation(n_expert) + 1
    p = ranks.astype(np.float64) ** (-s)
    p /= p.sum()
    ids = np.empty((n_tokens, top_k), np.int32)
    for t in range(n_tokens):
        ids[t] = rng.choice(n_expert, size=top_k, replace=False, p=p)
    return ids


# --------------------------------------------------------------------------
# the named workloads
# --------------------------------------------------------------------------

@dataclass
class Dense:
    """One dense W4A4 problem: y[m, n] = x[m, k] (rotated, quantised) . W[n, k]."""
    name: str
    w: np.ndarray  # fp32 [n, k], unrotated
    x: np.ndarray  # fp16/fp32 [m, k]

    @property
    def m(self):
        return self.x.shape[0]

    @property
    def n(self):
        return self.w.shape[0]

    @property
    def k(self):
        return self.w.shape[1]


def tiny(seed: int = 0) -> Dense:
    """M=64, K=N=256; fp32 activations with 2 outlier channels."""
    k, n, m = 256, 256, 64
    w = weights(n, k, rng_for(seed, 1, 0))
    x = activations(m, k, rng_for(seed, 1, 1), outlier_count(k, tiny=True), np.float32)
    return Dense("tiny_m64_k256_n256", w, x)


def ffn_up(seed: int = 0, m: int = 512) -> Dense:
    """Dense 27B-class FFN up projection: M=512, K=5120, N=17408, fp16 activations."""
    k, n = 5120, 17408
    w = weights(n, k, rng_for(seed, 2, 0))
    x = activations(m, k, rng_for(seed, 2, 1), outlier_count(k))
    return Dense(f"ffn_up_m{m}_k{k}_n{n}", w, x)


def layer_weights(seed: int = 0, workload: int = 3) -> dict:
    """fp32 weights of the seven dense projections, keyed by name."""
    return {name: weights(n, k, rng_for(seed, workload, i))
            for i, (name, k, n) in enumerate(DENSE_PROJECTIONS)}


def layer_inputs(m: int, seed: int = 0, workload: int = 3, microbatch: int = 0) -> dict:
    """fp16 activations of the four distinct projection inputs for one micro-batch."""
    ks = {"attn_in": 5120, "attn_out": 6144, "ffn_in": 5120, "ffn_act": 17408}
    out = {}
    for j, (name, k) in enumerate(ks.items()):
        rng = rng_for(seed, workload, 100 + 10 * microbatch + j)
        out[name] = activations(m, k, rng, outlier_count(k))
    return out


@dataclass
class MoE:
    w_gate: np.ndarray  # fp32 [E, d_ff, d_model]
    w_up: np.ndarray    # fp32 [E, d_ff, d_model]
    w_down: np.ndarray  # fp32 [E, d_model, d_ff]
    x: np.ndarray       # fp16 [T, d_model]  (gate/up input, one row per token)
    h: np.ndarray       # fp16 [T*top_k, d_ff]  (down input, one row per slot)
    ids: np.ndarray     # int32 [T, top_k]


def moe(seed: int = 0, n_tokens: int = MOE_TOKENS, n_expert: int = MOE_EXPERTS,
        top_k: int = MOE_TOP_K, d_model: int = MOE_D_MODEL, d_ff: int = MOE_D_FF,
        with_weights: bool = True) -> MoE:
    ids = zipf_ids(n_tokens, n_expert, top_k, rng_for(seed, 5, 0))
    x = activations(n_tokens, d_model, rng_for(seed, 5, 1), outlier_count(d_model))
    h = activations(n_tokens * top_k, d_ff, rng_for(seed, 5, 2), outlier_count(d_ff))
    if with_weights:
        wg = np.stack([weights(d_ff, d_model, rng_for(seed, 5, 1000 + e)) for e in range(n_expert)])
        wu = np.stack([weights(d_ff, d_model, rng_for(seed, 5, 2000 + e)) for e in range(n_expert)])
        wd = np.stack([weights(d_model, d_ff, rng_for(seed, 5, 3000 + e)) for e in range(n_expert)])
    else:
        wg = wu = wd = None
    return MoE(wg, wu, wd, x, h, ids)
