"""Benchmark of the W4A4 Q4_0-H32 hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-extras] [--no-cpu]

A step is one pass of the whole hot path over one batch: rotate + quantise the
activations of the 27B-class FFN up projection (M=512 tokens, K=5120, fp16)
and run the W4A4 GEMM against its H32-rotated Q4_0 weights (N=17408).  The
offline weight preparation (rotation, Q4_0, repack) happens before timing.
Weights rotate through copies totalling > 1 GB so the 256 MB last-level cache
cannot hold them across steps.

Prints ONE JSON line (stdout).  Besides the contract's fields it carries:
  roofline          the GEMM kernel's achieved int8-equivalent TOP/s (2*M*N*K
                    per launch over its median duration, from HIP events on
                    the launch stream around the GEMM of every 4th step of
                    the timed pass, the same pass as ms_per_step) against the 5.0 POP/s
                    dense int8 MFMA peak and against the int8 rate measured
                    in the same run; HBM traffic from rocprofv3 counters
                    recorded in profiles/ (null if the kernel source has
                    changed since they were taken);
  measured_ceilings a read stream over 2 GiB and the FP6 / int8 MFMA issue
                    rates, measured in this run (libw4a4_ceilings.so);
  cpu_baseline      the CPU oracle (test infrastructure) timed on a bounded
                    sample of the same workload on the host cores (and one
                    per extra workload, inside each extra);
  sclk_mhz          the shader clock reported before and after the run;
  extras            the 16-token verify set (GB/s vs 8 TB/s and vs the
                    measured read stream; per projection, the time of a plain
                    read of its weight bytes timed the same way), the MoE layer (MUL_MAT_ID, timed
                    cold), W4A8-H32, rotated W4A16, the unrotated ablation
                    and the dense layer set over a 1,838-token prompt.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_INT8_TOPS = 5000.0      # MI355X dense int8 MFMA, TOP/s
PEAK_FP6_TOPS = 10100.0      # MI355X dense FP6 / FP4 MFMA, TFLOP/s
PEAK_HBM_GBS = 8000.0        # MI355X HBM3E, GB/s
PEAK_FP16_TFLOPS = 2500.0    # MI355X dense fp16 / bf16 MFMA, TFLOP/s
COLD_BYTES = 1 << 30         # weight copies rotated per step exceed this
LLC_BYTES = 256 << 20        # MI355X last-level (Infinity) cache
PROFILE_JSON = os.path.join(ROOT, "profiles", "counters.json")
KERNEL_SOURCES = [os.path.join(ROOT, "hadamard_rotated_w4a4_amd", "csrc", f)
                  for f in ("common.h", "k_route.h", "k_dense.h", "k_smallm.h", "k_grouped.h", "k_rotq.h", "k_prep.h", "k_w16.h", "w4a4.hip")]


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def source_hash() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        h.update(open(p, "rb").read())
    return h.hexdigest()[:16]


def q4_bytes(n, k):
    return n * (k // 32) * 18


def gemm_bytes(m, n, k):
    """Algorithmic HBM bytes of one GEMM: Q4_0 weights, int4 codes, fp32 scales, fp32 out."""
    return q4_bytes(n, k) + m * k // 2 + m * (k // 32) * 4 + m * n * 4


def weight_copies(torch, packed, total_bytes=COLD_BYTES):
    n = max(2, -(-total_bytes // packed.numel()))
    return [packed] + [packed.clone() for _ in range(n - 1)]


# --------------------------------------------------------------------------
# the measured step: FFN up projection, M=512
# --------------------------------------------------------------------------

SAMPLE_EVERY = 4  # steps of the timed pass that carry kernel-duration events


def run_main(torch, ops, synth, steps, warmup):
    d = synth.ffn_up()
    m, n, k = d.m, d.n, d.k
    dev = torch.device("cuda:0")
    w = torch.from_numpy(d.w).to(dev)
    packed = ops.prepare_weights(w)
    del w
    copies = weight_copies(torch, packed)
    x = torch.from_numpy(d.x).to(dev)
    codes = torch.empty((m, k // 2), dtype=torch.uint8, device=dev)
    scales = torch.empty((m, k // 32), dtype=torch.float32, device=dev)
    y = torch.empty((m, n), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()

    act = torch.empty(max(1, ops.act_operand_bytes(m, k)), dtype=torch.uint8, device=dev)

    # one step = rotate-quantise (which also lays out the matrix-core operand),
    # then the matrix-core GEMM
    def rq():
        ops.rotate_quantize_prepare(x, act, codes=codes, scales=scales)

    def gemm(i):
        ops.gemm_prepared(copies[i % len(copies)], act, m, n, k, y=y)

    for i in range(warmup):
        rq()
        gemm(i)
    torch.cuda.synchronize()
    # the timed pass: exactly `steps` steps between two synchronisations.  On
    # every SAMPLE_EVERY-th step three events on the launch stream (before,
    # between and after its two kernels) give that step's kernel durations in
    # the same pass and interleaving as the step time; the other steps carry
    # no event (each event record costs the stream ~1.5-2 us, which would
    # otherwise be part of every step)
    sampled = [i for i in range(steps) if i % SAMPLE_EVERY == 0]
    ev = {i: [torch.cuda.Event(enable_timing=True) for _ in range(3)] for i in sampled}
    t0 = time.perf_counter()
    for i in range(steps):
        e = ev.get(i)
        if e: e[0].record()
        rq()
        if e: e[1].record()
        gemm(i)
        if e: e[2].record()
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / steps
    rq_us = np.array([ev[i][0].elapsed_time(ev[i][1]) * 1e3 for i in sampled])
    gemm_us = np.array([ev[i][1].elapsed_time(ev[i][2]) * 1e3 for i in sampled])
    step_us = np.array([ev[i][0].elapsed_time(ev[i][2]) * 1e3 for i in sampled])
    ops_per = 2.0 * m * n * k
    return dict(workload=d.name, m=m, n=n, k=k, wall_ms=wall_ms, rq_us=stats(rq_us), gemm_us=stats(gemm_us),
                step_us=stats(step_us), gemm_ops=ops_per, gemm_bytes=gemm_bytes(m, n, k),
                weight_copies=len(copies))


def stats(a):
    """Median, minimum and mean of per-call microseconds."""
    a = np.asarray(a, np.float64)
    return {"median": round(float(np.median(a)), 3), "min": round(float(a.min()), 3),
            "mean": round(float(a.mean()), 3), "n": int(a.size)}


# --------------------------------------------------------------------------
# extras
# --------------------------------------------------------------------------

def events_ms(torch, fn, reps):
    """Mean milliseconds of fn(i), i < reps, run back to back on the current
    stream between one pair of HIP events."""
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record()
    for i in range(reps):
        fn(i)
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / reps


GRAPH_CALLS = 64  # at least this many launches per timing graph of a short kernel
GRAPH_REPS = 20   # timed replays per graph
# --light (for counter passes under a profiler, where every dispatch is slow
# and times mean nothing): few copies, launches and replays; the kernels and
# their launch shapes are the same
LIGHT = False
LIGHT_COPIES = 4


STEP_GRAPH_STEPS = 16  # at least this many whole steps per timing graph of a step


def graph_steps(copies):
    """Steps per timing graph of a multi-kernel step over `copies` weight
    sets: whole rotations, at least STEP_GRAPH_STEPS."""
    return copies if LIGHT else max(1, -(-STEP_GRAPH_STEPS // copies)) * copies


def cold_copies(read_bytes):
    """Copies to rotate over so that the bytes a call reads, over one
    rotation, are twice the last-level cache: each call then finds its
    weights evicted."""
    n = max(2, -(-2 * LLC_BYTES // max(1, int(read_bytes))))
    return min(n, LIGHT_COPIES) if LIGHT else n


def graph_calls(copies):
    """Launches per timing graph over `copies` rotating buffers: whole
    rotations, at least GRAPH_CALLS, so that the replay's own cost (its
    submission and the event pair around it) is spread over many launches."""
    return copies if LIGHT else max(2, -(-GRAPH_CALLS // copies)) * copies


def graph_time_us(torch, fn, reps=None, inner=1):
    """Capture `fn` (which enqueues `inner` identical units of work) in a HIP
    graph, replay it `reps` times with an event pair around each replay, and
    return the median time of one unit in microseconds.  Graph replay removes
    the Python launch overhead between kernels."""
    stream = torch.cuda.Stream()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        fn()
    for _ in range(2):
        g.replay()
    torch.cuda.synchronize()
    reps = reps or GRAPH_REPS
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for a, b in ev:
        a.record()
        g.replay()
        b.record()
    torch.cuda.synchronize()
    return float(np.median([a.elapsed_time(b) for a, b in ev])) * 1e3 / inner


_READ_FLOOR = {}


def read_floor_us(torch, nbytes, copies):
    """The time of a plain read of `nbytes` in the regime the small-M
    products are timed in (a HIP graph of graph_calls(copies) back-to-back
    launches over `copies` buffers, as each product rotates over that many
    weight copies), with the committed read-stream probe (libw4a4_ceilings.so), at
    the best of four grid sizes: the size-matched ceiling of a weight stream
    of that many bytes, launch and ramp included.  None without the probe
    library."""
    import ctypes
    nbytes = (int(nbytes) + 255) // 256 * 256
    if (nbytes, copies) in _READ_FLOOR:
        return _READ_FLOOR[(nbytes, copies)]
    path = os.path.join(ROOT, "hadamard_rotated_w4a4_amd", "libw4a4_ceilings.so")
    if not os.path.exists(path):
        return None
    L = ctypes.CDLL(path)
    L.w4a4c_read_stream.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    dev = torch.device("cuda:0")
    nbuf = max(2, copies)
    bufs = [torch.ones(nbytes, dtype=torch.uint8, device=dev) for _ in range(nbuf)]
    sink = torch.empty(4096 * 256, dtype=torch.int32, device=dev)
    best = None
    for blocks in ((1024,) if LIGHT else (512, 1024, 2048, 4096)):
        def one(blocks=blocks):
            st = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
            for i in range(graph_calls(nbuf)):
                rc = L.w4a4c_read_stream(ctypes.c_void_p(bufs[i % nbuf].data_ptr()), nbytes,
                                         ctypes.c_void_p(sink.data_ptr()), blocks, st)
                if rc:
                    raise RuntimeError(f"read stream launch failed ({rc})")
        us = graph_time_us(torch, one, inner=graph_calls(nbuf))
        best = us if best is None else min(best, us)
    del bufs
    _READ_FLOOR[(nbytes, copies)] = best
    return best


def run_verify16(torch, ops, synth):
    """16-token verify block through the seven dense projections (M<=16 path)."""
    dev = torch.device("cuda:0")
    ws = synth.layer_weights(workload=4)
    xs = synth.layer_inputs(16, workload=4)
    packed = {name: ops.prepare_weights(torch.from_numpy(ws[name]).to(dev)) for name, _, _ in synth.DENSE_PROJECTIONS}
    del ws
    layer_bytes = sum(p.numel() for p in packed.values())
    nsets = max(2, -(-COLD_BYTES // layer_bytes))
    sets = [packed] + [{k_: v.clone() for k_, v in packed.items()} for _ in range(nsets - 1)]
    inputs = {name: torch.from_numpy(a).to(dev) for name, a in xs.items()}
    # each input quantised once with its record-ordered operand (the m <= 16
    # prepared path); the codes and scales feed the from-codes path
    acts = {inp: torch.empty(ops.small_act_operand_bytes(16, xin.shape[1]), dtype=torch.uint8, device=dev)
            for inp, xin in inputs.items()}
    q = {inp: ops.rotate_quantize_prepare_small(xin, acts[inp]) for inp, xin in inputs.items()}
    ys = {name: torch.empty((16, n), dtype=torch.float32, device=dev) for name, _, n in synth.DENSE_PROJECTIONS}
    gws = torch.empty(max(ops.gemm_workspace_bytes(16, n, k) for _, k, n in synth.DENSE_PROJECTIONS),
                      dtype=torch.uint8, device=dev)
    out = {"rows": 16, "weight_sets": nsets,
           "path": "rotate_quantize_prepare_small once per input (codes, scales and the record-ordered operand), "
                   "then gemm_prepared_small per projection; *_from_codes: gemm on the public codes and scales",
           "timing": "HIP graph replay; each projection alone over copies of its weights whose streamed bytes "
                     "per rotation are twice the 256 MB last-level cache, the steps over the layer's weight sets "
                     "(cold either way); read_floor_us: a plain read of the projection's weight bytes in the same "
                     "rotation"}
    tot_us, tot_bytes, codes_us = 0.0, 0, 0.0
    ncopies = {}
    for name, k, n in synth.DENSE_PROJECTIONS:
        inp = synth.DENSE_INPUT_OF[name]
        c, sc = q[inp]
        nc = ncopies[name] = cold_copies(n * k * 18 // 32)  # the 4-bit records this product streams
        copies = [packed[name]] + [packed[name].clone() for _ in range(nc - 1)]

        def one(k=k, n=n, act=acts[inp], copies=copies, nc=nc, y=ys[name]):
            for i in range(graph_calls(nc)):
                ops.gemm_prepared_small(copies[i % nc], act, 16, n, k, y=y, workspace=gws)

        def one_codes(k=k, n=n, c=c, sc=sc, copies=copies, nc=nc, y=ys[name]):
            for i in range(graph_calls(nc)):
                ops.gemm(copies[i % nc], c, sc, n, k, y=y, workspace=gws)
        us = graph_time_us(torch, one, inner=graph_calls(nc))
        us_c = graph_time_us(torch, one_codes, inner=graph_calls(nc))
        del copies
        b = gemm_bytes(16, n, k)
        tot_us += us
        codes_us += us_c
        tot_bytes += b
        out[name] = {"k": k, "n": n, "us": round(us, 2), "GB/s": round(b / (us * 1e-6) / 1e9, 1),
                     "us_from_codes": round(us_c, 2)}
        log(f"[bench] verify_m16 {name}: {us:.2f} us ({us_c:.2f} from codes) over {nc} copies")
    floors = {}
    for name, k, n in synth.DENSE_PROJECTIONS:
        floors[name] = read_floor_us(torch, n * k * 18 // 32, ncopies[name])
        log(f"[bench] verify_m16 {name}: read floor {floors[name]}")
    if all(f is not None for f in floors.values()):
        for name, _, _ in synth.DENSE_PROJECTIONS:
            out[name]["read_floor_us"] = round(floors[name], 2)
            out[name]["frac_of_read_floor"] = round(floors[name] / out[name]["us"], 3)
        out["read_floor_us_total"] = round(sum(floors.values()), 2)
        out["frac_of_read_floor"] = round(sum(floors.values()) / tot_us, 3)

    def step():
        for i in range(graph_steps(nsets)):
            for inp, xin in inputs.items():
                ops.rotate_quantize_prepare_small(xin, acts[inp], codes=q[inp][0], scales=q[inp][1])
            for name, k, n in synth.DENSE_PROJECTIONS:
                ops.gemm_prepared_small(sets[i % nsets][name], acts[synth.DENSE_INPUT_OF[name]], 16, n, k,
                                        y=ys[name], workspace=gws)
    step_us = graph_time_us(torch, step, inner=graph_steps(nsets))

    def step_codes():
        for i in range(graph_steps(nsets)):
            qq = {inp: ops.rotate_quantize_act(xin) for inp, xin in inputs.items()}
            for name, k, n in synth.DENSE_PROJECTIONS:
                c, sc = qq[synth.DENSE_INPUT_OF[name]]
                ops.gemm(sets[i % nsets][name], c, sc, n, k, y=ys[name], workspace=gws)
    step_codes_us = graph_time_us(torch, step_codes, inner=graph_steps(nsets))

    # rotate-quantise fused into the product (one launch per distinct input:
    # its first projection quantises, the others reuse the codes it wrote)
    firsts = {}
    for name, k, n in synth.DENSE_PROJECTIONS:
        firsts.setdefault(synth.DENSE_INPUT_OF[name], name)
    qbuf = {inp: (torch.empty((16, xin.shape[1] // 2), dtype=torch.uint8, device=dev),
                  torch.empty((16, xin.shape[1] // 32), dtype=torch.float32, device=dev))
            for inp, xin in inputs.items()}
    fq_ws = torch.zeros(max(ops.rotate_quantize_gemm_workspace_bytes(16, n, k) for _, k, n in synth.DENSE_PROJECTIONS),
                        dtype=torch.uint8, device=dev)  # zero before its first use

    def fused_step():
        for i in range(graph_steps(nsets)):
            for name, k, n in synth.DENSE_PROJECTIONS:
                inp = synth.DENSE_INPUT_OF[name]
                c, sc = qbuf[inp]
                if firsts[inp] == name:
                    ops.rotate_quantize_gemm(inputs[inp], sets[i % nsets][name], n, k, y=ys[name], codes=c, scales=sc,
                                             workspace=fq_ws)
                else:
                    ops.gemm(sets[i % nsets][name], c, sc, n, k, y=ys[name], workspace=gws)
    fused_step_us = graph_time_us(torch, fused_step, inner=graph_steps(nsets))
    out["rotate_quantize_fused"] = {"step_us": round(fused_step_us, 2),
                                    "tokens/s": round(16 / (fused_step_us * 1e-6), 1),
                                    "launches": "4 fused rotate-quantise + product, 3 products on the codes "
                                                "(K splits summed in the same launches)"}
    out["gemm_us_total"] = round(tot_us, 2)
    out["gemm_GB/s"] = round(tot_bytes / (tot_us * 1e-6) / 1e9, 1)
    out["hbm_frac"] = round(tot_bytes / (tot_us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)
    out["step_us"] = round(step_us, 2)
    out["tokens/s"] = round(16 / (step_us * 1e-6), 1)
    out["gemm_us_total_from_codes"] = round(codes_us, 2)
    out["step_us_from_codes"] = round(step_codes_us, 2)
    del sets, packed

    # The same set with the projections that read one input packed side by
    # side (q|k|v: n = 8192, gate|up: n = 34816): the same weight bytes and
    # arithmetic in 4 GEMMs instead of 7 (fewer launches and K-split sums).
    ws = synth.layer_weights(workload=4)
    groups = (("qkv", ("q", "k", "v"), "attn_in"), ("o", ("o",), "attn_out"),
              ("gate_up", ("gate", "up"), "ffn_in"), ("down", ("down",), "ffn_act"))
    fused = {g: ops.prepare_weights(torch.from_numpy(np.concatenate([ws[p] for p in parts])).to(dev))
             for g, parts, _ in groups}
    shape = {g: (ws[parts[0]].shape[1], sum(ws[p].shape[0] for p in parts)) for g, parts, _ in groups}
    del ws
    fsets = [fused] + [{k_: v.clone() for k_, v in fused.items()} for _ in range(nsets - 1)]
    fys = {g: torch.empty((16, shape[g][1]), dtype=torch.float32, device=dev) for g, _, _ in groups}
    fws = {g: torch.empty(max(1, ops.gemm_workspace_bytes(16, shape[g][1], shape[g][0])), dtype=torch.uint8, device=dev)
           for g, _, _ in groups}
    f_us = 0.0
    for g, _, inp in groups:
        k, n = shape[g]
        nc = cold_copies(n * k * 18 // 32)
        copies = [fused[g]] + [fused[g].clone() for _ in range(nc - 1)]

        def one(g=g, k=k, n=n, act=acts[inp], copies=copies, nc=nc):
            for i in range(graph_calls(nc)):
                ops.gemm_prepared_small(copies[i % nc], act, 16, n, k, y=fys[g], workspace=fws[g])
        f_us += graph_time_us(torch, one, inner=graph_calls(nc))
        del copies

    def fstep():
        for i in range(graph_steps(nsets)):
            for inp, xin in inputs.items():
                ops.rotate_quantize_prepare_small(xin, acts[inp], codes=q[inp][0], scales=q[inp][1])
            for g, _, inp in groups:
                k, n = shape[g]
                ops.gemm_prepared_small(fsets[i % nsets][g], acts[inp], 16, n, k, y=fys[g], workspace=fws[g])
    fstep_us = graph_time_us(torch, fstep, inner=graph_steps(nsets))
    fws2 = torch.zeros(max(ops.rotate_quantize_gemm_workspace_bytes(16, n, k) for k, n in shape.values()),
                       dtype=torch.uint8, device=dev)

    def fqstep():  # the four packed products, each with its rotate-quantise fused in
        for i in range(graph_steps(nsets)):
            for g, _, inp in groups:
                k, n = shape[g]
                ops.rotate_quantize_gemm(inputs[inp], fsets[i % nsets][g], n, k, y=fys[g], codes=qbuf[inp][0],
                                         scales=qbuf[inp][1], workspace=fws2)
    fqstep_us = graph_time_us(torch, fqstep, inner=graph_steps(nsets))
    out["same_input_fused"] = {"gemms": len(groups), "gemm_us_total": round(f_us, 2),
                               "rotate_quantize_fused_step_us": round(fqstep_us, 2),
                               "rotate_quantize_fused_tokens/s": round(16 / (fqstep_us * 1e-6), 1),
                               "gemm_GB/s": round(tot_bytes / (f_us * 1e-6) / 1e9, 1),
                               "hbm_frac": round(tot_bytes / (f_us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
                               "step_us": round(fstep_us, 2), "tokens/s": round(16 / (fstep_us * 1e-6), 1)}
    return out


def run_moe(torch, ops, synth):
    """MoE layer: gate, up (one activation row per token) and down (one per
    slot).  Timed cold: the three expert weight matrices are cloned into
    sets, consecutive calls take consecutive sets, and there are enough sets
    that the expert records one product streams, over a rotation, are twice
    the 256 MB last-level cache."""
    dev = torch.device("cuda:0")
    mo = synth.moe()
    E, T, top_k = mo.w_gate.shape[0], mo.ids.shape[0], mo.ids.shape[1]
    dm, dff = synth.MOE_D_MODEL, synth.MOE_D_FF

    def experts(w):
        return torch.cat([ops.prepare_weights(torch.from_numpy(w[e]).to(dev)) for e in range(E)])
    base = {"g": experts(mo.w_gate), "u": experts(mo.w_up), "d": experts(mo.w_down)}
    set_bytes = sum(t.numel() for t in base.values())
    counts = np.bincount(mo.ids.reshape(-1), minlength=E)
    streamed = int((counts > 0).sum()) * q4_bytes(dff, dm)  # one matrix's used experts, 4-bit records
    nsets = max(-(-COLD_BYTES // set_bytes), cold_copies(streamed))
    sets = [base] + [{k_: v.clone() for k_, v in base.items()} for _ in range(nsets - 1)]
    ids = torch.from_numpy(mo.ids).to(dev)
    x = torch.from_numpy(mo.x).to(dev)
    h = torch.from_numpy(mo.h).to(dev)
    ws = torch.empty(ops.gemm_id_workspace_bytes(E, T, top_k), dtype=torch.uint8, device=dev)
    yg = torch.empty((T, top_k, dff), dtype=torch.float32, device=dev)
    yu = torch.empty_like(yg)
    yd = torch.empty((T, top_k, dm), dtype=torch.float32, device=dev)
    cx, sx = ops.rotate_quantize_act(x)
    ch, sh = ops.rotate_quantize_act(h)

    def rotating(call):  # graph_calls(nsets) calls, consecutive sets
        return graph_time_us(torch, lambda: [call(sets[i % nsets]) for i in range(graph_calls(nsets))],
                             inner=graph_calls(nsets))

    def steps(fn):  # graph_steps(nsets) steps, consecutive sets
        return graph_time_us(torch, lambda: [fn(sets[i % nsets]) for i in range(graph_steps(nsets))],
                             inner=graph_steps(nsets))
    g = rotating(lambda st: ops.gemm_id(st["g"], E, cx, sx, 1, ids, dff, dm, y=yg, workspace=ws))
    u = rotating(lambda st: ops.gemm_id(st["u"], E, cx, sx, 1, ids, dff, dm, y=yu, workspace=ws))
    dd = rotating(lambda st: ops.gemm_id(st["d"], E, ch, sh, top_k, ids, dm, dff, y=yd, workspace=ws))
    # the quantisers alone: 20 calls per replay, so that the replay's own
    # launch cost is spread over them
    qx = graph_time_us(torch, lambda: [ops.rotate_quantize_act(x, codes=cx, scales=sx) for _ in range(20)], inner=20)
    qh = graph_time_us(torch, lambda: [ops.rotate_quantize_act(h, codes=ch, scales=sh) for _ in range(20)], inner=20)

    def step(st):
        ops.rotate_quantize_act(x, codes=cx, scales=sx)
        ops.rotate_quantize_act(h, codes=ch, scales=sh)
        ops.gemm_id(st["g"], E, cx, sx, 1, ids, dff, dm, y=yg, workspace=ws)
        ops.gemm_id(st["u"], E, cx, sx, 1, ids, dff, dm, y=yu, workspace=ws)
        ops.gemm_id(st["d"], E, ch, sh, top_k, ids, dm, dff, y=yd, workspace=ws)
    step_us = steps(step)

    # the same step routed once for the three products
    def rstep(st):
        ops.rotate_quantize_act(x, codes=cx, scales=sx)
        ops.rotate_quantize_act(h, codes=ch, scales=sh)
        ops.gemm_id_route(ids, E, workspace=ws)
        ops.gemm_id_routed(st["g"], E, cx, sx, 1, T, top_k, dff, dm, ws, y=yg)
        ops.gemm_id_routed(st["u"], E, cx, sx, 1, T, top_k, dff, dm, ws, y=yu)
        ops.gemm_id_routed(st["d"], E, ch, sh, top_k, T, top_k, dm, dff, ws, y=yd)
    rstep_us = steps(rstep)
    rows = T * top_k
    used = int((counts > 0).sum())
    b_gate = used * q4_bytes(dff, dm) + T * dm // 2 + T * dm // 8 + rows * dff * 4
    b_down = used * q4_bytes(dm, dff) + rows * dff // 2 + rows * dff // 8 + rows * dm * 4
    tot_ops = 2 * (2.0 * rows * dff * dm) + 2.0 * rows * dm * dff
    tot_bytes = 2 * b_gate + b_down
    gemm_us = g + u + dd
    del sets, base

    # gate|up of each expert packed as one 2 * d_ff-row matrix: one routed
    # GEMM for both (the same weight bytes and arithmetic), routed once
    base = {"gu": experts(np.concatenate([mo.w_gate, mo.w_up], axis=1)), "d": experts(mo.w_down)}
    sets = [base] + [{k_: v.clone() for k_, v in base.items()} for _ in range(nsets - 1)]
    ygu = torch.empty((T, top_k, 2 * dff), dtype=torch.float32, device=dev)
    gu = rotating(lambda st: ops.gemm_id(st["gu"], E, cx, sx, 1, ids, 2 * dff, dm, y=ygu, workspace=ws))

    def fstep(st):
        ops.rotate_quantize_act(x, codes=cx, scales=sx)
        ops.rotate_quantize_act(h, codes=ch, scales=sh)
        ops.gemm_id_route(ids, E, workspace=ws)
        ops.gemm_id_routed(st["gu"], E, cx, sx, 1, T, top_k, 2 * dff, dm, ws, y=ygu)
        ops.gemm_id_routed(st["d"], E, ch, sh, top_k, T, top_k, dm, dff, ws, y=yd)
    fstep_us = steps(fstep)
    del sets, base
    return {"experts": E, "tokens": T, "top_k": top_k, "count_min": int(counts.min()),
            "count_median": float(np.median(counts)), "count_max": int(counts.max()),
            "timing": f"HIP graph replay, median of 20; {nsets} weight sets of {set_bytes / 1e6:.0f} MB "
                      f"taken in turn (cold: more than the 256 MB last-level cache between reuses)",
            "gate_us": round(g, 2), "up_us": round(u, 2), "down_us": round(dd, 2),
            "quant_us": round(qx + qh, 2), "step_us": round(step_us, 2),
            "tokens/s": round(T / (step_us * 1e-6), 1),
            "step_us_routed_once": round(rstep_us, 2),
            "gemm_TOP/s": round(tot_ops / (gemm_us * 1e-6) / 1e12, 1),
            "mfma_frac": round(tot_ops / (gemm_us * 1e-6) / 1e12 / PEAK_INT8_TOPS, 4),
            "gemm_GB/s": round(tot_bytes / (gemm_us * 1e-6) / 1e9, 1),
            "hbm_frac": round(tot_bytes / (gemm_us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
            "gate_up_fused": {"gate_up_us": round(gu, 2), "step_us_routed_once": round(fstep_us, 2),
                              "tokens/s": round(T / (fstep_us * 1e-6), 1),
                              "gemm_GB/s": round(tot_bytes / ((gu + dd) * 1e-6) / 1e9, 1)}}


def run_w4a8(torch, ops, synth):
    """W4A8-H32 (int8 activation codes on the rotated file): the FFN-up step at
    M=512 and the gate projection of the 16-token verify block."""
    dev = torch.device("cuda:0")
    d = synth.ffn_up()
    packed = ops.prepare_weights(torch.from_numpy(d.w).to(dev))
    copies = weight_copies(torch, packed)
    x = torch.from_numpy(d.x).to(dev)
    codes = torch.empty((d.m, d.k), dtype=torch.int8, device=dev)
    scales = torch.empty((d.m, d.k // 32), dtype=torch.float32, device=dev)
    y = torch.empty((d.m, d.n), dtype=torch.float32, device=dev)
    # the int8 codes' two FP6 planes, written by the quantiser itself
    act = torch.empty(ops.act8_operand_bytes(d.m, d.k), dtype=torch.uint8, device=dev)
    # the two-call form re-lays the codes in its own pre-pass
    ws512 = torch.empty(ops.lib().w4a4_gemm_a8_workspace_bytes(d.m, d.n, d.k), dtype=torch.uint8, device=dev)

    def step(i):
        ops.rotate_quantize_prepare8(x, act, codes=codes, scales=scales)
        ops.gemm_a8_prepared(copies[i % len(copies)], act, d.m, d.n, d.k, y=y)
    for i in range(3):
        step(i)
    step_us = events_ms(torch, step, 10) * 1e3
    gemm_us = events_ms(torch, lambda i: ops.gemm_a8_prepared(copies[i % len(copies)], act, d.m, d.n, d.k, y=y),
                        10) * 1e3
    call_us = events_ms(torch, lambda i: ops.gemm_a8(copies[i % len(copies)], codes, scales, d.n, d.k, y=y,
                                                     workspace=ws512), 10) * 1e3
    ops_per = 2.0 * d.m * d.n * d.k
    # verify block: m=16, gate 5120 -> 17408
    x16 = x[:16].contiguous()
    c16, s16 = ops.rotate_quantize_act8(x16)
    y16 = torch.empty((16, d.n), dtype=torch.float32, device=dev)
    ws = torch.empty(max(1, ops.lib().w4a4_gemm_a8_workspace_bytes(16, d.n, d.k)), dtype=torch.uint8, device=dev)
    nsets = len(copies)

    def one():
        for i in range(graph_calls(nsets)):
            ops.gemm_a8(copies[i % nsets], c16, s16, d.n, d.k, y=y16, workspace=ws)
    us16 = graph_time_us(torch, one, inner=graph_calls(nsets))
    b16 = gemm_bytes(16, d.n, d.k) + 16 * d.k // 2  # int8 codes: twice the int4 bytes
    return {"ffn_up_m512": {"step_us": round(step_us, 2), "gemm_us": round(gemm_us, 2),
                            "gemm_a8_call_us": round(call_us, 2),
                            "tokens/s": round(d.m / (step_us * 1e-6), 1),
                            "TOP/s": round(ops_per / (gemm_us * 1e-6) / 1e12, 1),
                            "frac_of_int8_peak": round(ops_per / (gemm_us * 1e-6) / 1e12 / PEAK_INT8_TOPS, 4)},
            "gate_m16": {"us": round(us16, 2), "GB/s": round(b16 / (us16 * 1e-6) / 1e9, 1),
                         "hbm_frac": round(b16 / (us16 * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)},
            "timing": "events over back-to-back calls (M=512: step = quantiser writing the two FP6 planes + "
                      "prepared product; gemm_a8_call = the codes-and-scales call with its own re-laying "
                      "pre-pass); HIP graph replay (m=16)"}


def run_w4a16(torch, ops, synth):
    """Rotated W4A16 (section "Hadamard-rotated Q4_0: W4A4 prompt processing":
    the rotated file with 16-bit rotated activations): the FFN-up step at
    M=512, fp16 operands on the fp16 matrix cores, and its error against the
    exact product beside W4A4's on sampled rows."""
    import numpy as np
    dev = torch.device("cuda:0")
    d = synth.ffn_up()
    w = torch.from_numpy(d.w).to(dev)
    q4 = ops.quantize_q4_0_h32(w)
    w16 = ops.dequantize_w16(q4, d.n, d.k)
    packed = ops.repack_q4_0_h32(q4, d.n, d.k)
    del w
    nbytes = w16.numel() * w16.element_size()
    copies = [w16] + [w16.clone() for _ in range(max(1, -(-COLD_BYTES // nbytes) - 1))]
    x = torch.from_numpy(d.x).to(dev)
    a16 = ops.rotate_act16(x)
    y = torch.empty((d.m, d.n), dtype=torch.float32, device=dev)

    def step(i):
        ops.rotate_act16(x, out=a16)
        ops.gemm_w16(copies[i % len(copies)], a16, d.m, d.n, d.k, y=y)
    for i in range(3):
        step(i)
    step_us = events_ms(torch, step, 10) * 1e3
    gemm_us = events_ms(torch, lambda i: ops.gemm_w16(copies[i % len(copies)], a16, d.m, d.n, d.k, y=y), 10) * 1e3
    rot_us = events_ms(torch, lambda i: ops.rotate_act16(x, out=a16), 20) * 1e3
    # context only: the platform's library fp16 GEMM (fp16 out) on the same
    # operands, weights pre-transposed to K x N, two copies alternated
    wt = [ops.w16_to_rows(c, d.n, d.k).t().contiguous() for c in copies[:2]]
    a_rows = ops.w16_to_rows(a16, d.m, d.k)
    lib_out = torch.empty((d.m, d.n), dtype=torch.float16, device=dev)
    for i in range(3):
        torch.mm(a_rows, wt[i % 2], out=lib_out)
    lib_us = events_ms(torch, lambda i: torch.mm(a_rows, wt[i % 2], out=lib_out), 10) * 1e3
    del wt, a_rows
    flops = 2.0 * d.m * d.n * d.k
    rows = np.arange(0, d.m, d.m // 16)
    ops.gemm_w16(w16, a16, d.m, d.n, d.k, y=y)
    y4 = ops.gemm(packed, *ops.rotate_quantize_act(x), d.n, d.k)
    torch.cuda.synchronize()
    exact = d.x[rows].astype(np.float64) @ d.w.astype(np.float64).T
    err = {name: float(np.abs(t.cpu().numpy()[rows].astype(np.float64) - exact).mean())
           for name, t in (("w4a16", y), ("w4a4", y4))}
    return {"workload": d.name, "step_us": round(step_us, 2), "gemm_us": round(gemm_us, 2),
            "rotate_act16_us": round(rot_us, 2), "tokens/s": round(d.m / (step_us * 1e-6), 1),
            "TFLOP/s": round(flops / (gemm_us * 1e-6) / 1e12, 1),
            "frac_of_fp16_peak": round(flops / (gemm_us * 1e-6) / 1e12 / PEAK_FP16_TFLOPS, 4),
            "library_fp16_gemm_us": round(lib_us, 2),
            "mean_abs_err": {k_: round(v, 6) for k_, v in err.items()}, "rows_sampled": len(rows),
            "timing": "events over back-to-back calls"}


def run_ablation(torch, ops, synth):
    """Unrotated W4A4 ablation (section "MoE: W4A4 on the experts": without
    the rotation W4A4 costs about twice the accuracy): the FFN-up workload
    through both pipelines, errors against the exact fp64 product of the
    unquantised operands on sampled rows, and the unrotated quantiser's time."""
    import numpy as np
    dev = torch.device("cuda:0")
    d = synth.ffn_up()
    w = torch.from_numpy(d.w).to(dev)
    x = torch.from_numpy(d.x).to(dev)
    y_rot = ops.gemm(ops.prepare_weights(w), *ops.rotate_quantize_act(x), d.n, d.k)
    y_plain = ops.gemm(ops.prepare_weights_plain(w), *ops.quantize_act(x), d.n, d.k)
    rows = np.arange(0, d.m, d.m // 16)
    torch.cuda.synchronize()
    exact = d.x[rows].astype(np.float64) @ d.w.astype(np.float64).T
    out = {"workload": d.name, "rows_sampled": len(rows)}
    for name, y in (("rotated", y_rot), ("unrotated", y_plain)):
        e = y.cpu().numpy()[rows].astype(np.float64) - exact
        out[name] = {"mean_abs_err": float(np.abs(e).mean()),
                     "rel_rms_err": float(np.sqrt((e ** 2).mean() / (exact ** 2).mean()))}
    out["err_ratio_unrotated_over_rotated"] = round(out["unrotated"]["mean_abs_err"] / out["rotated"]["mean_abs_err"], 3)
    codes = torch.empty((d.m, d.k // 2), dtype=torch.uint8, device=dev)
    scales = torch.empty((d.m, d.k // 32), dtype=torch.float32, device=dev)
    q_rot = events_ms(torch, lambda i: ops.rotate_quantize_act(x, codes=codes, scales=scales), 20) * 1e3
    q_plain = events_ms(torch, lambda i: ops.quantize_act(x, codes=codes, scales=scales), 20) * 1e3
    out["quantise_us"] = {"rotated": round(q_rot, 2), "unrotated": round(q_plain, 2)}
    return out


def run_layer_prompt(torch, ops, synth):
    """Dense layer's seven projections over a 1,838-token prompt (512+512+512+302)."""
    dev = torch.device("cuda:0")
    ws = synth.layer_weights(workload=3)
    packed = {name: ops.prepare_weights(torch.from_numpy(ws[name]).to(dev)) for name, _, _ in synth.DENSE_PROJECTIONS}
    del ws
    mbs = []
    for i, mrows in enumerate(synth.PROMPT_MICROBATCHES):
        xs = synth.layer_inputs(mrows, workload=3, microbatch=i)
        mbs.append({k_: torch.from_numpy(v).to(dev) for k_, v in xs.items()})
    ys = [{name: torch.empty((mb["attn_in"].shape[0], n), dtype=torch.float32, device=dev)
           for name, _, n in synth.DENSE_PROJECTIONS} for mb in mbs]
    acts = {name: torch.empty(max(1, ops.act_operand_bytes(512, k)), dtype=torch.uint8, device=dev)
            for name, k in (("attn_in", 5120), ("attn_out", 6144), ("ffn_in", 5120), ("ffn_act", 17408))}
    # one split-K workspace for every product (they run one after another on one stream)
    ws_bytes = max(ops.gemm_prepared_workspace_bytes(mr, n, k) for mr in synth.PROMPT_MICROBATCHES
                   for _, k, n in synth.DENSE_PROJECTIONS + (("qkv", 5120, 8192), ("gate_up", 5120, 34816)))
    wsp = torch.empty(max(1, ws_bytes), dtype=torch.uint8, device=dev)

    def layer():
        # each distinct input is quantised and prepared once (Q/K/V share one,
        # gate/up share one), then every projection runs on it
        for mb, yb in zip(mbs, ys):
            mrows = mb["attn_in"].shape[0]
            for inp, xin in mb.items():
                ops.rotate_quantize_prepare(xin, acts[inp])
            for name, k, n in synth.DENSE_PROJECTIONS:
                ops.gemm_prepared(packed[name], acts[synth.DENSE_INPUT_OF[name]], mrows, n, k, y=yb[name], workspace=wsp)
    us = graph_time_us(torch, layer, reps=5)
    del packed, ys

    # q|k|v and gate|up packed side by side: 4 GEMMs per micro-batch
    ws = synth.layer_weights(workload=3)
    groups = (("qkv", ("q", "k", "v"), "attn_in"), ("o", ("o",), "attn_out"),
              ("gate_up", ("gate", "up"), "ffn_in"), ("down", ("down",), "ffn_act"))
    shape = {g: (ws[parts[0]].shape[1], sum(ws[p].shape[0] for p in parts)) for g, parts, _ in groups}
    fused = {g: ops.prepare_weights(torch.from_numpy(np.concatenate([ws[p] for p in parts])).to(dev))
             for g, parts, _ in groups}
    del ws
    fys = [{g: torch.empty((mb["attn_in"].shape[0], shape[g][1]), dtype=torch.float32, device=dev)
            for g, _, _ in groups} for mb in mbs]

    def flayer():
        for mb, yb in zip(mbs, fys):
            mrows = mb["attn_in"].shape[0]
            for inp, xin in mb.items():
                ops.rotate_quantize_prepare(xin, acts[inp])
            for g, _, inp in groups:
                k, n = shape[g]
                ops.gemm_prepared(fused[g], acts[inp], mrows, n, k, y=yb[g], workspace=wsp)
    fus = graph_time_us(torch, flayer, reps=5)
    tokens = sum(synth.PROMPT_MICROBATCHES)
    ops_tot = sum(2.0 * tokens * n * k for _, k, n in synth.DENSE_PROJECTIONS)
    return {"tokens": tokens, "microbatches": list(synth.PROMPT_MICROBATCHES), "layer_ms": round(us * 1e-3, 4),
            "timing": "HIP graph replay of the four micro-batches",
            "tokens/s": round(tokens / (us * 1e-6), 1),
            "TOP/s": round(ops_tot / (us * 1e-6) / 1e12, 1),
            "mfma_frac": round(ops_tot / (us * 1e-6) / 1e12 / PEAK_INT8_TOPS, 4),
            "same_input_fused": {"gemms_per_microbatch": len(groups), "layer_ms": round(fus * 1e-3, 4),
                                 "tokens/s": round(tokens / (fus * 1e-6), 1),
                                 "TOP/s": round(ops_tot / (fus * 1e-6) / 1e12, 1)}}


# --------------------------------------------------------------------------
# CPU baseline: the oracle on a bounded sample of the same workload
# --------------------------------------------------------------------------

def cpu_baseline(synth, target_s=12.0):
    """The oracle's rate on the host cores over a bounded sample: whole steps of
    the FFN-up workload (rotate-quantise + GEMM of all its rows) repeated until
    about target_s of CPU work has run; fewer rows only if one step is slower."""
    import oracle  # test infrastructure, timed here as a baseline only
    d = synth.ffn_up()
    threads = oracle.default_threads()
    q4 = oracle.prepare_weights(d.w)  # offline step, not timed

    def step(rows):
        t0 = time.perf_counter()
        c, s = oracle.rotate_quantize_act(d.x[:rows], threads=threads)
        oracle.gemm(q4, c, s, d.k, threads=threads)
        return time.perf_counter() - t0

    probe = 16
    est = step(probe) * d.m / probe  # estimated seconds of one whole step
    rows = d.m if est <= target_s else max(probe, int(d.m * target_s / est))
    reps, total = 0, 0.0
    while total < target_s * 0.8:
        total += step(rows)
        reps += 1
    return {"value": round(rows * reps / total, 3), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{reps} x rotate-quantise + GEMM of {rows} of {d.m} token rows of {d.name} "
                      f"(all N={d.n} outputs per row), {total:.1f} s wall, fp64 sums, {threads} threads",
            "ops/s": round(2.0 * rows * reps * d.n * d.k / total, 1)}


def cpu_baseline_extras(synth, target_s=4.0):
    """Bounded oracle samples of the other workloads, each about target_s of
    CPU work (rates per token are independent of the batch size for the
    oracle, which computes every output on its own):
      verify_m16     the seven projections of the 16-token verify block,
                     every row, on an eighth of each projection's columns;
      layer_prompt   the seven projections on 16 rows of the prompt's first
                     micro-batch, an eighth of each projection's columns;
      moe            4 tokens, all 8 slots, through gate, up and down (the
                     experts they route to)."""
    import oracle  # test infrastructure, timed here as a baseline only
    threads = oracle.default_threads()
    out = {}

    def repeat(fn):
        reps, total = 0, 0.0
        while total < target_s * 0.8 or reps == 0:
            t0 = time.perf_counter()
            fn()
            total += time.perf_counter() - t0
            reps += 1
        return reps, total

    for name, workload, rows in (("verify_m16", 4, 16), ("layer_prompt", 3, 16)):
        xs = synth.layer_inputs(rows, workload=workload, microbatch=0)
        cols = {}
        for i, (proj, k, n) in enumerate(synth.DENSE_PROJECTIONS):
            cols[proj] = (oracle.prepare_weights(synth.weights(n // 8, k, synth.rng_for(0, workload, i))), k)

        def step():
            q = {inp: oracle.rotate_quantize_act(xin, threads=threads) for inp, xin in xs.items()}
            for proj, (q4, k) in cols.items():
                oracle.gemm(q4, *q[synth.DENSE_INPUT_OF[proj]], k, threads=threads)
        reps, total = repeat(step)
        # the sample is 1/8 of the columns: a whole-set step takes 8 x as long
        out[name] = {"value": round(rows * reps / (8 * total), 3), "unit": "tokens/s", "cores": threads,
                     "kind": "oracle",
                     "sample": f"{reps} x rotate-quantise + the seven projections of {rows} rows on 1/8 of "
                               f"their columns, {total:.1f} s wall, scaled to whole projections"}
    mo = synth.moe(n_tokens=4, with_weights=False)
    E, top_k = synth.MOE_EXPERTS, mo.ids.shape[1]
    dm, dff = synth.MOE_D_MODEL, synth.MOE_D_FF
    used = np.unique(mo.ids)
    remap = np.full(E, -1, np.int32)
    remap[used] = np.arange(used.size)
    ids = remap[mo.ids]
    # the experts these tokens route to, drawn as the full layer draws them
    q4 = {nm: np.stack([oracle.prepare_weights(synth.weights(n, k, synth.rng_for(0, 5, base + int(e))))
                        for e in used])
          for nm, base, n, k in (("g", 1000, dff, dm), ("u", 2000, dff, dm), ("d", 3000, dm, dff))}

    def moe_step():
        cx, sx = oracle.rotate_quantize_act(mo.x, threads=threads)
        ch, sh = oracle.rotate_quantize_act(mo.h, threads=threads)
        oracle.gemm_id(q4["g"], cx, sx, 1, ids, dff, dm, threads=threads)
        oracle.gemm_id(q4["u"], cx, sx, 1, ids, dff, dm, threads=threads)
        oracle.gemm_id(q4["d"], ch, sh, top_k, ids, dm, dff, threads=threads)
    reps, total = repeat(moe_step)
    out["moe"] = {"value": round(4 * reps / total, 3), "unit": "tokens/s", "cores": threads, "kind": "oracle",
                  "sample": f"{reps} x rotate-quantise + gate, up and down of 4 tokens x top-{top_k} over "
                            f"the {used.size} experts they use, {total:.1f} s wall"}
    return out


def measure_ceilings(torch):
    """The part's practical ceilings, measured in this run with the committed
    probes (libw4a4_ceilings.so): an HBM read stream over 2 GiB, and the
    issue rates of the FP6 32x32x64 and int8 32x32x32 MFMAs over the whole
    chip at two waves per SIMD."""
    import ctypes
    path = os.path.join(ROOT, "hadamard_rotated_w4a4_amd", "libw4a4_ceilings.so")
    if not os.path.exists(path):
        return None
    L = ctypes.CDLL(path)
    L.w4a4c_read_stream.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    L.w4a4c_mfma_loop.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    dev = torch.device("cuda:0")
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    nbytes = 2 << 30
    buf = torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(1)
    blocks = cus * 8
    sink = torch.empty(blocks * 256, dtype=torch.int32, device=dev)

    def timed(fn, reps):
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        fn()
        for a, b in ev:
            a.record()
            fn()
            b.record()
        torch.cuda.synchronize()
        return float(np.median([a.elapsed_time(b) for a, b in ev])) * 1e-3

    t = timed(lambda: L.w4a4c_read_stream(ctypes.c_void_p(buf.data_ptr()), nbytes, ctypes.c_void_p(sink.data_ptr()),
                                          blocks, stream), 5)
    read_gbs = nbytes / t / 1e9
    del buf
    mblocks, iters = cus * 2, 4000
    sinkf = torch.empty(mblocks * 256, dtype=torch.float32, device=dev)
    rates = {}
    for kind, name, ops_each in ((0, "fp6_32x32x64", 131072.0), (1, "int8_32x32x32", 65536.0)):
        t = timed(lambda: L.w4a4c_mfma_loop(kind, iters, mblocks, ctypes.c_void_p(sinkf.data_ptr()), stream), 3)
        rates[name] = ops_each * 4 * iters * (mblocks * 4) / t / 1e12
    return {"read_GB/s": round(read_gbs, 1), "read_frac_of_spec": round(read_gbs / PEAK_HBM_GBS, 4),
            "fp6_TFLOP/s": round(rates["fp6_32x32x64"], 1), "int8_TOP/s": round(rates["int8_32x32x32"], 1),
            "int8_frac_of_spec": round(rates["int8_32x32x32"] / PEAK_INT8_TOPS, 4),
            "probes": "libw4a4_ceilings.so: 2 GiB read stream (16-byte loads, 4 in flight per thread); "
                      "independent MFMA chains, 2 waves per SIMD, no memory traffic"}


def gpu_clock_mhz():
    """The shader clock the driver reports for the GPU (sysfs: the hwmon
    frequency, else the starred pp_dpm_sclk level), in MHz; None if it cannot
    be read.  A file read, not a tool: a process that has initialised the GPU
    must not start other programs.  Recorded before and after the run (an idle
    part reports its low idle level)."""
    import glob
    import re
    for dev in sorted(glob.glob("/sys/class/drm/card*/device")):
        try:
            if open(os.path.join(dev, "vendor")).read().strip() != "0x1002":
                continue
        except OSError:
            continue
        for f in glob.glob(os.path.join(dev, "hwmon", "hwmon*", "freq1_input")):
            try:
                return int(open(f).read().strip()) // 1000000
            except (OSError, ValueError):
                pass
        try:
            for line in open(os.path.join(dev, "pp_dpm_sclk")):
                m = re.search(r"(\d+)\s*Mhz\s*\*", line, flags=re.I)
                if m:
                    return int(m.group(1))
        except OSError:
            pass
    return None


def counters_for(*kernels: str):
    """HBM bytes of one launch of each named kernel, summed, from the committed
    rocprofv3 counter runs; None if any is missing or the sources changed."""
    if not os.path.exists(PROFILE_JSON):
        return None
    rec = json.load(open(PROFILE_JSON))
    if rec.get("source_hash") != source_hash():
        return None
    total = 0
    for kernel in kernels:
        k = rec.get("kernels", {}).get(kernel)
        if k is None:
            return None
        total += k["hbm_bytes_per_launch"]
    return total


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-extras", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--calibrate-copy-mb", type=int, default=0,
                    help="first run 5 plain device copies of this many MiB (scales rocprofv3 byte counters)")
    ap.add_argument("--light", action="store_true",
                    help="extras with few weight copies, launches and replays (counter passes under a profiler)")
    args = ap.parse_args()
    global LIGHT, GRAPH_REPS
    if args.light:
        LIGHT, GRAPH_REPS = True, 3
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: the library has no multi-GPU path "
              "(the GEMM would shard over N with no exchange).", file=sys.stderr)
        sys.exit(2)

    import torch
    from hadamard_rotated_w4a4_amd import _lib as ops
    from hadamard_rotated_w4a4_amd import synth

    ops.lib()
    log(f"[bench] device: {torch.cuda.get_device_name(0)}")
    if args.calibrate_copy_mb:
        src = torch.empty(args.calibrate_copy_mb << 20, dtype=torch.uint8, device="cuda:0").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] calibration: 5 copies of {args.calibrate_copy_mb} MiB")
        del src, dst
    clock_before = gpu_clock_mhz()
    log("[bench] main: ffn_up M=512 K=5120 N=17408")
    r = run_main(torch, ops, synth, args.steps, args.warmup)
    g = r["gemm_us"]
    gemm_tops = r["gemm_ops"] / (g["median"] * 1e-6) / 1e12
    log(f"[bench] main: {r['wall_ms']:.4f} ms/step (sampled steps with events: median {r['step_us']['median']} us), "
        f"rotq+prepare median {r['rq_us']['median']} us, gemm median {g['median']} us (min {g['min']}), "
        f"{gemm_tops:.1f} TOP/s")
    value = r["m"] / (r["wall_ms"] * 1e-3)
    log("[bench] measured ceilings (read stream, MFMA issue)")
    ceil = measure_ceilings(torch)
    log(f"[bench] ceilings: {ceil}")
    traffic = counters_for("gemm_mx_kernel")
    util = None
    if traffic is not None:  # the same hash guard as the byte counters
        util = json.load(open(PROFILE_JSON)).get("mfma_utilisation", {}).get("gemm_mx_kernel")
    roofline = {"bound": "mfma", "achieved": round(gemm_tops, 2), "peak": PEAK_INT8_TOPS,
                "unit": "TOP/s", "frac": round(gemm_tops / PEAK_INT8_TOPS, 4), "traffic": traffic,
                "kernel": "gemm_mx_kernel (whole tiles, then K pieces of the leftover tiles, one launch: "
                          "FP6 32x32x64 MFMA block dots, two-block bf16 MFMA scale products, fp32 epilogue)",
                "ops_per_launch": r["gemm_ops"], "algorithmic_bytes_per_launch": r["gemm_bytes"],
                "launch_us": g, "mean_launch_us": g["mean"],
                "timing": "HIP events on the launch stream before, between and after the two kernels "
                          "of every 4th step of the timed pass (the same pass as ms_per_step; the other "
                          "steps carry no event records); achieved uses the median",
                "mfma_busy_pct": None if util is None else util["mfma_busy_pct"],
                "frac_of_fp6_peak": round(gemm_tops / PEAK_FP6_TOPS, 4),
                "frac_of_measured_int8": None if not ceil else round(gemm_tops / ceil["int8_TOP/s"], 4),
                "target_frac": 0.60,
                "note": "int8-equivalent ops (2 M N K): the exact 32-code block dots run on the FP6 "
                        "matrix cores at half their K, i.e. at the int8 rate; the per-block fp32 "
                        "scaling adds one vector multiply-add per output and block"}
    extras = {}
    if not args.no_extras:
        log("[bench] extra: 16-token verify block, seven projections")
        extras["verify_m16"] = run_verify16(torch, ops, synth)
        if ceil:
            v = extras["verify_m16"]
            v["frac_of_measured_read"] = round(v["gemm_GB/s"] / ceil["read_GB/s"], 4)
            v["same_input_fused"]["frac_of_measured_read"] = round(
                v["same_input_fused"]["gemm_GB/s"] / ceil["read_GB/s"], 4)
            v["target_hbm_frac"] = 0.70
        log(f"[bench] verify_m16: {extras['verify_m16']['gemm_GB/s']} GB/s, "
            f"{extras['verify_m16'].get('frac_of_read_floor')} of the size-matched read floor")
        log("[bench] extra: MoE MUL_MAT_ID layer (cold)")
        extras["moe"] = run_moe(torch, ops, synth)
        log(f"[bench] moe: {extras['moe']['step_us']} us/step")
        log("[bench] extra: W4A8-H32 (int8 activations)")
        extras["w4a8"] = run_w4a8(torch, ops, synth)
        log(f"[bench] w4a8: {extras['w4a8']['ffn_up_m512']}")
        extras["w4a16"] = run_w4a16(torch, ops, synth)
        log(f"[bench] w4a16: {extras['w4a16']['gemm_us']} us, {extras['w4a16']['TFLOP/s']} TFLOP/s")
        extras["ablation_unrotated"] = run_ablation(torch, ops, synth)
        log(f"[bench] ablation: error ratio {extras['ablation_unrotated']['err_ratio_unrotated_over_rotated']}")
        log("[bench] extra: dense layer set over a 1,838-token prompt")
        extras["layer_prompt_1838"] = run_layer_prompt(torch, ops, synth)
        log(f"[bench] layer: {extras['layer_prompt_1838']['layer_ms']} ms")
    clock_after = gpu_clock_mhz()
    cpu = None
    if not args.no_cpu:
        log("[bench] cpu baseline (oracle, bounded sample)")
        cpu = cpu_baseline(synth)
        log(f"[bench] cpu: {cpu['value']} tokens/s on {cpu['cores']} threads")
        if not args.no_extras:
            for name, rec in cpu_baseline_extras(synth).items():
                key = {"verify_m16": "verify_m16", "layer_prompt": "layer_prompt_1838", "moe": "moe"}[name]
                extras[key]["cpu_baseline"] = rec
                log(f"[bench] cpu {name}: {rec['value']} tokens/s")
    out = {
        "metric": "W4A4 Q4_0-H32 GEMM tokens/s & int8 TOPS at M=512 (% MFMA peak); GB/s at M=16",
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["wall_ms"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp6",
        "data": "synthetic",
        "config": {"workload": r["workload"], "m": r["m"], "k": r["k"], "n": r["n"],
                   "activations": "fp16 N(0,1), 1% channels x20", "weights": "N(0,0.02) H32-rotated Q4_0",
                   "step": "rotate_quantize_prepare + gemm_prepared",
                   "weight_copies": r["weight_copies"]},
        "roofline": roofline,
        "cpu_baseline": cpu,
        # the event-bearing (sampled) steps: each also carries its three event
        # records, so it reads above ms_per_step, the average of all steps
        "sampled_step_us": r["step_us"],
        "gemm_us": g,
        "rotate_quantize_prepare_us": r["rq_us"],
        "sampled_steps": f"every {SAMPLE_EVERY}th of the {args.steps} timed steps",
        "measured_ceilings": ceil,
        "sclk_mhz": {"before": clock_before, "after": clock_after},
        "extras": extras,
        "source_hash": source_hash(),
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
