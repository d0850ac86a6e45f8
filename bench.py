#!/usr/bin/env python3
"""Benchmark of the Palimpsa chunked forward on one MI355X.

One step = one palimpsa_fwd_chunked pass over the 760M-model layer workload
(B=8, H=12, T=4096, d_k=d_v=128, bf16 inputs and output, float32 state),
inputs resident in HBM.  Prints ONE JSON line.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]

Every roofline object reports its kernel (or call) against MI355X's published
peaks: FP32 vector 157.3 TFLOP/s, HBM3E 8 TB/s, dense bf16 matrix cores
2.5 PFLOP/s.  `frac` is achieved / peak for the roof named in `bound`, and
`valu_frac`, `hbm_frac` and `mfma_frac` give all three.  The exact forward is
bound by the FP32 vector ALU (the readout divides by a per-token, per-entry
precision, so there is no dense contraction for the matrix cores, and the
kernel needs only a few hundred GB/s of HBM); per state-entry update the
method needs 4 FMA + 2 MUL + 1 reciprocal = 10 flops.  A secondary
`issue_model` states the same time against this build's own instruction-issue
bound (no packed FP32: one wave64 FP32 VALU instruction per SIMD every 4
clocks, transcendentals not counted), which no kernel can exceed.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

# Published MI355X peaks.  The FP32 vector figure counts a packed FMA
# (2 lanes x 2 flops) on every lane and clock: 256 CUs x 4 SIMDs x 16 lanes x
# 2 x 2 flops x 2.4 GHz.
FP32_PEAK_TFLOPS = 157.3
HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
# Instruction-issue bound of this build (secondary): each SIMD issues one
# wave64 FP32 VALU instruction every 4 clocks (16 lane-ops per clock; packed
# FP32 is switched off in the build), 256 CUs x 4 SIMDs at 2.4 GHz.
CUS, SIMDS, LANES_PER_CLK, CLOCK_HZ = 256, 4, 16, 2.4e9
LANE_OPS_PER_S = CUS * SIMDS * LANES_PER_CLK * CLOCK_HZ       # 3.93e13
# Per state-entry update and token, VALU instructions other than
# transcendentals (v_rcp_f32, v_rsq_f32), and algorithmic flops (FMA = 2,
# MUL/ADD = 1, transcendentals not counted):
#  forward: w = fma(beta, k2, c), I = fma(a, I, w), t = bv k, M = fma(a, M, t),
#           u = M r, acc = fma(u, q, acc)                       6 VALU, 10 flops
#  backward: replay of the update 4 VALU (7 flops) + reverse step 16 VALU
#           (22 flops)                                           20 VALU, 29 flops
#  2x2 block-diagonal forward, per entry: 10.5 VALU, 16.5 flops
#  4x4 block-diagonal forward, per entry: 18.5 VALU, 29.5 flops
#  2x2 backward, per entry: replay 5.5 + reverse 25 VALU, 45 flops
#  4x4 backward, per entry: replay 8.5 + reverse 40 VALU, 75 flops
FWD = dict(valu=6, flops=10)
BWD = dict(valu=20, flops=29)
BD2 = dict(valu=10.5, flops=16.5)
BD4 = dict(valu=18.5, flops=29.5)
BD2_BWD = dict(valu=30.5, flops=45)
BD4_BWD = dict(valu=48.5, flops=75)


def roofline(bound, seconds, flops=0.0, nbytes=0.0, mfma_flops=0.0, traffic=None, mix=None, **extra):
    """A roofline object for `seconds` of work that must do `flops` FP32
    vector flops, move `nbytes` of HBM bytes and do `mfma_flops` of matrix-core
    flops (all algorithmic).  `mix` (per-unit VALU count and flops) adds the
    instruction-issue model."""
    valu = flops / seconds / 1e12
    hbm = nbytes / seconds / 1e9
    mfma = mfma_flops / seconds / 1e12
    if bound == "alu":
        achieved, peak, unit = valu, FP32_PEAK_TFLOPS, "TFLOP/s"
    elif bound == "hbm":
        achieved, peak, unit = hbm, HBM_PEAK_GBS, "GB/s"
    else:
        achieved, peak, unit = mfma, MFMA_BF16_PEAK_TFLOPS, "TFLOP/s"
    out = {"bound": bound, "achieved": achieved, "peak": peak, "unit": unit, "frac": achieved / peak,
           "traffic": traffic, "valu_frac": valu / FP32_PEAK_TFLOPS, "hbm_frac": hbm / HBM_PEAK_GBS,
           "mfma_frac": mfma / MFMA_BF16_PEAK_TFLOPS, "algorithmic_bytes": nbytes}
    if mix is not None:
        model = LANE_OPS_PER_S / mix["valu"] * mix["flops"] / 1e12
        out["issue_model"] = {"peak": model, "unit": "TFLOP/s", "frac": valu / model,
                              "per_unit": "%g VALU (transcendentals not counted), %g flops"
                                          % (mix["valu"], mix["flops"])}
    out.update(extra)
    return out


def fwd_bytes(w, esz_in, esz_out, state_in=False):
    """Algorithmic HBM bytes of one chunked forward: the per-token inputs and y,
    the final state written (and the start state read when given)."""
    per_tok = w.B * w.T * w.H
    state = w.B * w.H * w.dv * w.dk * 4
    return (per_tok * ((2 * w.dk + 2 * w.dv + 1) * esz_in + w.dv * esz_out)
            + 2 * state * (2 if state_in else 1))


def kernel_source_hash():
    p = os.path.join(ROOT, "bayesian_metaplastic_memory_amd", "csrc", "palimpsa.hip")
    return hashlib.sha256(open(p, "rb").read()).hexdigest()[:16]


def load_traffic(name):
    """HBM traffic per launch from a committed rocprofv3 counter summary, if it
    was taken on the current kernel source; else None."""
    p = os.path.join(ROOT, "profiles", name)
    try:
        d = json.load(open(p))
    except (OSError, ValueError):
        return None
    if d.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    return d.get("hbm_bytes_per_launch")


def time_launches(fn, steps, warmup, torch):
    """Run fn() warmup times, then time `steps` calls with one event pair per
    launch on the current stream (the stream the kernels are enqueued on)."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    outer0 = torch.cuda.Event(enable_timing=True)
    outer1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    outer0.record()
    for i in range(steps):
        starts[i].record()
        fn()
        ends[i].record()
    outer1.record()
    torch.cuda.synchronize()
    per = [s.elapsed_time(e) for s, e in zip(starts, ends)]
    return outer0.elapsed_time(outer1), per


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(inp, w, max_heads):
    """The float64 oracle (plain sequential Eq. (5) in C, OpenMP over heads)
    on the host cores: once with every thread the runtime offers, once with
    one thread, on the same sample of heads at full length."""
    import oracle
    heads = [(b, h) for b in range(w.B) for h in range(w.H)][:max_heads]
    sub = oracle.select_heads(inp, heads)
    threads = oracle.max_threads()
    t0 = time.perf_counter()
    oracle.fwd(**sub, nthreads=threads)
    wall = time.perf_counter() - t0
    t0 = time.perf_counter()
    oracle.fwd(**sub, nthreads=1)
    wall1 = time.perf_counter() - t0
    layer_seqs = len(heads) / w.H                # sampled heads as a fraction of B sequences
    return {"value": layer_seqs * w.T / wall, "unit": "tokens/s", "cores": threads,
            "kind": "oracle", "cpu_model": cpu_model(), "wall_s": wall,
            "one_thread": {"value": layer_seqs * w.T / wall1, "unit": "tokens/s", "wall_s": wall1},
            "sample": "%d of %d heads (b,h) at full T=%d, float64 sequential Eq. (5), "
                      "OpenMP over heads: %.1f s wall on %d threads, %.1f s on 1"
                      % (len(heads), w.B * w.H, w.T, wall, threads, wall1)}


def graph_step_time(torch, fn, steps, per_graph=16):
    """Per-call time of a short kernel: a captured HIP graph of `per_graph`
    calls (they record no memsets or allocations), replayed and timed."""
    fn()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(per_graph):
            fn()
    _, per = time_launches(graph.replay, max(2, steps // per_graph), 3, torch)
    return sum(per) / len(per) / 1e3 / per_graph


def decode_extra(torch, pm, workloads, steps):
    """Decode step at B=64, H=32, d=128 (state 268 MB read + written per step)."""
    w = workloads.WORKLOADS[3]
    dev = torch.device("cuda:0")
    A, Ip = (x.to(dev) for x in workloads.head_constants(w))
    mu0, I0 = workloads.random_state(w.B, w.H, w.dv, w.dk, Ip.cpu(), seed=7)
    mu, I = mu0.to(dev), I0.to(dev)
    d = {n: x.to(dev) for n, x in workloads.decode_inputs(w, 0).items()}
    y = torch.empty(w.B, w.H, w.dv, dtype=w.dtype, device=dev)
    fn = lambda: pm.step(d["q"], d["k"], d["v"], d["beta"], d["dt"], A, Ip, mu, I, y=y)
    # A decode kernel takes under 90 us, less than the Python binding needs to
    # submit it, so the timed loop replays a captured graph of 16 steps.
    avg_s = graph_step_time(torch, fn, steps)
    updates = w.B * w.H * w.dv * w.dk
    nbytes = 16 * updates + 2 * w.B * w.H * (2 * w.dk + 2 * w.dv + 1) + 2 * w.B * w.H * w.dv
    return {"workload": "decode B=64 H=32 d_k=d_v=128, bf16 inputs, fp32 state",
            "tokens_per_s": w.B / avg_s, "us_per_step": avg_s * 1e6,
            "timing": "HIP graph of 16 steps, replayed",
            "roofline": roofline("hbm", avg_s, flops=updates * FWD["flops"], nbytes=nbytes,
                                 traffic=load_traffic("step_kernel_decode_B64_H32_d128_traffic.json"),
                                 kernel="step_kernel<128, bf16, bf16>")}


def blockdiag_decode_extra(torch, pm, workloads, steps):
    """Decode step of the 2x2 block-diagonal path at B=64, H=32, d=128: mu and
    the precision blocks (12 bytes per state entry) read and written per step."""
    w = workloads.WORKLOADS[3]
    dev = torch.device("cuda:0")
    A, Ip = (x.to(dev) for x in workloads.head_constants(w))
    mu0, P0 = workloads.random_block_state(w.B, w.H, w.dv, w.dk, 2, Ip.cpu(), seed=7)
    mu, P = mu0.to(dev), P0.to(dev)
    d = {n: x.to(dev) for n, x in workloads.decode_inputs(w, 0).items()}
    y = torch.empty(w.B, w.H, w.dv, dtype=w.dtype, device=dev)
    fn = lambda: pm.step_blockdiag(d["q"], d["k"], d["v"], d["beta"], d["dt"], A, Ip, mu, P, y=y)
    avg_s = graph_step_time(torch, fn, steps)
    entries = w.B * w.H * w.dv * w.dk
    nbytes = 2 * 12 * entries + 2 * w.B * w.H * (2 * w.dk + 2 * w.dv + 1) + 2 * w.B * w.H * w.dv
    return {"workload": "2x2 block-diagonal decode B=64 H=32 d_k=d_v=128, bf16 inputs, fp32 state",
            "tokens_per_s": w.B / avg_s, "us_per_step": avg_s * 1e6,
            "timing": "HIP graph of 16 steps, replayed",
            "roofline": roofline("hbm", avg_s, flops=entries * BD2["flops"], nbytes=nbytes,
                                 traffic=load_traffic("bd2_step_decode_B64_H32_d128_traffic.json"),
                                 kernel="bd2_step_kernel<128, bf16, bf16>")}


def grad_bytes(w, esz):
    """Algorithmic HBM bytes of a backward call: read q, k, v, beta, dt, gy and
    the final-state gradients; write the float32 per-token gradients and the
    start-state gradients."""
    btok = w.B * w.T * w.H
    state = w.B * w.H * w.dv * w.dk * 4
    return btok * ((2 * w.dk + 3 * w.dv + 1) * esz + (2 * w.dk + 2 * w.dv + 1) * 4) + 4 * state


def backward_extra(torch, pm, workloads, w, g, steps):
    """palimpsa_bwd on the same workload: checkpoint pass, backward kernel and
    the finishing kernels, timed as one call."""
    dev = g["q"].device
    gr = {n: (x.to(dev) if x is not None else None)
          for n, x in workloads.upstream_grads(w.B, w.T, w.H, w.dv, w.dk, w.dtype, seed=2).items()}
    ws = torch.empty(pm.bwd_workspace_size(w.B, w.T, w.H, w.dk, w.dv), dtype=torch.uint8, device=dev)
    args = (g["q"], g["k"], g["v"], g["beta"], g["dt"], g["A"], g["I_prior"], gr["gy"])
    out = pm.bwd(*args, gmuT=gr["gmuT"], gIT=gr["gIT"], workspace=ws)
    fn = lambda: pm.bwd(*args, gmuT=gr["gmuT"], gIT=gr["gIT"], workspace=ws, out=out)
    _, per = time_launches(fn, steps, 3, torch)
    avg_s = sum(per) / len(per) / 1e3
    updates = w.B * w.H * w.T * w.dv * w.dk
    esz = 2 if w.dtype == torch.bfloat16 else 4
    return {"workload": w.name + ", backward (gq, gk, gv, gbeta, gdt, gA, gIp, gmu0, gI0)",
            "tokens_per_s": w.B * w.T / avg_s, "ms_per_call": avg_s * 1e3,
            "workspace_GB": ws.numel() / 1e9,
            "roofline": roofline("alu", avg_s, flops=updates * BWD["flops"], nbytes=grad_bytes(w, esz) + 8 *
                                 w.B * w.H * w.dv * w.dk, mix=BWD,
                                 traffic=load_traffic("bwd_layer760m_bf16_traffic.json")
                                 if w.name.startswith("layer760m") else None,
                                 scope="whole call (checkpoint pass, reverse walk, finishing kernels); "
                                       "per-kernel split in the committed trace")}


def training_extra(torch, pm, workloads, w, g, steps):
    """One training step of the layer: the forward that stores the backward's
    checkpoints, then the backward that reuses them; beside it the same step
    with the plain forward and a backward that recomputes its checkpoints."""
    dev = g["q"].device
    gr = {n: (x.to(dev) if x is not None else None)
          for n, x in workloads.upstream_grads(w.B, w.T, w.H, w.dv, w.dk, w.dtype, seed=2).items()}
    ws = torch.empty(pm.bwd_workspace_size(w.B, w.T, w.H, w.dk, w.dv), dtype=torch.uint8, device=dev)
    args = (g["q"], g["k"], g["v"], g["beta"], g["dt"], g["A"], g["I_prior"])
    y = torch.empty(w.B, w.T, w.H, w.dv, dtype=w.dtype, device=dev)
    muT = torch.empty(w.B, w.H, w.dv, w.dk, device=dev)
    IT = torch.empty_like(muT)
    out = pm.bwd(*args, gr["gy"], gmuT=gr["gmuT"], gIT=gr["gIT"], workspace=ws)

    fwd_save = lambda: pm.fwd_chunked(*args, y=y, muT=muT, IT=IT, workspace=ws, save_checkpoints=True)

    def fused():
        fwd_save()
        pm.bwd(*args, gr["gy"], gmuT=gr["gmuT"], gIT=gr["gIT"], workspace=ws, out=out, checkpoints_saved=True)

    def recompute():
        pm.fwd_chunked(*args, y=y, muT=muT, IT=IT)
        pm.bwd(*args, gr["gy"], gmuT=gr["gmuT"], gIT=gr["gIT"], workspace=ws, out=out)

    _, per_s = time_launches(fwd_save, steps, 3, torch)
    _, per_f = time_launches(fused, steps, 3, torch)
    _, per_r = time_launches(recompute, steps, 3, torch)
    mean_s = lambda per: sum(per) / len(per) / 1e3
    s_s, f_s, r_s = mean_s(per_s), mean_s(per_f), mean_s(per_r)
    ck_bytes = w.B * w.H * ((w.T + 15) // 16) * 2 * w.dv * w.dk * 4
    updates = w.B * w.H * w.T * w.dv * w.dk
    esz = 2 if w.dtype == torch.bfloat16 else 4
    return {"workload": w.name + ", training step (forward with y and final state, then the full backward)",
            "tokens_per_s": w.B * w.T / f_s, "ms_per_step": f_s * 1e3,
            "recompute_ms_per_step": r_s * 1e3,
            "roofline": roofline("alu", f_s, flops=updates * (FWD["flops"] + BWD["flops"]),
                                 nbytes=fwd_bytes(w, esz, esz) + grad_bytes(w, esz),
                                 mix=dict(valu=FWD["valu"] + BWD["valu"], flops=FWD["flops"] + BWD["flops"]),
                                 scope="whole step (checkpointing forward + backward); algorithmic bytes of the "
                                       "forward and of the backward's inputs and gradients"),
            "checkpointing_forward": {
                "ms_per_launch": s_s * 1e3, "checkpoint_GB": ck_bytes / 1e9,
                "checkpoint_write_GBs": ck_bytes / s_s / 1e9,
                "traffic": load_traffic("fwd_ckpt_layer760m_bf16_traffic.json")
                if w.name.startswith("layer760m") else None},
            "note": "checkpointing forward + backward reusing its checkpoints; "
                    "recompute_ms_per_step is plain forward + backward with its own checkpoint pass"}


def frozen_mfma_flops(w):
    """Matrix-core flops of the chunked frozen forward (64-token chunks): per
    chunk Q S^T, the masked scores Q K^T, their product with W, and the state
    update W^T K."""
    per_chunk = 2 * 64 * (2 * w.dv * w.dk + 64 * w.dk + 64 * w.dv)
    return w.B * w.H * ((w.T + 63) // 64) * per_chunk


def frozen_extra(torch, pm, w, g, steps):
    """palimpsa_fwd_frozen (importance held at I_prior) on the same workload."""
    y = torch.empty(w.B, w.T, w.H, w.dv, dtype=w.dtype, device=g["q"].device)
    muT = torch.empty(w.B, w.H, w.dv, w.dk, device=g["q"].device)
    fn = lambda: pm.fwd_frozen(g["q"], g["k"], g["v"], g["beta"], g["dt"], g["A"], g["I_prior"], y=y, muT=muT)
    _, per = time_launches(fn, steps, 10, torch)
    avg_s = sum(per) / len(per) / 1e3
    esz = 2 if w.dtype == torch.bfloat16 else 4
    hbm = w.B * w.T * w.H * (2 * w.dk + 2 * w.dv + 1 + w.dv) * esz + 4 * w.B * w.H * w.dv * w.dk
    return {"workload": w.name + ", frozen importance (Mamba2 limit) on MFMA",
            "tokens_per_s": w.B * w.T / avg_s, "ms_per_launch": avg_s * 1e3,
            "roofline": roofline("hbm", avg_s, nbytes=hbm, mfma_flops=frozen_mfma_flops(w),
                                 traffic=load_traffic("frozen_fwd_layer760m_bf16_traffic.json")
                                 if w.name.startswith("layer760m") else None,
                                 kernel="frozen_fwd_kernel<%d>" % w.dk)}


def frozen_backward_extra(torch, pm, workloads, w, g, steps):
    """palimpsa_bwd_frozen (backward of the frozen-importance recurrence) on the
    same workload, timed as one call.  bf16 inputs with d = 64 or 128 take the
    chunked matrix-core form (state and adjoint walk over the chunks, per-chunk
    gradients, batch sums); its roofline is HBM, over the bytes the call must
    move (inputs and gradients; the chunk-boundary states it passes between its
    kernels are extra traffic)."""
    dev = g["q"].device
    gr = workloads.upstream_grads(w.B, w.T, w.H, w.dv, w.dk, w.dtype, seed=2)
    gy, gmuT = gr["gy"].to(dev), gr["gmuT"].to(dev)
    ws = torch.empty(pm.bwd_workspace_size(w.B, w.T, w.H, w.dk, w.dv), dtype=torch.uint8, device=dev)
    args = (g["q"], g["k"], g["v"], g["beta"], g["dt"], g["A"], g["I_prior"], gy)
    out = pm.bwd_frozen(*args, gmuT=gmuT, workspace=ws)
    fn = lambda: pm.bwd_frozen(*args, gmuT=gmuT, workspace=ws, out=out)
    _, per = time_launches(fn, steps, 3, torch)
    avg_s = sum(per) / len(per) / 1e3
    esz = 2 if w.dtype == torch.bfloat16 else 4
    alg = grad_bytes(w, esz) - 2 * w.B * w.H * w.dv * w.dk * 4     # no gIT read, no gI0 written
    nc = (w.T + 63) // 64
    boundary = 3 * w.B * w.H * nc * w.dv * w.dk * 2     # S_0^T, G_E, G_E^T per chunk, bf16
    return {"workload": w.name + ", frozen-importance backward (gq, gk, gv, gbeta, gdt, gA, gIp, gmu0)",
            "tokens_per_s": w.B * w.T / avg_s, "ms_per_call": avg_s * 1e3,
            "roofline": roofline("hbm", avg_s, nbytes=alg, mfma_flops=3 * frozen_mfma_flops(w),
                                 traffic=load_traffic("frozen_bwd_layer760m_bf16_traffic.json")
                                 if w.name.startswith("layer760m") else None,
                                 chunk_boundary_bytes=boundary, scope="whole call (3 kernels)")}


def blockdiag_extra(torch, pm, w, g, steps, block=2):
    """palimpsa_fwd_blockdiag (2x2 or 4x4 precision blocks along the key axis)
    on the same workload."""
    y, muT, PT = pm.fwd_blockdiag(g["q"], g["k"], g["v"], g["beta"], g["dt"], g["A"], g["I_prior"], block=block)
    fn = lambda: pm.fwd_blockdiag(g["q"], g["k"], g["v"], g["beta"], g["dt"], g["A"], g["I_prior"], block=block,
                                  y=y, muT=muT, PT=PT)
    _, per = time_launches(fn, steps, 5, torch)
    avg_s = sum(per) / len(per) / 1e3
    entries = w.B * w.H * w.T * w.dv * w.dk
    mix = BD2 if block == 2 else BD4
    esz = 2 if w.dtype == torch.bfloat16 else 4
    state = w.B * w.H * w.dv * w.dk * 4 * (1 + (block + 1) / 2)     # mu + upper triangle of P
    return {"workload": w.name + ", %dx%d block-diagonal precision" % (block, block),
            "tokens_per_s": w.B * w.T / avg_s, "ms_per_launch": avg_s * 1e3,
            "roofline": roofline("alu", avg_s, flops=entries * mix["flops"],
                                 nbytes=w.B * w.T * w.H * (2 * w.dk + 3 * w.dv + 1) * esz + state, mix=mix,
                                 traffic=load_traffic("bd%d_fwd_layer760m_bf16_traffic.json" % block)
                                 if w.name.startswith("layer760m") else None,
                                 kernel="bd%d_fwd_kernel<%d, C, bf16, bf16>" % (block, w.dk))}


def blockdiag_backward_extra(torch, pm, workloads, w, g, steps, block=2):
    """palimpsa_bwd_blockdiag (backward of the block-diagonal path) on the
    same workload, timed as one call (checkpoint pass, reverse walk, three
    finishing kernels)."""
    dev = g["q"].device
    gr = workloads.upstream_grads(w.B, w.T, w.H, w.dv, w.dk, w.dtype, seed=2)
    gy, gmuT = gr["gy"].to(dev), gr["gmuT"].to(dev)
    ws = torch.empty(pm.bwd_blockdiag_workspace_size(w.B, w.T, w.H, w.dk, w.dv, block), dtype=torch.uint8,
                     device=dev)
    args = (g["q"], g["k"], g["v"], g["beta"], g["dt"], g["A"], g["I_prior"], gy)
    out = pm.bwd_blockdiag(*args, block=block, gmuT=gmuT, workspace=ws)
    fn = lambda: pm.bwd_blockdiag(*args, block=block, gmuT=gmuT, workspace=ws, out=out)
    _, per = time_launches(fn, steps, 2, torch)
    avg_s = sum(per) / len(per) / 1e3
    entries = w.B * w.H * w.T * w.dv * w.dk
    mix = BD2_BWD if block == 2 else BD4_BWD
    # one training step: the forward that stores the checkpoints, then the
    # backward that reuses them; beside it the plain forward and a backward
    # that recomputes them
    fargs = args[:7]
    y, muT, PT = pm.fwd_blockdiag(*fargs, block=block)

    def fused():
        pm.fwd_blockdiag(*fargs, block=block, y=y, muT=muT, PT=PT, save_checkpoints=True, workspace=ws)
        pm.bwd_blockdiag(*args, block=block, gmuT=gmuT, workspace=ws, out=out, checkpoints_saved=True)

    def recompute():
        pm.fwd_blockdiag(*fargs, block=block, y=y, muT=muT, PT=PT)
        fn()

    _, per_f = time_launches(fused, steps, 2, torch)
    _, per_r = time_launches(recompute, steps, 2, torch)
    f_s, r_s = sum(per_f) / len(per_f) / 1e3, sum(per_r) / len(per_r) / 1e3
    return {"workload": w.name + ", %dx%d block-diagonal backward (gq, gk, gv, gbeta, gdt, gA, gIp, gmu0, gP0)"
            % (block, block),
            "tokens_per_s": w.B * w.T / avg_s, "ms_per_call": avg_s * 1e3,
            "workspace_GB": ws.numel() / 1e9,
            "training_step_ms": f_s * 1e3, "recompute_training_step_ms": r_s * 1e3,
            "roofline": roofline("alu", avg_s, flops=entries * mix["flops"], mix=mix,
                                 traffic=load_traffic("bd%d_bwd_layer760m_bf16_traffic.json" % block)
                                 if w.name.startswith("layer760m") else None,
                                 scope="whole call (5 kernels); per-kernel split in the committed trace")}


def forward_config_extra(torch, pm, workloads, key, steps):
    """The chunked forward on another of the workloads (the MQAR-scale fp32
    layer, the 32k-token context and its beta = 1e-6 variant), in the launch
    configuration the library picks for it (a time split where B*H is small),
    timed as one call."""
    w = workloads.WORKLOADS[key]
    dev = torch.device("cuda:0")
    inp = workloads.make_inputs(w)
    g = {n: (x.to(dev) if isinstance(x, torch.Tensor) else x) for n, x in inp.items()}
    y = torch.empty(w.B, w.T, w.H, w.dv, dtype=w.dtype, device=dev)
    muT = torch.empty(w.B, w.H, w.dv, w.dk, device=dev)
    IT = torch.empty_like(muT)
    nws = pm.workspace_size(w.B, w.T, w.H, w.dk, w.dv, 0)
    ws = torch.empty(max(nws, 1), dtype=torch.uint8, device=dev)
    fn = lambda: pm.fwd_chunked(g["q"], g["k"], g["v"], g["beta"], g["dt"], g["A"], g["I_prior"],
                                chunk=w.chunk, y=y, muT=muT, IT=IT, workspace=ws if nws else None)
    _, per = time_launches(fn, steps, 3, torch)
    avg_s = sum(per) / len(per) / 1e3
    updates = w.B * w.H * w.T * w.dv * w.dk
    esz = 2 if w.dtype == torch.bfloat16 else 4
    # workspace floats: (nseg - 1) summaries of 2 bh dv dk + bh, a start-state copy of 2 bh dv dk
    bh = w.B * w.H
    nseg = (nws // 4 + bh) // (2 * bh * w.dv * w.dk + bh) if nws else 1
    del g, inp
    return {"workload": w.name + ", chunked forward", "tokens_per_s": w.B * w.T / avg_s,
            "ms_per_call": avg_s * 1e3, "segments": nseg, "chunk": w.chunk,
            "roofline": roofline("alu", avg_s, flops=updates * FWD["flops"], nbytes=fwd_bytes(w, esz, esz),
                                 mix=FWD, traffic=None,
                                 scope="whole call" + (" (summary pass + replay pass)" if nseg > 1 else ""))}


def fig7_extra(torch, pm, workloads, dev, D, steps):
    """One head as wide as the model, the shape of the pages' recurrent-kernel
    measurement (B=16, L=2048, H=1, d_k = d_v = D; bf16 inputs, fp32 state),
    through the chunked forward with its workspace: the row-parallel form (a
    prep pass of column records, the recurrence with the state in registers for
    the whole sequence, and the sum over column slices)."""
    w = workloads.WORKLOADS[2].with_(name="recurrent-shape B16 L2048 H1 D%d" % D, B=16, T=2048, H=1, dk=D, dv=D)
    inp = workloads.make_inputs(w, seed=70 + D // 512)
    g = {n: (x.to(dev) if isinstance(x, torch.Tensor) else x) for n, x in inp.items()}
    y = torch.empty(w.B, w.T, w.H, w.dv, dtype=w.dtype, device=dev)
    muT = torch.empty(w.B, w.H, w.dv, w.dk, device=dev)
    IT = torch.empty_like(muT)
    nws = pm.workspace_size(w.B, w.T, w.H, w.dk, w.dv)
    ws = torch.empty(nws, dtype=torch.uint8, device=dev) if nws else None
    fn = lambda: pm.fwd_chunked(g["q"], g["k"], g["v"], g["beta"], g["dt"], g["A"], g["I_prior"], y=y, muT=muT, IT=IT,
                                workspace=ws)
    _, per = time_launches(fn, steps, 2, torch)
    avg_s = sum(per) / len(per) / 1e3
    updates = w.B * w.H * w.T * w.dv * w.dk
    kcl = 32 if D >= 1024 else 16
    return {"workload": w.name, "tokens_per_s": w.B * w.T / avg_s, "ms_per_launch": avg_s * 1e3,
            "state_updates_per_s": updates / avg_s, "workspace_bytes": nws,
            "roofline": roofline("alu", avg_s, flops=updates * FWD["flops"], nbytes=fwd_bytes(w, 2, 2), mix=FWD,
                                 traffic=load_traffic("wide_rows_recurrent_shape_D2048_bf16_traffic.json")
                                 if D == 2048 else None,
                                 kernel="wide_prep_kernel<bf16> + wide_rows_kernel<%d, bf16> + wide_sum_kernel<bf16>"
                                        % kcl, scope="whole call")}


EXTRAS = ("decode", "backward", "training_step", "frozen", "frozen_backward", "blockdiag", "blockdiag_decode",
          "blockdiag4", "blockdiag_backward", "blockdiag4_backward", "recurrent_shape", "configs")


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[1])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-heads", type=int, default=0,
                    help="heads in the oracle sample (0: all heads of the workload)")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-extras", action="store_true", help="skip every object beside the headline forward")
    ap.add_argument("--only", default="",
                    help="comma-separated subset of the extra objects to run (%s)" % ", ".join(EXTRAS))
    ap.add_argument("--chunk", type=int, default=0)
    ap.add_argument("--workload", default="2",
                    help="forward workload to time: 2 (760M layer, default), 0, 1, 4 or 4b")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB three times "
                         "(calibrates the HBM byte counters) and exit")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(heads shard across GPUs with no communication; see the design notes). "
              "Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    import bayesian_metaplastic_memory_amd as pm
    import workloads

    dev = torch.device("cuda:0")
    if args.copy_probe:
        n = args.copy_probe * (1 << 20) // 4
        src = torch.ones(n, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes_each_way": 4 * n, "launches": 3}))
        return
    t_start = time.time()
    w = workloads.WORKLOADS[int(args.workload) if args.workload.isdigit() else args.workload]
    inp = workloads.make_inputs(w)
    g = {n: (x.to(dev) if isinstance(x, torch.Tensor) else x) for n, x in inp.items()}
    y = torch.empty(w.B, w.T, w.H, w.dv, dtype=w.dtype, device=dev)
    muT = torch.empty(w.B, w.H, w.dv, w.dk, device=dev)
    IT = torch.empty_like(muT)
    args_fwd = (g["q"], g["k"], g["v"], g["beta"], g["dt"], g["A"], g["I_prior"])
    fn = lambda: pm.fwd_chunked(*args_fwd, chunk=args.chunk, y=y, muT=muT, IT=IT)

    total_ms, per = time_launches(fn, args.steps, args.warmup, torch)
    avg_launch_s = sum(per) / len(per) / 1e3
    tokens = w.B * w.T
    updates = w.B * w.H * w.T * w.dv * w.dk
    traffic = load_traffic("fwd_chunked_layer760m_bf16_traffic.json") if args.workload == "2" else None
    esz = 2 if w.dtype == torch.bfloat16 else 4
    tname = str(w.dtype).replace("torch.", "").replace("bfloat16", "bf16")
    out = {
        "metric": "tokens/s of Palimpsa chunked forward (B*T/s) and % of HBM/MFMA roofline",
        "value": tokens * args.steps / (total_ms / 1e3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": total_ms / args.steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": w.name + ", chunked forward", "B": w.B, "H": w.H,
                   "T": w.T, "d_k": w.dk, "d_v": w.dv, "chunk": args.chunk or "auto",
                   "inputs": str(w.dtype).replace("torch.", ""), "state": "fp32",
                   "global_batch": w.B, "seq_len": w.T},
        "roofline": roofline("alu", avg_launch_s, flops=updates * FWD["flops"], nbytes=fwd_bytes(w, esz, esz),
                             mix=FWD, traffic=traffic,
                             kernel="fwd_chunked_kernel<%d, C, %s, %s>" % (w.dk, tname, tname),
                             avg_launch_ms=avg_launch_s * 1e3,
                             per_update="4 FMA + 2 MUL (10 flops) + 1 v_rcp_f32"),
    }
    def progress(name):
        print("[bench] %s done, %.1f s" % (name, time.time() - t_start), file=sys.stderr, flush=True)

    progress("forward")
    want = set(EXTRAS) if not args.only else set(args.only.split(","))
    if args.no_extras:
        want = set()
    if args.no_decode:
        want.discard("decode")
    if "decode" in want:
        out["decode"] = decode_extra(torch, pm, workloads, max(64, args.steps))
        progress("decode")
    if w.dtype == torch.bfloat16:
        few = max(5, args.steps // 5)
        if "backward" in want:
            out["backward"] = backward_extra(torch, pm, workloads, w, g, few)
            progress("backward")
        if "training_step" in want:
            out["training_step"] = training_extra(torch, pm, workloads, w, g, few)
            progress("training_step")
        if "frozen" in want:
            out["frozen"] = frozen_extra(torch, pm, w, g, max(20, args.steps))
            progress("frozen")
        if "frozen_backward" in want:
            out["frozen_backward"] = frozen_backward_extra(torch, pm, workloads, w, g, few)
            progress("frozen_backward")
        if "blockdiag" in want:
            out["blockdiag"] = blockdiag_extra(torch, pm, w, g, max(20, args.steps // 2))
            progress("blockdiag")
        if "blockdiag_decode" in want:
            out["blockdiag_decode"] = blockdiag_decode_extra(torch, pm, workloads, max(64, args.steps))
            progress("blockdiag_decode")
        if "blockdiag4" in want:
            out["blockdiag4"] = blockdiag_extra(torch, pm, w, g, max(10, args.steps // 5), block=4)
            progress("blockdiag4")
        if "blockdiag_backward" in want:
            out["blockdiag_backward"] = blockdiag_backward_extra(torch, pm, workloads, w, g, few)
            progress("blockdiag_backward")
        if "blockdiag4_backward" in want:
            out["blockdiag4_backward"] = blockdiag_backward_extra(torch, pm, workloads, w, g, few, block=4)
            progress("blockdiag4_backward")
        if "recurrent_shape" in want:
            out["recurrent_shape"] = [fig7_extra(torch, pm, workloads, dev, D, 5) for D in (512, 2048)]
            progress("recurrent_shape")
    if "configs" in want:
        del g
        torch.cuda.empty_cache()
        out["configs"] = {str(key): forward_config_extra(torch, pm, workloads, key, max(10, args.steps // 2))
                          for key in (1, 4, "4b") if str(key) != args.workload}
        progress("configs")
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(inp, w, args.cpu_heads or w.B * w.H)
        progress("cpu_baseline")
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
