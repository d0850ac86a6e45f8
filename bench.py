#!/usr/bin/env python3
"""Benchmark of the Palimpsa chunked forward on one MI355X.

One step = one palimpsa_fwd_chunked pass over the 760M-model layer workload
(B=8, H=12, T=4096, d_k=d_v=128, bf16 inputs and output, float32 state),
inputs resident in HBM.  Prints ONE JSON line.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]

The roofline object reports the chunked-forward kernel against the FP32
vector-ALU issue roof (the binding one: the readout divides by a per-token,
per-entry precision, so there is no dense contraction for the matrix cores,
and the kernel needs only a few hundred GB/s of HBM).  Per state-entry update
the method needs 4 FMA + 2 MUL + 1 reciprocal = 10 flops + 1 rcp.
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

# Chip constants used by the ALU roof (MI355X: 256 CUs x 4 SIMDs, each SIMD
# issuing one wave64 FP32 VALU instruction every 4 clocks = 16 lane-ops/clk,
# at the 2.4 GHz peak engine clock).  Packed FP32 is not used by this build,
# so one FMA is one lane-op.
CUS, SIMDS, LANES_PER_CLK, CLOCK_HZ = 256, 4, 16, 2.4e9
LANE_OPS_PER_S = CUS * SIMDS * LANES_PER_CLK * CLOCK_HZ       # 3.93e13
VALU_PER_UPDATE = 6          # 4 FMA + 2 MUL
RCP_SLOTS = 2                # v_rcp_f32 issue cost in FMA slots: half rate on gfx950
FLOPS_PER_UPDATE = 10        # FMA = 2 flops, MUL = 1; the reciprocal is not counted
HBM_PEAK_GBS = 8000.0
# Backward per state entry and token: replay of the update (2 FMA + MUL + FMA
# = 4 VALU, 7 flops) and the reverse step (16 VALU = 22 flops, plus one
# v_rcp_f32 = 2 slots): 22 issue slots, 29 flops.
BWD_SLOTS_PER_UPDATE = 22
BWD_FLOPS_PER_UPDATE = 29
# 2x2 block-diagonal precision, per block of two entries and token: precision
# 2 + 2 + 3 VALU, content 4, determinant 2, solve 6, readout 2 = 21 VALU
# (33 flops) plus one v_rcp_f32 (2 slots): 11.5 slots and 16.5 flops per entry.
BD2_SLOTS_PER_ENTRY = 11.5
BD2_FLOPS_PER_ENTRY = 16.5
# 4x4 blocks, per block and token: update 34 VALU (52 flops), Cholesky solve
# 36 VALU (58 flops) plus four v_rsq_f32 (2 slots each), readout 4 FMA:
# 82 slots and 118 flops per block, 20.5 slots and 29.5 flops per entry.
BD4_SLOTS_PER_ENTRY = 20.5
BD4_FLOPS_PER_ENTRY = 29.5
# Backward of the 2x2 path, per entry and token: one replay of the update
# (11 VALU, 18 flops per block) and the reverse step per block (determinant
# and solves 16 VALU + one v_rcp_f32, adjoint updates 19, gradient terms 15:
# 50 VALU and 2 rcp slots, 72 flops): 31.5 slots and 45 flops per entry.
BD2_BWD_SLOTS_PER_ENTRY = 31.5
BD2_BWD_FLOPS_PER_ENTRY = 45
# 4x4 blocks, per block and token: one replay of the update (34 VALU, 52
# flops) and the reverse step (Cholesky factor 16 VALU + 4 v_rsq_f32, two
# solves 40, G_h, S and the gradient terms 104: 160 VALU and 8 rsq slots,
# 248 flops): 50.5 slots and 75 flops per entry.
BD4_BWD_SLOTS_PER_ENTRY = 50.5
BD4_BWD_FLOPS_PER_ENTRY = 75


def alu_peak_tflops():
    updates_per_s = LANE_OPS_PER_S / (VALU_PER_UPDATE + RCP_SLOTS)
    return updates_per_s * FLOPS_PER_UPDATE / 1e12


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


def bwd_peak_tflops():
    return LANE_OPS_PER_S / BWD_SLOTS_PER_UPDATE * BWD_FLOPS_PER_UPDATE / 1e12


def bd2_peak_tflops():
    return LANE_OPS_PER_S / BD2_SLOTS_PER_ENTRY * BD2_FLOPS_PER_ENTRY / 1e12


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


def cpu_baseline(inp, w, max_heads):
    import numpy as np
    import oracle
    heads = [(b, h) for b in range(w.B) for h in range(w.H)][:max_heads]
    sub = oracle.select_heads(inp, heads)
    threads = oracle.max_threads()
    t0 = time.perf_counter()
    oracle.fwd(**sub, nthreads=threads)
    wall = time.perf_counter() - t0
    layer_seqs = len(heads) / w.H                # sampled heads as a fraction of B sequences
    return {"value": layer_seqs * w.T / wall, "unit": "tokens/s", "cores": threads,
            "kind": "oracle",
            "sample": "%d of %d heads (b,h) at full T=%d, float64 sequential Eq. (5), "
                      "OpenMP over heads; %.1f s wall" % (len(heads), w.B * w.H, w.T, wall)}


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
    # A decode kernel takes ~85 us, less than the Python binding needs to
    # submit it, so the timed loop replays a captured graph of 16 steps (the
    # launches contain no memsets or allocations) and reports per-step time.
    per_graph = 16
    fn()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(per_graph):
            fn()
    total_ms, per = time_launches(graph.replay, max(2, steps // per_graph), 3, torch)
    avg_s = sum(per) / len(per) / 1e3 / per_graph
    state_bytes = 16 * w.B * w.H * w.dv * w.dk
    in_bytes = 2 * w.B * w.H * (2 * w.dk + 2 * w.dv + 1) + 2 * w.B * w.H * w.dv
    return {"workload": "decode B=64 H=32 d_k=d_v=128, bf16 inputs, fp32 state",
            "tokens_per_s": w.B / avg_s, "us_per_step": avg_s * 1e6,
            "timing": "HIP graph of 16 steps, replayed",
            "roofline": {"bound": "hbm", "achieved": (state_bytes + in_bytes) / avg_s / 1e9,
                         "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": (state_bytes + in_bytes) / avg_s / 1e9 / HBM_PEAK_GBS,
                         "traffic": load_traffic("step_kernel_decode_B64_H32_d128_traffic.json")}}


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
    per_graph = 16                       # as decode_extra: a captured graph of 16 steps, replayed
    fn()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(per_graph):
            fn()
    _, per = time_launches(graph.replay, max(2, steps // per_graph), 3, torch)
    avg_s = sum(per) / len(per) / 1e3 / per_graph
    state_bytes = 2 * 12 * w.B * w.H * w.dv * w.dk
    in_bytes = 2 * w.B * w.H * (2 * w.dk + 2 * w.dv + 1) + 2 * w.B * w.H * w.dv
    return {"workload": "2x2 block-diagonal decode B=64 H=32 d_k=d_v=128, bf16 inputs, fp32 state",
            "tokens_per_s": w.B / avg_s, "us_per_step": avg_s * 1e6,
            "timing": "HIP graph of 16 steps, replayed",
            "roofline": {"bound": "hbm", "achieved": (state_bytes + in_bytes) / avg_s / 1e9,
                         "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": (state_bytes + in_bytes) / avg_s / 1e9 / HBM_PEAK_GBS,
                         "traffic": load_traffic("bd2_step_decode_B64_H32_d128_traffic.json")}}


def backward_extra(torch, pm, workloads, w, g, steps):
    """palimpsa_bwd on the same workload: checkpoint pass, backward kernel and
    the three finishing kernels, timed as one call."""
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
    achieved = updates * BWD_FLOPS_PER_UPDATE / avg_s / 1e12
    return {"workload": w.name + ", backward (gq, gk, gv, gbeta, gdt, gA, gIp, gmu0, gI0)",
            "tokens_per_s": w.B * w.T / avg_s, "ms_per_call": avg_s * 1e3,
            "workspace_GB": ws.numel() / 1e9,
            "roofline": {"bound": "alu", "achieved": achieved, "peak": bwd_peak_tflops(), "unit": "TFLOP/s",
                         "frac": achieved / bwd_peak_tflops(),
                         "traffic": load_traffic("bwd_layer760m_bf16_traffic.json") if w.name.startswith("layer760m") else None,
                         "scope": "whole call (5 kernels); per-kernel split in the committed trace",
                         "per_update": "replay 4 VALU + reverse 16 VALU + 1 v_rcp_f32 = 22 slots, 29 flops"}}


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
    ck_bytes = w.B * w.H * ((w.T + 7) // 8) * 2 * w.dv * w.dk * 4
    return {"workload": w.name + ", training step (forward with y and final state, then the full backward)",
            "tokens_per_s": w.B * w.T / f_s, "ms_per_step": f_s * 1e3,
            "recompute_ms_per_step": r_s * 1e3,
            "checkpointing_forward": {
                "ms_per_launch": s_s * 1e3, "checkpoint_GB": ck_bytes / 1e9,
                "checkpoint_write_GBs": ck_bytes / s_s / 1e9,
                "traffic": load_traffic("fwd_ckpt_layer760m_bf16_traffic.json")
                if w.name.startswith("layer760m") else None},
            "note": "checkpointing forward + backward reusing its checkpoints; "
                    "recompute_ms_per_step is plain forward + backward with its own checkpoint pass"}


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
            "roofline": {"bound": "hbm", "achieved": hbm / avg_s / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": hbm / avg_s / 1e9 / HBM_PEAK_GBS,
                         "traffic": load_traffic("frozen_fwd_layer760m_bf16_traffic.json") if w.name.startswith("layer760m") else None,
                         "algorithmic_bytes": hbm}}


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
    btok = w.B * w.T * w.H
    state = w.B * w.H * w.dv * w.dk * 4
    # read q, k, v, beta, gy, dt and gmuT; write gq, gk, gv, gbeta, gdt (fp32) and gmu0
    alg = btok * ((2 * w.dk + 3 * w.dv + 1) * esz + (2 * w.dk + 2 * w.dv + 1) * 4) + 2 * state
    nc = (w.T + 63) // 64
    boundary = 3 * w.B * w.H * nc * w.dv * w.dk * 2     # S_0^T, G_E, G_E^T per chunk, bf16
    return {"workload": w.name + ", frozen-importance backward (gq, gk, gv, gbeta, gdt, gA, gIp, gmu0)",
            "tokens_per_s": w.B * w.T / avg_s, "ms_per_call": avg_s * 1e3,
            "roofline": {"bound": "hbm", "achieved": alg / avg_s / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": alg / avg_s / 1e9 / HBM_PEAK_GBS,
                         "traffic": load_traffic("frozen_bwd_layer760m_bf16_traffic.json")
                         if w.name.startswith("layer760m") else None,
                         "algorithmic_bytes": alg,
                         "chunk_boundary_bytes": boundary,
                         "scope": "whole call (3 kernels)"}}


def blockdiag_extra(torch, pm, w, g, steps):
    """palimpsa_fwd_blockdiag (2x2 precision blocks along the key axis) on the same workload."""
    y, muT, PT = pm.fwd_blockdiag(g["q"], g["k"], g["v"], g["beta"], g["dt"], g["A"], g["I_prior"], block=2)
    fn = lambda: pm.fwd_blockdiag(g["q"], g["k"], g["v"], g["beta"], g["dt"], g["A"], g["I_prior"], block=2,
                                  y=y, muT=muT, PT=PT)
    _, per = time_launches(fn, steps, 10, torch)
    avg_s = sum(per) / len(per) / 1e3
    entries = w.B * w.H * w.T * w.dv * w.dk
    achieved = entries * BD2_FLOPS_PER_ENTRY / avg_s / 1e12
    return {"workload": w.name + ", 2x2 block-diagonal precision",
            "tokens_per_s": w.B * w.T / avg_s, "ms_per_launch": avg_s * 1e3,
            "roofline": {"bound": "alu", "achieved": achieved, "peak": bd2_peak_tflops(), "unit": "TFLOP/s",
                         "frac": achieved / bd2_peak_tflops(),
                         "traffic": load_traffic("bd2_fwd_layer760m_bf16_traffic.json")
                         if w.name.startswith("layer760m") else None,
                         "per_entry": "10.5 VALU + 0.5 v_rcp_f32 = 11.5 slots, 16.5 flops"}}


def blockdiag4_extra(torch, pm, w, g, steps):
    """palimpsa_fwd_blockdiag with 4x4 precision blocks on the same workload."""
    y, muT, PT = pm.fwd_blockdiag(g["q"], g["k"], g["v"], g["beta"], g["dt"], g["A"], g["I_prior"], block=4)
    fn = lambda: pm.fwd_blockdiag(g["q"], g["k"], g["v"], g["beta"], g["dt"], g["A"], g["I_prior"], block=4,
                                  y=y, muT=muT, PT=PT)
    _, per = time_launches(fn, steps, 5, torch)
    avg_s = sum(per) / len(per) / 1e3
    entries = w.B * w.H * w.T * w.dv * w.dk
    peak = LANE_OPS_PER_S / BD4_SLOTS_PER_ENTRY * BD4_FLOPS_PER_ENTRY / 1e12
    achieved = entries * BD4_FLOPS_PER_ENTRY / avg_s / 1e12
    return {"workload": w.name + ", 4x4 block-diagonal precision",
            "tokens_per_s": w.B * w.T / avg_s, "ms_per_launch": avg_s * 1e3,
            "roofline": {"bound": "alu", "achieved": achieved, "peak": peak, "unit": "TFLOP/s",
                         "frac": achieved / peak,
                         "traffic": load_traffic("bd4_fwd_layer760m_bf16_traffic.json")
                         if w.name.startswith("layer760m") else None,
                         "per_entry": "18.5 VALU + 1 v_rsq_f32 = 20.5 slots, 29.5 flops"}}


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
    slots, flops = ((BD2_BWD_SLOTS_PER_ENTRY, BD2_BWD_FLOPS_PER_ENTRY) if block == 2 else
                    (BD4_BWD_SLOTS_PER_ENTRY, BD4_BWD_FLOPS_PER_ENTRY))
    peak = LANE_OPS_PER_S / slots * flops / 1e12
    achieved = entries * flops / avg_s / 1e12
    per_entry = ("replay 5.5 + reverse 25 VALU + 0.5 v_rcp_f32 = 31.5 slots, 45 flops" if block == 2 else
                 "replay 8.5 + reverse 40 VALU + 1 v_rsq_f32 = 50.5 slots, 75 flops")
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
            "roofline": {"bound": "alu", "achieved": achieved, "peak": peak, "unit": "TFLOP/s",
                         "frac": achieved / peak,
                         "traffic": load_traffic("bd%d_bwd_layer760m_bf16_traffic.json" % block)
                         if w.name.startswith("layer760m") else None,
                         "scope": "whole call (5 kernels); per-kernel split in the committed trace",
                         "per_entry": per_entry}}


def fig7_extra(torch, pm, workloads, dev, D, steps):
    """One head as wide as the model, the shape of the pages' recurrent-kernel
    measurement (B=16, L=2048, H=1, d_k = d_v = D; bf16 inputs, fp32 state),
    through the chunked forward (the state stays on chip for the whole
    sequence, as in a recurrent kernel)."""
    w = workloads.WORKLOADS[2].with_(name="recurrent-shape B16 L2048 H1 D%d" % D, B=16, T=2048, H=1, dk=D, dv=D)
    inp = workloads.make_inputs(w, seed=70 + D // 512)
    g = {n: (x.to(dev) if isinstance(x, torch.Tensor) else x) for n, x in inp.items()}
    y = torch.empty(w.B, w.T, w.H, w.dv, dtype=w.dtype, device=dev)
    muT = torch.empty(w.B, w.H, w.dv, w.dk, device=dev)
    IT = torch.empty_like(muT)
    fn = lambda: pm.fwd_chunked(g["q"], g["k"], g["v"], g["beta"], g["dt"], g["A"], g["I_prior"], y=y, muT=muT, IT=IT)
    _, per = time_launches(fn, steps, 2, torch)
    avg_s = sum(per) / len(per) / 1e3
    updates = w.B * w.H * w.T * w.dv * w.dk
    achieved = updates * FLOPS_PER_UPDATE / avg_s / 1e12
    return {"workload": w.name, "tokens_per_s": w.B * w.T / avg_s, "ms_per_launch": avg_s * 1e3,
            "state_updates_per_s": updates / avg_s,
            "roofline": {"bound": "alu", "achieved": achieved, "peak": alu_peak_tflops(), "unit": "TFLOP/s",
                         "frac": achieved / alu_peak_tflops(), "traffic": None}}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[1])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-heads", type=int, default=0,
                    help="heads in the oracle sample (0: all heads of the workload)")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-extras", action="store_true", help="skip the backward and frozen-path timings")
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
    achieved = updates * FLOPS_PER_UPDATE / avg_launch_s / 1e12
    peak = alu_peak_tflops()
    traffic = load_traffic("fwd_chunked_layer760m_bf16_traffic.json") if args.workload == "2" else None
    esz = 2 if w.dtype == torch.bfloat16 else 4
    hbm_alg = (w.B * w.T * w.H * (2 * w.dk + 2 * w.dv + 1 + w.dv) * esz
               + 8 * w.B * w.H * w.dv * w.dk)
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
        "roofline": {"bound": "alu", "achieved": achieved, "peak": peak, "unit": "TFLOP/s",
                     "frac": achieved / peak, "traffic": traffic,
                     "kernel": "fwd_chunked_kernel<%d, C, %s, %s>" % (w.dk, *(2 * [str(w.dtype)[6:]])),
                     "avg_launch_ms": avg_launch_s * 1e3,
                     "per_update": "4 FMA + 2 MUL (10 flops) + 1 v_rcp_f32 (2 FMA slots)",
                     "hbm_algorithmic_GBs": hbm_alg / avg_launch_s / 1e9},
    }
    if not args.no_decode:
        out["decode"] = decode_extra(torch, pm, workloads, max(64, args.steps))
    if not args.no_extras and w.dtype == torch.bfloat16:
        out["backward"] = backward_extra(torch, pm, workloads, w, g, max(5, args.steps // 5))
        out["training_step"] = training_extra(torch, pm, workloads, w, g, max(5, args.steps // 5))
        out["frozen"] = frozen_extra(torch, pm, w, g, max(20, args.steps))
        out["frozen_backward"] = frozen_backward_extra(torch, pm, workloads, w, g, max(5, args.steps // 5))
        out["blockdiag"] = blockdiag_extra(torch, pm, w, g, max(20, args.steps // 2))
        out["blockdiag_decode"] = blockdiag_decode_extra(torch, pm, workloads, max(64, args.steps))
        out["blockdiag4"] = blockdiag4_extra(torch, pm, w, g, max(10, args.steps // 5))
        out["blockdiag_backward"] = blockdiag_backward_extra(torch, pm, workloads, w, g, max(5, args.steps // 5))
        out["blockdiag4_backward"] = blockdiag_backward_extra(torch, pm, workloads, w, g, max(5, args.steps // 5),
                                                              block=4)
        out["recurrent_shape"] = [fig7_extra(torch, pm, workloads, dev, D, 5) for D in (512, 2048)]
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(inp, w, args.cpu_heads or w.B * w.H)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
