"""GPU parity: the HIP path through the C ABI against the float64 oracle.

Small cases compare every output element; full-size workloads run the GPU on
the whole batch and the oracle on sampled heads (heads are independent, so a
sampled head's outputs are exactly that head's slice of the full run).
Every case prints its name and shape before it touches the GPU.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from parity_utils import (TOL_BF16, TOL_BWD, TOL_F32, assert_close, gpu_args, rel_err, report_per_head, to_device, to_np,
                          tol_for)

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def _pm():
    import bayesian_metaplastic_memory_amd as pm
    return pm


def _announce(what, **shape):
    print("\n[case] %s %s" % (what, " ".join("%s=%s" % kv for kv in shape.items())), flush=True)


def _run_fwd(inp, chunk=0, out_dtype=None):
    g = to_device(inp, DEV)
    y, muT, IT = _pm().fwd_chunked(*gpu_args(g), mu0=g.get("mu0"), I0=g.get("I0"),
                                   chunk=chunk, out_dtype=out_dtype)
    torch.cuda.synchronize()
    return y, muT, IT


def _compare_full(inp, y, muT, IT, tol, log=None, per_head=False, ref=None):
    y_ref, mu_ref, I_ref = oracle.fwd(**inp) if ref is None else ref
    assert_close("y", y, y_ref, tol, log)
    assert_close("muT", muT, mu_ref, tol, log)
    assert_close("IT", IT, I_ref, tol, log)
    if per_head:
        report_per_head("y", y, y_ref, (0, 2), tol)
        report_per_head("muT", muT, mu_ref, (0, 1), tol)
        report_per_head("IT", IT, I_ref, (0, 1), tol)
    return y_ref, mu_ref, I_ref


def _compare_sampled(inp, heads, y, muT, IT, tol):
    sub = oracle.select_heads(inp, heads)
    y_ref, mu_ref, I_ref = oracle.fwd(**sub, nthreads=len(heads))
    bs = [b for b, _ in heads]
    hs = [h for _, h in heads]
    y_s = to_np(y)[bs, :, hs, :].transpose(1, 0, 2)[None]       # [1, T, S, dv]
    assert_close("y (sampled heads)", y_s, y_ref, tol)
    assert_close("muT (sampled heads)", to_np(muT)[bs, hs][None], mu_ref, tol)
    assert_close("IT (sampled heads)", to_np(IT)[bs, hs][None], I_ref, tol)


# ---------------------------------------------------------------------------
# the five workloads
# ---------------------------------------------------------------------------

def test_tiny_fp32_full():
    w = workloads.WORKLOADS[0]
    _announce("fwd tiny fp32", B=w.B, H=w.H, T=w.T, d=w.dk, chunk=w.chunk)
    inp = workloads.make_inputs(w)
    y, muT, IT = _run_fwd(inp, chunk=w.chunk)
    _compare_full(inp, y, muT, IT, tol_for(w.dtype))


def test_tiny_fp32_step_sequence():
    w = workloads.WORKLOADS[0]
    _announce("step x T tiny fp32", B=w.B, H=w.H, T=w.T, d=w.dk)
    inp = workloads.make_inputs(w)
    g = to_device(inp, DEV)
    mu = torch.zeros(w.B, w.H, w.dv, w.dk, device=DEV)
    I = g["I_prior"].view(1, -1, 1, 1).expand(w.B, w.H, w.dv, w.dk).contiguous()
    ys = []
    for t in range(w.T):
        ys.append(_pm().step(g["q"][:, t].contiguous(), g["k"][:, t].contiguous(),
                             g["v"][:, t].contiguous(), g["beta"][:, t].contiguous(),
                             g["dt"][:, t].contiguous(), g["A"], g["I_prior"], mu, I))
    torch.cuda.synchronize()
    y = torch.stack(ys, dim=1)
    _compare_full(inp, y, mu, I, tol_for(w.dtype))


def test_mqar_fp32_full():
    w = workloads.WORKLOADS[1]
    _announce("fwd mqar fp32", B=w.B, H=w.H, T=w.T, d=w.dk, chunk=w.chunk)
    inp = workloads.make_inputs(w)
    y, muT, IT = _run_fwd(inp, chunk=w.chunk)
    _compare_full(inp, y, muT, IT, tol_for(w.dtype))


def test_layer760m_bf16_every_head():
    """The 760M layer at full size, every (b, h) against the oracle: y in
    bf16 (the bf16 bar), then y in float32, where only the kernels' float32
    arithmetic separates the two (held to the float32 bar, as the state)."""
    w = workloads.WORKLOADS[2]
    _announce("fwd 760M-layer bf16, every head", B=w.B, H=w.H, T=w.T, d=w.dk, chunk=w.chunk)
    inp = workloads.make_inputs(w)
    y, muT, IT = _run_fwd(inp, chunk=w.chunk)
    ref = _compare_full(inp, y, muT, IT, tol_for(w.dtype), per_head=True)
    _announce("fwd 760M-layer bf16 inputs, fp32 y, every head", B=w.B, H=w.H, T=w.T, d=w.dk)
    y32, muT32, IT32 = _run_fwd(inp, chunk=0, out_dtype=torch.float32)
    assert torch.equal(muT32, muT) and torch.equal(IT32, IT)
    _compare_full(inp, y32, muT32, IT32, TOL_F32, per_head=True, ref=ref)


def test_layer760m_bf16_default_chunk_bitwise_equal():
    """The launch the bench times (library-chosen chunk) gives the same bits."""
    w = workloads.WORKLOADS[2]
    _announce("fwd 760M-layer bf16 chunk invariance", B=w.B, H=w.H, T=w.T)
    inp = workloads.make_inputs(w)
    a = _run_fwd(inp, chunk=w.chunk)
    b = _run_fwd(inp, chunk=0)
    for x, z in zip(a, b):
        assert torch.equal(x, z)


@pytest.mark.parametrize("variant", [4, "4b"])
def test_long_context_bf16_every_head(variant):
    """32k tokens, every head (the launch the library chooses: a time split),
    with y in bf16 and in float32."""
    w = workloads.WORKLOADS[variant]
    _announce("fwd long-context bf16 %s, every head" % variant, B=w.B, H=w.H, T=w.T, d=w.dk)
    inp = workloads.make_inputs(w)
    y, muT, IT = _run_fwd(inp, chunk=w.chunk)
    ref = _compare_full(inp, y, muT, IT, tol_for(w.dtype), per_head=True)
    _announce("fwd long-context %s, fp32 y" % variant, B=w.B, H=w.H, T=w.T, d=w.dk)
    y32, muT32, IT32 = _run_fwd(inp, out_dtype=torch.float32)
    _compare_full(inp, y32, muT32, IT32, TOL_F32, per_head=True, ref=ref)
    del y32, ref
    if variant == "4b":
        # importance stays at I_prior: the Mamba2-form recurrence gives the same readout
        heads = [(0, 0), (0, 31)]
        sub = oracle.select_heads(inp, heads)
        y_lim, _ = oracle.fwd_mamba2_limit(**{n: sub[n] for n in
                                              ("q", "k", "v", "beta", "dt", "A", "I_prior")})
        y_s = to_np(y)[[0, 0], :, [0, 31], :].transpose(1, 0, 2)[None]
        e = rel_err(y_s, y_lim)
        print("  y vs Mamba2-limit recurrence: %.3e" % e, flush=True)
        assert e <= 1e-2
        Ibar = (to_np(IT) - 1.0).max()
        print("  max excess importance: %.3e" % Ibar, flush=True)
        assert Ibar < 1e-3


def test_decode_bf16_after_prefill():
    w = workloads.WORKLOADS[3]
    steps = workloads.DECODE_STEPS
    _announce("prefill + decode bf16", B=w.B, H=w.H, T=w.T, steps=steps, d=w.dk)
    inp = workloads.make_inputs(w, device=DEV)          # drawn on the GPU (2.1 GB per array)
    y_pre, mu, I = _pm().fwd_chunked(*gpu_args(inp), chunk=w.chunk)
    torch.cuda.synchronize()
    # 64 (b, h) pairs: every sequence once and every head twice
    heads = [(b, (5 * b + 3) % w.H) for b in range(w.B)]
    bs = [b for b, _ in heads]
    hs = [h for _, h in heads]
    sub_in = {}
    for n in ("q", "k", "v", "beta"):
        sub_in[n] = inp[n][bs, :, hs, :].transpose(0, 1).unsqueeze(0).cpu()   # [1, T, S, d]
    sub_in["dt"] = inp["dt"][bs, :, hs].transpose(0, 1).unsqueeze(0).cpu()
    sub_in["A"] = inp["A"][hs].cpu()
    sub_in["I_prior"] = inp["I_prior"][hs].cpu()
    y_ref, m_ref, P_ref = oracle.fwd(**sub_in)
    tol = tol_for(w.dtype)
    y_s = to_np(y_pre[bs, :, hs, :].transpose(0, 1).unsqueeze(0))
    assert_close("prefill y (sampled)", y_s, y_ref, tol)
    assert_close("prefill mu (sampled)", to_np(mu[bs, hs]).reshape(m_ref.shape), m_ref, tol)
    assert_close("prefill I (sampled)", to_np(I[bs, hs]).reshape(P_ref.shape), P_ref, tol)
    del inp, y_pre
    worst = 0.0
    A_s, Ip_s = sub_in["A"], sub_in["I_prior"]
    for s in range(steps):
        d = workloads.decode_inputs(w, s, device=DEV)
        y = _pm().step(d["q"], d["k"], d["v"], d["beta"], d["dt"], w_A(w, DEV), w_Ip(w, DEV), mu, I)
        ds = {n: d[n][bs, hs].unsqueeze(0).cpu() for n in ("q", "k", "v", "beta", "dt")}
        yr, m_ref, P_ref = oracle.step(ds["q"], ds["k"], ds["v"], ds["beta"], ds["dt"],
                                       A_s, Ip_s, m_ref, P_ref)
        e = rel_err(to_np(y[bs, hs]).reshape(yr.shape), yr)
        worst = max(worst, e)
        if s % 256 == 0:
            print("  step %4d y rel err %.3e" % (s, e), flush=True)
        assert e <= tol, "step %d: %.3e" % (s, e)
    torch.cuda.synchronize()
    print("  worst step y rel err %.3e" % worst, flush=True)
    assert_close("final mu (sampled)", to_np(mu[bs, hs]).reshape(m_ref.shape), m_ref, tol)
    assert_close("final I (sampled)", to_np(I[bs, hs]).reshape(P_ref.shape), P_ref, tol)


def w_A(w, dev):
    return workloads.head_constants(w)[0].to(dev)


def w_Ip(w, dev):
    return workloads.head_constants(w)[1].to(dev)


# ---------------------------------------------------------------------------
# invariances and cross-entry consistency
# ---------------------------------------------------------------------------

def test_chunk_size_is_bitwise_invariant():
    w = workloads.WORKLOADS[1].with_(B=2, H=3)
    _announce("chunk invariance", B=w.B, H=w.H, T=300, d=w.dk)
    inp = workloads.make_inputs(w, T=300)
    mu0, I0 = workloads.random_state(w.B, w.H, w.dv, w.dk, inp["I_prior"], seed=5)
    inp["mu0"], inp["I0"] = mu0, I0
    outs = [_run_fwd(inp, chunk=c) for c in (8, 16, 32, 64, 128, 0)]
    for o in outs[1:]:
        for x, z in zip(outs[0], o):
            assert torch.equal(x, z)
    _compare_full(inp, *outs[0], tol=1e-4)


def test_split_and_resume_matches_one_pass():
    w = workloads.WORKLOADS[1].with_(B=2, H=2)
    T, T1 = 257, 100
    _announce("split/resume", B=w.B, H=w.H, T=T, T1=T1, d=w.dk)
    inp = workloads.make_inputs(w, T=T)
    g = to_device(inp, DEV)
    pm = _pm()
    y, muT, IT = pm.fwd_chunked(*gpu_args(g))
    first = {n: (x[:, :T1].contiguous() if n in ("q", "k", "v", "beta", "dt") else x) for n, x in g.items()}
    second = {n: (x[:, T1:].contiguous() if n in ("q", "k", "v", "beta", "dt") else x) for n, x in g.items()}
    y1, mu1, I1 = pm.fwd_chunked(*gpu_args(first))
    # resume in place: the final state overwrites the initial state
    y2, mu2, I2 = pm.fwd_chunked(*gpu_args(second), mu0=mu1, I0=I1, muT=mu1, IT=I1)
    torch.cuda.synchronize()
    assert mu2.data_ptr() == mu1.data_ptr()
    assert rel_err(torch.cat([y1, y2], dim=1), y) <= 1e-5
    assert rel_err(mu2, muT) <= 1e-5 and rel_err(I2, IT) <= 1e-6
    _compare_full(inp, torch.cat([y1, y2], dim=1), mu2, I2, tol=1e-4)


@pytest.mark.parametrize("segments", [3, 4])
def test_split_resume_in_place_matches_out_of_place(segments):
    """A time-split forward whose final state overwrites its start state
    (muT aliasing mu0, IT aliasing I0) on a grid of several thousand
    workgroups, far more than the GPU holds at once: the last segment's rows
    finish while other segments of the same rows have not started, and the
    result must still be bitwise that of the out-of-place call."""
    w = workloads.WORKLOADS[2].with_(B=4, H=32)
    T = 1024
    _announce("split resume in place", B=w.B, H=w.H, T=T, d=w.dk, segments=segments)
    inp = workloads.make_inputs(w, T=T)
    mu0, I0 = workloads.random_state(w.B, w.H, w.dv, w.dk, inp["I_prior"], seed=11)
    g = to_device(inp, DEV)
    pm = _pm()
    nwg = w.B * w.H * (w.dv // 16) * segments
    print("  workgroups per pass: %d" % nwg, flush=True)
    y_a, mu_a, I_a = pm.fwd_chunked(*gpu_args(g), mu0=mu0.to(DEV), I0=I0.to(DEV), segments=segments)
    mu, I = mu0.to(DEV), I0.to(DEV)
    y_b, mu_b, I_b = pm.fwd_chunked(*gpu_args(g), mu0=mu, I0=I, muT=mu, IT=I, segments=segments)
    torch.cuda.synchronize()
    assert mu_b.data_ptr() == mu.data_ptr() and I_b.data_ptr() == I.data_ptr()
    assert torch.equal(y_a, y_b)
    assert torch.equal(mu_a, mu_b) and torch.equal(I_a, I_b)
    inp["mu0"], inp["I0"] = mu0, I0
    _compare_sampled(inp, [(0, 0), (3, 31), (2, 17)], y_b, mu_b, I_b, tol_for(w.dtype))


def test_step_sequence_matches_chunked():
    w = workloads.WORKLOADS[2].with_(B=2, H=3)
    T = 40
    _announce("step^T vs fwd bf16", B=w.B, H=w.H, T=T, d=w.dk)
    inp = workloads.make_inputs(w, T=T)
    g = to_device(inp, DEV)
    pm = _pm()
    y, muT, IT = pm.fwd_chunked(*gpu_args(g), out_dtype=torch.float32)
    mu = torch.zeros_like(muT)
    I = g["I_prior"].view(1, -1, 1, 1).expand_as(IT).contiguous()
    ys = [pm.step(g["q"][:, t].contiguous(), g["k"][:, t].contiguous(), g["v"][:, t].contiguous(),
                  g["beta"][:, t].contiguous(), g["dt"][:, t].contiguous(), g["A"], g["I_prior"],
                  mu, I, out_dtype=torch.float32) for t in range(T)]
    torch.cuda.synchronize()
    assert rel_err(torch.stack(ys, 1), y) <= 1e-5
    assert rel_err(mu, muT) <= 1e-5 and rel_err(I, IT) <= 1e-6


HEAD_SHAPES = [(32, 32), (32, 64), (64, 32), (64, 128), (128, 64), (32, 128), (128, 32)]


@pytest.mark.parametrize("dk,dv", HEAD_SHAPES)
@pytest.mark.parametrize("T", [1, 37])
def test_head_shapes_ragged_lengths(dk, dv, T):
    w = workloads.WORKLOADS[0].with_(B=2, H=3, dk=dk, dv=dv, A_mode="logspace16")
    _announce("fwd shapes fp32", B=w.B, H=w.H, T=T, dk=dk, dv=dv)
    inp = workloads.make_inputs(w, T=T)
    mu0, I0 = workloads.random_state(w.B, w.H, dv, dk, inp["I_prior"], seed=T + dk + dv)
    inp["mu0"], inp["I0"] = mu0, I0
    y, muT, IT = _run_fwd(inp, chunk=16)
    _compare_full(inp, y, muT, IT, tol=1e-4)


@pytest.mark.parametrize("dk,dv", [(32, 64), (128, 128), (64, 32)])
def test_step_head_shapes(dk, dv):
    w = workloads.WORKLOADS[0].with_(B=3, H=5, dk=dk, dv=dv, A_mode="logspace16")
    _announce("step shapes fp32", B=w.B, H=w.H, dk=dk, dv=dv)
    A, Ip = workloads.head_constants(w)
    mu0, I0 = workloads.random_state(w.B, w.H, dv, dk, Ip, seed=dk * dv)
    mu, I = mu0.to(DEV), I0.to(DEV)
    m, P = mu0, I0
    for s in range(3):
        d = workloads.decode_inputs(w, s)
        gd = to_device(d, DEV)
        y = _pm().step(gd["q"], gd["k"], gd["v"], gd["beta"], gd["dt"], A.to(DEV), Ip.to(DEV), mu, I)
        yr, m, P = oracle.step(d["q"], d["k"], d["v"], d["beta"], d["dt"], A, Ip, m, P)
        torch.cuda.synchronize()
        assert_close("step y", y, yr, 1e-4)
    assert_close("step mu", mu, m, 1e-4)
    assert_close("step I", I, P, 1e-4)


def test_bf16_inputs_fp32_outputs_and_fp32_inputs_bf16_outputs():
    w = workloads.WORKLOADS[2].with_(B=1, H=8)
    _announce("dtype pairs", B=w.B, H=w.H, T=70)
    inp = workloads.make_inputs(w, T=70)
    y, muT, IT = _run_fwd(inp, out_dtype=torch.float32)
    assert y.dtype == torch.float32
    _compare_full(inp, y, muT, IT, tol=1e-4)      # inputs exact in bf16, arithmetic fp32
    inp32 = {n: (x.float() if isinstance(x, torch.Tensor) else x) for n, x in inp.items()}
    y2, _, _ = _run_fwd(inp32, out_dtype=torch.bfloat16)
    assert y2.dtype == torch.bfloat16
    assert rel_err(y2, y) <= 4e-3


def test_empty_sequence_copies_state_through():
    w = workloads.WORKLOADS[0].with_(B=2, H=2)
    _announce("T=0", B=w.B, H=w.H)
    inp = workloads.make_inputs(w, T=0)
    mu0, I0 = workloads.random_state(2, 2, 32, 32, inp["I_prior"], seed=3)
    inp["mu0"], inp["I0"] = mu0, I0
    y, muT, IT = _run_fwd(inp)
    assert y.shape == (2, 0, 2, 32)
    assert torch.equal(muT.cpu(), mu0) and torch.equal(IT.cpu(), I0)
    inp["mu0"] = inp["I0"] = None
    y, muT, IT = _run_fwd(inp)
    assert torch.equal(muT.cpu(), torch.zeros_like(mu0))
    assert torch.equal(IT.cpu(), torch.ones_like(I0))


def test_no_forgetting_long_accumulation():
    """dt = 0 for 4096 tokens: importance grows to thousands; fp32 stays accurate."""
    w = workloads.WORKLOADS[0].with_(B=1, H=2, dk=64, dv=64)
    T = 4096
    _announce("alpha=1 accumulation", B=1, H=2, T=T, d=64)
    inp = workloads.make_inputs(w, T=T)
    inp["dt"] = torch.zeros_like(inp["dt"])
    y, muT, IT = _run_fwd(inp)
    _compare_full(inp, y, muT, IT, tol=1e-4)


def test_binding_reports_library_errors():
    pm = _pm()
    _announce("error paths")
    x = torch.zeros(1, 4, 1, 33, device=DEV)[..., 1:]      # offset view: not contiguous
    with pytest.raises(ValueError):
        pm.fwd_chunked(x, x, x, x, torch.zeros(1, 4, 1, device=DEV),
                       torch.ones(1, device=DEV), torch.ones(1, device=DEV))
    base = torch.zeros(1 * 4 * 1 * 32 + 1, device=DEV)
    xm = base[1:].view(1, 4, 1, 32)                          # contiguous but 4-byte offset
    dt = torch.zeros(1, 4, 1, device=DEV)
    with pytest.raises(pm.PalimpsaError) as e:
        pm.fwd_chunked(xm, xm, xm, xm, dt, torch.ones(1, device=DEV), torch.ones(1, device=DEV))
    assert e.value.status == 3
    x48 = torch.zeros(1, 4, 1, 48, device=DEV)
    with pytest.raises(pm.PalimpsaError) as e:
        pm.fwd_chunked(x48, x48, x48, x48, dt, torch.ones(1, device=DEV), torch.ones(1, device=DEV))
    assert e.value.status == 2


# ---------------------------------------------------------------------------
# time-split forward (summary pass + replay pass)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("segments", [2, 3, 5, 64])
@pytest.mark.parametrize("dk,dv,T", [(64, 64, 1000), (128, 32, 333), (32, 128, 700)])
def test_time_split_matches_oracle_and_single_pass(segments, dk, dv, T):
    w = workloads.WORKLOADS[1].with_(B=2, H=2, dk=dk, dv=dv, key_pool=0, A_mode="logspace16")
    _announce("time split", segments=segments, T=T, dk=dk, dv=dv)
    inp = workloads.make_inputs(w, T=T)
    mu0, I0 = workloads.random_state(2, 2, dv, dk, inp["I_prior"], seed=segments + T)
    inp["mu0"], inp["I0"] = mu0, I0
    g = to_device(inp, DEV)
    pm = _pm()
    assert pm.workspace_size(2, T, 2, dk, dv, segments) > 0
    y1, mu1, I1 = pm.fwd_chunked(*gpu_args(g), mu0=g["mu0"], I0=g["I0"], segments=1)
    ys, mus, Is = pm.fwd_chunked(*gpu_args(g), mu0=g["mu0"], I0=g["I0"], segments=segments)
    torch.cuda.synchronize()
    assert rel_err(ys, y1) <= 1e-5 and rel_err(mus, mu1) <= 1e-5 and rel_err(Is, I1) <= 1e-5
    _compare_full(inp, ys, mus, Is, tol=1e-4)


def test_time_split_chunk_invariance_and_bf16():
    w = workloads.WORKLOADS[4].with_(H=4, T=3000)
    _announce("time split bf16 chunk invariance", B=1, H=4, T=3000)
    inp = workloads.make_inputs(w)
    outs = [_pm().fwd_chunked(*gpu_args(to_device(inp, DEV)), segments=4, chunk=c) for c in (16, 32, 64)]
    torch.cuda.synchronize()
    for o in outs[1:]:
        for x, z in zip(outs[0], o):
            assert torch.equal(x, z)
    _compare_full(inp, *outs[0], tol=tol_for(w.dtype))


def test_time_split_requires_workspace():
    pm = _pm()
    w = workloads.WORKLOADS[0]
    _announce("time split without workspace")
    g = to_device(workloads.make_inputs(w), DEV)
    with pytest.raises(pm.PalimpsaError) as e:
        pm.fwd_chunked(*gpu_args(g), segments=3, workspace=torch.empty(0, dtype=torch.uint8, device=DEV))
    assert e.value.status == 1
    # auto with no workspace runs in one pass
    y, muT, IT = pm.fwd_chunked(*gpu_args(g), segments=0,
                                workspace=torch.empty(0, dtype=torch.uint8, device=DEV))
    torch.cuda.synchronize()
    _compare_full(workloads.make_inputs(w), y, muT, IT, tol=1e-4)


def test_long_context_auto_split_matches_single_pass():
    w = workloads.WORKLOADS[4]
    pm = _pm()
    assert pm.workspace_size(w.B, w.T, w.H, w.dk, w.dv, 0) > 0      # the auto path splits here
    _announce("long context auto split vs one pass", B=w.B, H=w.H, T=w.T)
    g = to_device(workloads.make_inputs(w), DEV)
    a = pm.fwd_chunked(*gpu_args(g), segments=0, out_dtype=torch.float32)
    b = pm.fwd_chunked(*gpu_args(g), segments=1, out_dtype=torch.float32)
    torch.cuda.synchronize()
    for x, z in zip(a, b):
        assert rel_err(x, z) <= 1e-5


def test_decode_steps_replay_in_a_hip_graph():
    """Captured decode launches replay to the same results as eager ones, every
    replay, with eager work and synchronisations in between."""
    pm = _pm()
    w = workloads.WORKLOADS[3].with_(B=4, H=4)
    _announce("decode graph replay", B=w.B, H=w.H, steps_per_graph=3, replays=4)
    A, Ip = (x.to(DEV) for x in workloads.head_constants(w))
    mu0, I0 = workloads.random_state(w.B, w.H, w.dv, w.dk, Ip.cpu(), seed=11)
    d = [to_device(workloads.decode_inputs(w, s), DEV) for s in range(3)]
    mu_g, I_g = mu0.to(DEV), I0.to(DEV)
    ys = [torch.empty(w.B, w.H, w.dv, dtype=w.dtype, device=DEV) for _ in range(3)]
    run = lambda mu, I, out: [pm.step(x["q"], x["k"], x["v"], x["beta"], x["dt"], A, Ip, mu, I, y=o)
                              for x, o in zip(d, out)]
    run(mu_g.clone(), I_g.clone(), [torch.empty_like(y) for y in ys])    # warm the binding
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run(mu_g, I_g, ys)
    mu_e, I_e = mu0.to(DEV), I0.to(DEV)
    for r in range(4):
        mu_g.copy_(mu_e)
        I_g.copy_(I_e)
        torch.cuda.synchronize()
        graph.replay()
        ye = [torch.empty_like(y) for y in ys]
        run(mu_e, I_e, ye)                      # eager reference advances from the same state
        torch.cuda.synchronize()
        for a, b in zip(ys, ye):
            assert torch.equal(a, b), "replay %d" % r
        assert torch.equal(mu_g, mu_e) and torch.equal(I_g, I_e)


@pytest.mark.parametrize("path", ["exact", "blockdiag2", "blockdiag4"])
def test_training_step_replays_in_a_hip_graph(path):
    """A captured training step (the forward that stores the checkpoints, then
    the backward that reuses them; no memsets or allocations inside) replays
    to the eager results, bitwise, every replay, with eager work and
    synchronisations in between."""
    pm = _pm()
    B, T, H, dk, dv = 2, 100, 2, 64, 48
    w = workloads.WORKLOADS[0].with_(B=B, H=H, dk=dk, dv=dv, dtype=torch.bfloat16, A_mode="logspace16")
    _announce("training step graph replay", path=path, B=B, T=T, H=H, dk=dk, dv=dv, replays=3)
    inp = workloads.make_inputs(w, T=T, seed=77)
    g = to_device(inp, DEV)
    args = gpu_args(g)
    gr = workloads.upstream_grads(B, T, H, dv, dk, torch.bfloat16, seed=77)
    gy, gmuT = gr["gy"].to(DEV), gr["gmuT"].to(DEV)
    if path == "exact":
        ws = torch.empty(pm.bwd_workspace_size(B, T, H, dk, dv), dtype=torch.uint8, device=DEV)
        fo = [torch.empty(B, T, H, dv, dtype=torch.bfloat16, device=DEV),
              torch.empty(B, H, dv, dk, device=DEV), torch.empty(B, H, dv, dk, device=DEV)]
        out = pm.bwd(*args, gy, gmuT=gmuT, workspace=ws)

        def step(fo, out):
            pm.fwd_chunked(*args, y=fo[0], muT=fo[1], IT=fo[2], workspace=ws, save_checkpoints=True)
            pm.bwd(*args, gy, gmuT=gmuT, workspace=ws, out=out, checkpoints_saved=True)
    else:
        block = 2 if path == "blockdiag2" else 4
        ws = torch.empty(pm.bwd_blockdiag_workspace_size(B, T, H, dk, dv, block), dtype=torch.uint8, device=DEV)
        fo = list(pm.fwd_blockdiag(*args, block=block))
        out = pm.bwd_blockdiag(*args, gy, block=block, gmuT=gmuT, workspace=ws)

        def step(fo, out):
            pm.fwd_blockdiag(*args, block=block, y=fo[0], muT=fo[1], PT=fo[2], save_checkpoints=True,
                             workspace=ws)
            pm.bwd_blockdiag(*args, gy, block=block, gmuT=gmuT, workspace=ws, out=out, checkpoints_saved=True)
    step(fo, out)                                   # warm the binding and the kernels
    torch.cuda.synchronize()
    ref_fo = [x.clone() for x in fo]
    ref_out = {n: x.clone() for n, x in out.items() if x is not None}
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(fo, out)
    for r in range(3):
        for x in fo:
            x.zero_()
        for x in out.values():
            if x is not None:
                x.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for a, b in zip(fo, ref_fo):
            assert torch.equal(a, b), "forward output, replay %d" % r
        for n, x in ref_out.items():
            assert torch.equal(out[n], x), "%s, replay %d" % (n, r)
        step([torch.empty_like(x) for x in fo], {n: torch.empty_like(x) for n, x in ref_out.items()})
        torch.cuda.synchronize()                    # eager work between the replays


# ---------------------------------------------------------------------------
# frozen-importance (Mamba2-limit) forward on the matrix cores
# ---------------------------------------------------------------------------

def _frozen_ref(inp, mu0=None, vstar=False):
    import numpy as np
    args = {n: inp[n] for n in ("q", "k", "v", "beta", "dt", "A", "I_prior")}
    if vstar:
        args["beta"] = np.ones(tuple(inp["v"].shape))
    return oracle.fwd_mamba2_limit(**args, mu0=mu0)


# T = 200, 100, 64, 63, 1: 4 (ragged), 2 (ragged), 1, 1 (ragged) chunks of 64 and a single token;
# the staging alternates two register sets per pair of chunks
@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 64), (128, 64), (64, 128)])
@pytest.mark.parametrize("T", [200, 100, 64, 63, 1])
def test_frozen_matches_mamba2_limit_oracle(dk, dv, T):
    w = workloads.WORKLOADS[2].with_(B=2, H=3, dk=dk, dv=dv)
    _announce("frozen fwd", T=T, dk=dk, dv=dv)
    inp = workloads.make_inputs(w, T=T)
    mu0, _ = workloads.random_state(2, 3, dv, dk, inp["I_prior"], seed=T + dk)
    g = to_device(inp, DEV)
    y, muT = _pm().fwd_frozen(*gpu_args(g), mu0=mu0.to(DEV), out_dtype=torch.float32)
    torch.cuda.synchronize()
    y_ref, mu_ref = _frozen_ref(inp, mu0=mu0)
    assert_close("frozen y", y, y_ref, 2e-2)
    assert_close("frozen muT", muT, mu_ref, 2e-2)


def test_frozen_empty_sequence_copies_state_through():
    """T = 0: no chunk runs; muT is mu0 bit for bit (zero without mu0)."""
    w = workloads.WORKLOADS[2].with_(B=2, H=3)
    _announce("frozen fwd T=0", B=2, H=3)
    inp = workloads.make_inputs(w, T=0)
    mu0, _ = workloads.random_state(2, 3, w.dv, w.dk, inp["I_prior"], seed=5)
    g = to_device(inp, DEV)
    y, muT = _pm().fwd_frozen(*gpu_args(g), mu0=mu0.to(DEV))
    torch.cuda.synchronize()
    assert tuple(y.shape) == (2, 0, 3, w.dv)
    assert torch.equal(muT.cpu(), mu0)
    y, muT = _pm().fwd_frozen(*gpu_args(g))
    torch.cuda.synchronize()
    assert torch.equal(muT.cpu(), torch.zeros_like(mu0))


def test_frozen_vstar_input_and_bf16_output():
    w = workloads.WORKLOADS[2].with_(B=1, H=4)
    T = 300
    _announce("frozen fwd v*", T=T)
    inp = workloads.make_inputs(w, T=T)
    g = to_device(inp, DEV)
    y, muT = _pm().fwd_frozen(g["q"], g["k"], g["v"], None, g["dt"], g["A"], g["I_prior"])
    torch.cuda.synchronize()
    assert y.dtype == torch.bfloat16
    y_ref, mu_ref = _frozen_ref(inp, vstar=True)
    assert_close("frozen y (v*)", y, y_ref, 2e-2)
    assert_close("frozen muT (v*)", muT, mu_ref, 2e-2)


def test_frozen_layer760m_every_head():
    """The 760M layer at full size on the matrix cores (the launch the bench
    times), every (b, h) against the oracle at the bf16 bar."""
    w = workloads.WORKLOADS[2]
    _announce("frozen fwd 760M layer, every head", B=w.B, H=w.H, T=w.T)
    inp = workloads.make_inputs(w)
    g = to_device(inp, DEV)
    y, muT = _pm().fwd_frozen(*gpu_args(g))
    torch.cuda.synchronize()
    y_ref, mu_ref = _frozen_ref(inp)
    assert_close("frozen y", y, y_ref, 2e-2)
    assert_close("frozen muT", muT, mu_ref, 2e-2)
    report_per_head("frozen y", y, y_ref, (0, 2), 2e-2)
    report_per_head("frozen muT", muT, mu_ref, (0, 1), 2e-2)


def test_frozen_agrees_with_exact_path_when_importance_stays_at_prior():
    """beta = 1e-6 with v* = beta . v fixed: the exact recurrence reaches the same readout."""
    w = workloads.WORKLOADS[2].with_(B=1, H=4)
    T = 256
    _announce("frozen vs exact at tiny beta", T=T)
    inp = workloads.make_inputs(w, T=T)
    g = to_device(inp, DEV)
    vstar = (g["beta"].float() * g["v"].float())
    beta = torch.full_like(g["beta"], 1e-6)
    v_big = (vstar / beta.float()).to(torch.bfloat16)
    vstar_eff = (beta.float() * v_big.float()).to(torch.bfloat16)      # what the exact path writes
    y_ex, _, _ = _pm().fwd_chunked(g["q"], g["k"], v_big, beta, g["dt"], g["A"], g["I_prior"],
                                   out_dtype=torch.float32)
    y_fz, _ = _pm().fwd_frozen(g["q"], g["k"], vstar_eff, None, g["dt"], g["A"], g["I_prior"],
                               out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert rel_err(y_fz, y_ex) <= 2e-2


# ---------------------------------------------------------------------------
# backward (training)
# ---------------------------------------------------------------------------

BWD_NAMES = ("gq", "gk", "gv", "gbeta", "gdt", "gA", "gIp", "gmu0", "gI0")


def _run_bwd(inp, gr, want_state=True):
    g = to_device(inp, DEV)
    gg = to_device(gr, DEV)
    out = _pm().bwd(*gpu_args(g), gg["gy"], mu0=g.get("mu0"), I0=g.get("I0"),
                    gmuT=gg.get("gmuT"), gIT=gg.get("gIT"), want_state_grads=want_state)
    torch.cuda.synchronize()
    return out


def _bwd_ref(inp, gr, nthreads=0):
    return oracle.bwd(**inp, gy=gr["gy"], gmuT=gr.get("gmuT"), gIT=gr.get("gIT"), nthreads=nthreads)


def _compare_bwd(got, ref, tol, names=BWD_NAMES, log=None):
    for n in names:
        if n in got:
            assert_close(n, got[n], ref[n], tol, log)


BWD_CASES = [
    # B, T, H, dk, dv, dtype, start state given, final-state gradients
    (1, 37, 2, 32, 32, torch.float32, True, True),
    (2, 64, 3, 64, 64, torch.float32, False, False),
    (1, 100, 2, 128, 128, torch.bfloat16, True, True),
    (2, 17, 2, 64, 128, torch.float32, True, False),
    (1, 9, 3, 128, 64, torch.bfloat16, False, True),
    (1, 1, 2, 32, 64, torch.float32, True, True),
    (2, 8, 1, 128, 32, torch.float32, False, True),
    (1, 200, 1, 32, 128, torch.bfloat16, False, False),
]


@pytest.mark.parametrize("B,T,H,dk,dv,dtype,state,final", BWD_CASES)
def test_bwd_matches_oracle(B, T, H, dk, dv, dtype, state, final):
    w = workloads.WORKLOADS[0].with_(B=B, H=H, dk=dk, dv=dv, dtype=dtype, A_mode="logspace16")
    _announce("bwd", B=B, T=T, H=H, dk=dk, dv=dv, dtype=dtype, state=state, final=final)
    inp = workloads.make_inputs(w, T=T, seed=T + dk + 3 * dv)
    if state:
        inp["mu0"], inp["I0"] = workloads.random_state(B, H, dv, dk, inp["I_prior"], seed=T + 1)
    gr = workloads.upstream_grads(B, T, H, dv, dk, dtype, seed=T + dk, final=final)
    got = _run_bwd(inp, gr)
    _compare_bwd(got, _bwd_ref(inp, gr), TOL_BWD)


def test_bwd_empty_sequence():
    w = workloads.WORKLOADS[0].with_(B=2, H=3, dk=64, dv=32)
    _announce("bwd T=0", B=2, H=3, dk=64, dv=32)
    inp = workloads.make_inputs(w, T=0)
    inp["mu0"], inp["I0"] = workloads.random_state(2, 3, 32, 64, inp["I_prior"], seed=4)
    gr = workloads.upstream_grads(2, 0, 3, 32, 64, torch.float32, seed=4)
    got = _run_bwd(inp, gr)
    assert torch.equal(got["gmu0"].cpu(), gr["gmuT"]) and torch.equal(got["gI0"].cpu(), gr["gIT"])
    assert float(got["gA"].abs().max()) == 0.0 and float(got["gIp"].abs().max()) == 0.0


def test_bwd_tiny_workload_full():
    w = workloads.WORKLOADS[0]
    _announce("bwd tiny fp32", B=w.B, H=w.H, T=w.T, d=w.dk)
    inp = workloads.make_inputs(w)
    gr = workloads.upstream_grads(w.B, w.T, w.H, w.dv, w.dk, w.dtype, seed=0)
    _compare_bwd(_run_bwd(inp, gr), _bwd_ref(inp, gr), TOL_BWD)


def test_bwd_mqar_workload_full():
    w = workloads.WORKLOADS[1]
    _announce("bwd mqar fp32", B=w.B, H=w.H, T=w.T, d=w.dk)
    inp = workloads.make_inputs(w)
    gr = workloads.upstream_grads(w.B, w.T, w.H, w.dv, w.dk, w.dtype, seed=1)
    _compare_bwd(_run_bwd(inp, gr), _bwd_ref(inp, gr), TOL_BWD)


def test_bwd_layer760m_every_head():
    """Full 760M-layer backward on the GPU (the launch the bench times)
    against the oracle on every (b, h): each gradient normwise at the float32
    bar, the per-token ones also per (b, h)."""
    w = workloads.WORKLOADS[2]
    _announce("bwd 760M layer bf16, every head", B=w.B, H=w.H, T=w.T, d=w.dk)
    inp = workloads.make_inputs(w)
    gr = workloads.upstream_grads(w.B, w.T, w.H, w.dv, w.dk, w.dtype, seed=2)
    got = _run_bwd(inp, gr)
    ref = _bwd_ref(inp, gr, nthreads=16)
    _compare_bwd(got, ref, TOL_BWD)
    for n in ("gq", "gk", "gv", "gbeta", "gdt"):
        report_per_head(n, got[n], ref[n], (0, 2), TOL_BWD)


def test_bwd_is_deterministic_and_ignores_stale_workspace():
    w = workloads.WORKLOADS[0].with_(B=2, H=2, dk=64, dv=64)
    _announce("bwd determinism", B=2, H=2, T=77, dk=64, dv=64)
    inp = workloads.make_inputs(w, T=77)
    gr = workloads.upstream_grads(2, 77, 2, 64, 64, torch.float32, seed=5)
    g = to_device(inp, DEV)
    gg = to_device(gr, DEV)
    ws = torch.full((_pm().bwd_workspace_size(2, 77, 2, 64, 64),), 0x7F, dtype=torch.uint8, device=DEV)
    a = _pm().bwd(*gpu_args(g), gg["gy"], gmuT=gg["gmuT"], gIT=gg["gIT"], workspace=ws)
    b = _pm().bwd(*gpu_args(g), gg["gy"], gmuT=gg["gmuT"], gIT=gg["gIT"])
    torch.cuda.synchronize()
    for n in BWD_NAMES:
        assert torch.equal(a[n], b[n]), n


# ---------------------------------------------------------------------------
# backward of the frozen-importance (Mamba2-limit) recurrence
# ---------------------------------------------------------------------------

FZ_BWD_NAMES = ("gq", "gk", "gv", "gbeta", "gdt", "gA", "gIp", "gmu0")


def _run_bwd_frozen(inp, gr, mu0=None, vstar=False, workspace=None):
    g = to_device(inp, DEV)
    gg = to_device(gr, DEV)
    out = _pm().bwd_frozen(g["q"], g["k"], g["v"], None if vstar else g["beta"], g["dt"], g["A"],
                           g["I_prior"], gg["gy"], mu0=None if mu0 is None else mu0.to(DEV),
                           gmuT=gg.get("gmuT"), workspace=workspace)
    torch.cuda.synchronize()
    return out


def _bwd_frozen_ref(inp, gr, mu0=None, vstar=False):
    return oracle.bwd_mamba2_limit(inp["q"], inp["k"], inp["v"], None if vstar else inp["beta"], inp["dt"],
                                   inp["A"], inp["I_prior"], gr["gy"], mu0=mu0, gmuT=gr.get("gmuT"))


def _fz_mfma(dtype, dk, dv):
    """bf16 inputs with dk in {64, 128} and dv in {64, 128, 256} take the
    matrix-core path (bf16 operands, the frozen forward's 2e-2 bar); the rest
    the float32 one."""
    return dtype == torch.bfloat16 and dk in (64, 128) and dv in (64, 128, 256)


def _fz_tol(dtype, dk, dv):
    return 2e-2 if _fz_mfma(dtype, dk, dv) else TOL_BWD


def _sum_terms(inp, ref, vstar):
    """Per head, the sums of |terms| of gA = sum_(b,t) -dt dl and of
    gI_prior = -(1 / I_prior) sum gw . w, from the oracle's gradients
    (dl = -gdt / A; gw . w = gbeta beta, or gv v for a v* input)."""
    A, Ip = to_np(inp["A"]), to_np(inp["I_prior"])
    sa = np.abs(to_np(inp["dt"]) * to_np(ref["gdt"])).sum(axis=(0, 1)) / np.abs(A)
    gww = to_np(ref["gv"]) * to_np(inp["v"]) if vstar else to_np(ref["gbeta"]) * to_np(inp["beta"])
    si = np.abs(gww).sum(axis=(0, 1, 3)) / Ip
    return {"gA": sa, "gIp": si}


def assert_sum_close(name, x, ref, terms, tol):
    """A batch sum against the oracle, relative to the sum of its terms'
    magnitudes (a sum of terms that each carry relative error e is off by at
    most e times that, whatever the cancellation between them), and also
    normwise, relative to the sum itself, against the bf16 bar."""
    x, ref = to_np(x), to_np(ref)
    den = float(np.max(terms))
    e = float(np.abs(x - ref).max() / (den if den > 0 else 1.0))
    en = rel_err(x, ref)
    print("  %-22s max componentwise err %.3e (bar %.0e); normwise %.3e (bar %.0e)" % (name, e, tol, en, TOL_BF16),
          flush=True)
    assert np.isfinite(x).all() and e <= tol, "%s: err %.3e > %.1e" % (name, e, tol)
    assert en <= TOL_BF16, "%s: normwise err %.3e > %.1e" % (name, en, TOL_BF16)


def _compare_bwd_frozen(got, ref, vstar, tol=TOL_BWD, inp=None):
    """Every gradient normwise against the oracle.  On the matrix-core path
    (inp given) the batch sums gA and gI_prior are bounded componentwise."""
    sums = _sum_terms(inp, ref, vstar) if inp is not None else {}
    for n in FZ_BWD_NAMES:
        if n == "gbeta" and vstar:
            assert got[n] is None and ref[n] is None
            continue
        if n in sums:
            assert_sum_close("frozen " + n, got[n], ref[n], sums[n], tol)
        elif n in got:
            assert_close("frozen " + n, got[n], ref[n], tol)


FZ_BWD_CASES = [
    # B, T, H, dk, dv, dtype, start state given, final-state gradient, v* input
    (1, 37, 2, 32, 32, torch.float32, True, True, False),
    (2, 64, 3, 64, 64, torch.float32, False, False, False),
    (1, 100, 2, 128, 128, torch.bfloat16, True, True, False),
    (2, 17, 2, 64, 128, torch.float32, True, False, True),
    (1, 9, 3, 128, 64, torch.bfloat16, False, True, True),
    (1, 1, 2, 32, 64, torch.float32, True, True, False),
    (2, 8, 1, 128, 32, torch.float32, False, True, False),
    (1, 200, 1, 32, 128, torch.bfloat16, False, False, False),
    (1, 33, 2, 128, 48, torch.float32, True, True, True),
    # matrix-core path: several chunks, ragged tails, one exact chunk, T = 1
    (2, 200, 3, 128, 128, torch.bfloat16, True, True, False),
    (1, 64, 2, 64, 64, torch.bfloat16, False, True, False),
    (1, 1, 2, 128, 64, torch.bfloat16, True, False, True),
    (2, 130, 2, 64, 128, torch.bfloat16, True, True, True),
    (1, 300, 1, 128, 64, torch.bfloat16, False, False, False),
    # value expansion dv = 2 dk on the matrix cores
    (1, 150, 2, 128, 256, torch.bfloat16, True, True, False),
    (2, 70, 1, 64, 256, torch.bfloat16, False, True, True),
]


@pytest.mark.parametrize("B,T,H,dk,dv,dtype,state,final,vstar", FZ_BWD_CASES)
def test_bwd_frozen_matches_oracle(B, T, H, dk, dv, dtype, state, final, vstar):
    w = workloads.WORKLOADS[0].with_(B=B, H=H, dk=dk, dv=dv, dtype=dtype, A_mode="logspace16")
    _announce("bwd frozen", B=B, T=T, H=H, dk=dk, dv=dv, dtype=dtype, state=state, final=final, vstar=vstar)
    inp = workloads.make_inputs(w, T=T, seed=T + 2 * dk + dv)
    mu0 = workloads.random_state(B, H, dv, dk, inp["I_prior"], seed=T + 5)[0] if state else None
    gr = workloads.upstream_grads(B, T, H, dv, dk, dtype, seed=T + dv, final=final)
    got = _run_bwd_frozen(inp, gr, mu0=mu0, vstar=vstar)
    _compare_bwd_frozen(got, _bwd_frozen_ref(inp, gr, mu0=mu0, vstar=vstar), vstar, _fz_tol(dtype, dk, dv),
                        inp if _fz_mfma(dtype, dk, dv) else None)


def test_bwd_frozen_bf16_inputs_fp32_upstream_gradient():
    w = workloads.WORKLOADS[0].with_(B=1, H=2, dk=128, dv=128, dtype=torch.bfloat16, A_mode="logspace16")
    T = 150
    _announce("bwd frozen bf16 in, fp32 gy", T=T)
    inp = workloads.make_inputs(w, T=T, seed=31)
    mu0 = workloads.random_state(1, 2, 128, 128, inp["I_prior"], seed=31)[0]
    gr = workloads.upstream_grads(1, T, 2, 128, 128, torch.float32, seed=31)
    got = _run_bwd_frozen(inp, gr, mu0=mu0)
    _compare_bwd_frozen(got, _bwd_frozen_ref(inp, gr, mu0=mu0), False, 2e-2, inp)


def test_bwd_frozen_unaligned_value_gradients_and_mixed_dtypes():
    """gv and gbeta only 4-byte aligned (the matrix-core path's scalar stores),
    and float32 inputs with a bf16 upstream gradient (the float32 walk)."""
    w = workloads.WORKLOADS[0].with_(B=1, H=2, dk=128, dv=128, dtype=torch.bfloat16, A_mode="logspace16")
    T = 90
    _announce("bwd frozen unaligned gv/gbeta", T=T)
    inp = workloads.make_inputs(w, T=T, seed=41)
    gr = workloads.upstream_grads(1, T, 2, 128, 128, torch.bfloat16, seed=41)
    n = T * 2 * 128
    out = {name: torch.empty(n + 1, dtype=torch.float32, device=DEV)[1:].view(1, T, 2, 128) for name in ("gv", "gbeta")}
    assert out["gv"].data_ptr() % 16 != 0
    g = to_device(inp, DEV)
    got = _pm().bwd_frozen(g["q"], g["k"], g["v"], g["beta"], g["dt"], g["A"], g["I_prior"],
                           gr["gy"].to(DEV), gmuT=gr["gmuT"].to(DEV), out=out)
    torch.cuda.synchronize()
    _compare_bwd_frozen(got, _bwd_frozen_ref(inp, gr), False, 2e-2, inp)
    # float32 inputs, bf16 gy: the float32 walk
    w32 = w.with_(dtype=torch.float32, dk=64, dv=64)
    inp32 = workloads.make_inputs(w32, T=T, seed=42)
    gr16 = workloads.upstream_grads(1, T, 2, 64, 64, torch.bfloat16, seed=42)
    _announce("bwd frozen fp32 in, bf16 gy", T=T)
    _compare_bwd_frozen(_run_bwd_frozen(inp32, gr16), _bwd_frozen_ref(inp32, gr16), False, TOL_BWD)


def test_bwd_frozen_matrix_core_agrees_with_float32_walk():
    """The same bf16-representable inputs through both paths (bf16 tensors take
    the matrix cores, their float32 copies the float32 walk): the two agree to
    the matrix-core path's bar."""
    w = workloads.WORKLOADS[0].with_(B=2, H=2, dk=64, dv=128, dtype=torch.bfloat16, A_mode="logspace16")
    T = 100
    _announce("bwd frozen: matrix cores vs float32 walk", T=T)
    inp = workloads.make_inputs(w, T=T, seed=43)
    mu0 = workloads.random_state(2, 2, 128, 64, inp["I_prior"], seed=43)[0]
    gr = workloads.upstream_grads(2, T, 2, 128, 64, torch.bfloat16, seed=43)
    inp32 = {k_: (x.float() if isinstance(x, torch.Tensor) and x.dtype == torch.bfloat16 else x) for k_, x in inp.items()}
    gr32 = {k_: (x.float() if isinstance(x, torch.Tensor) else x) for k_, x in gr.items()}
    a16 = _run_bwd_frozen(inp, gr, mu0=mu0)
    a32 = _run_bwd_frozen(inp32, gr32, mu0=mu0)
    for n_ in FZ_BWD_NAMES:
        if n_ not in ("gA", "gIp"):
            assert_close("bf16 path vs fp32 " + n_, a16[n_], a32[n_], 2e-2)


def test_bwd_frozen_matrix_core_empty_sequence():
    w = workloads.WORKLOADS[0].with_(B=2, H=3, dk=128, dv=64, dtype=torch.bfloat16)
    _announce("bwd frozen bf16 T=0", B=2, H=3, dk=128, dv=64)
    inp = workloads.make_inputs(w, T=0)
    mu0 = workloads.random_state(2, 3, 64, 128, inp["I_prior"], seed=7)[0]
    gr = workloads.upstream_grads(2, 0, 3, 64, 128, torch.bfloat16, seed=7)
    got = _run_bwd_frozen(inp, gr, mu0=mu0)
    assert torch.equal(got["gmu0"].cpu(), gr["gmuT"])
    assert float(got["gA"].abs().max()) == 0.0 and float(got["gIp"].abs().max()) == 0.0


def test_bwd_frozen_empty_sequence():
    w = workloads.WORKLOADS[0].with_(B=2, H=3, dk=64, dv=32)
    _announce("bwd frozen T=0", B=2, H=3, dk=64, dv=32)
    inp = workloads.make_inputs(w, T=0)
    mu0 = workloads.random_state(2, 3, 32, 64, inp["I_prior"], seed=6)[0]
    gr = workloads.upstream_grads(2, 0, 3, 32, 64, torch.float32, seed=6)
    got = _run_bwd_frozen(inp, gr, mu0=mu0)
    assert torch.equal(got["gmu0"].cpu(), gr["gmuT"])
    assert float(got["gA"].abs().max()) == 0.0 and float(got["gIp"].abs().max()) == 0.0


def test_bwd_frozen_mqar_workload_full():
    w = workloads.WORKLOADS[1]
    _announce("bwd frozen MQAR workload", B=w.B, H=w.H, T=w.T, dk=w.dk, dv=w.dv)
    inp = workloads.make_inputs(w)
    gr = workloads.upstream_grads(w.B, w.T, w.H, w.dv, w.dk, w.dtype, seed=8)
    _compare_bwd_frozen(_run_bwd_frozen(inp, gr), _bwd_frozen_ref(inp, gr), False)


# heads 0, 5, 11: A = 1, about 3.5 and 16 (the slowest and the fastest decay)
@pytest.mark.parametrize("h", [0, 5, 11])
def test_bwd_frozen_layer760m_sampled_head(h):
    """Full 760M-layer frozen backward; the oracle runs head h of every
    sequence, so gA[h] and gIp[h] (sums over b) compare exactly."""
    w = workloads.WORKLOADS[2]
    _announce("bwd frozen 760M layer bf16", B=w.B, H=w.H, T=w.T, d=w.dk, sampled_head=h)
    inp = workloads.make_inputs(w)
    gr = workloads.upstream_grads(w.B, w.T, w.H, w.dv, w.dk, w.dtype, seed=3)
    got = _run_bwd_frozen(inp, gr)
    sub = oracle.select_heads(inp, [(b, h) for b in range(w.B)])
    gy_s = to_np(gr["gy"])[:, :, h, :].transpose(1, 0, 2)[None]
    gm_s = to_np(gr["gmuT"])[:, h][None]
    ref = _bwd_frozen_ref(sub, {"gy": gy_s, "gmuT": gm_s})
    bs = list(range(w.B))
    tol = _fz_tol(w.dtype, w.dk, w.dv)
    for n in ("gq", "gk", "gv", "gbeta"):
        assert_close(n + " (head %d)" % h, to_np(got[n])[bs, :, h, :].transpose(1, 0, 2)[None], ref[n], tol)
    assert_close("gdt (head %d)" % h, to_np(got["gdt"])[:, :, h].T[None], ref["gdt"], tol)
    terms = _sum_terms(sub, ref, False)
    assert_sum_close("gA[h]", to_np(got["gA"])[h:h + 1], ref["gA"].sum(keepdims=True), terms["gA"].sum(), tol)
    assert_sum_close("gIp[h]", to_np(got["gIp"])[h:h + 1], ref["gIp"].sum(keepdims=True), terms["gIp"].sum(), tol)
    assert_close("gmu0 (head %d)" % h, to_np(got["gmu0"])[:, h][None], ref["gmu0"], tol)


@pytest.mark.parametrize("dtype,d", [(torch.float32, 64), (torch.bfloat16, 128)])
def test_bwd_frozen_is_deterministic_and_ignores_stale_workspace(dtype, d):
    w = workloads.WORKLOADS[0].with_(B=2, H=2, dk=d, dv=d, dtype=dtype)
    _announce("bwd frozen determinism", B=2, H=2, T=77, dk=d, dv=d, dtype=dtype)
    inp = workloads.make_inputs(w, T=77)
    gr = workloads.upstream_grads(2, 77, 2, d, d, dtype, seed=9)
    ws = torch.full((_pm().bwd_workspace_size(2, 77, 2, d, d),), 0x7F, dtype=torch.uint8, device=DEV)
    a = _run_bwd_frozen(inp, gr, workspace=ws)
    b = _run_bwd_frozen(inp, gr)
    for n in FZ_BWD_NAMES:
        assert torch.equal(a[n], b[n]), n


# ---------------------------------------------------------------------------
# training forward: the forward also stores the backward's checkpoints
# ---------------------------------------------------------------------------

TRAIN_CASES = [
    # B, T, H, dk, dv, dtype, start state given, prior per entry, v*
    (1, 37, 2, 32, 32, torch.float32, True, False, False),
    (2, 64, 3, 64, 64, torch.float32, False, False, False),
    (1, 100, 2, 128, 128, torch.bfloat16, True, False, False),
    (2, 8, 1, 128, 32, torch.float32, False, False, False),
    (1, 9, 2, 64, 48, torch.bfloat16, False, True, False),
    (1, 1, 2, 32, 64, torch.float32, True, False, True),
    (1, 24, 2, 128, 256, torch.bfloat16, True, True, True),
    (2, 17, 2, 128, 128, torch.float32, False, True, False),
    (2, 0, 2, 64, 64, torch.float32, True, False, False),
]


@pytest.mark.parametrize("B,T,H,dk,dv,dtype,state,per_entry,vstar", TRAIN_CASES)
def test_training_forward_checkpoints_feed_the_backward(B, T, H, dk, dv, dtype, state, per_entry, vstar):
    """The checkpointing forward gives the plain forward's outputs bit for bit,
    stores the same checkpoint bytes the backward's own first pass would, and
    a backward that reuses them gives the plain backward's gradients bit for
    bit (and the oracle's within the backward tolerance)."""
    w = workloads.WORKLOADS[0].with_(B=B, H=H, dk=dk, dv=dv, dtype=dtype, A_mode="logspace16")
    _announce("training fwd + bwd(saved)", B=B, T=T, H=H, dk=dk, dv=dv, dtype=dtype, state=state,
              per_entry=per_entry, vstar=vstar)
    inp = workloads.make_inputs(w, T=T, seed=11 * T + dk + dv)
    if per_entry:
        inp["I_prior"] = workloads.per_entry_prior(H, dv, dk, seed=dk + 2 * dv)
    if state:
        ip = torch.ones(H) if per_entry else inp["I_prior"]
        inp["mu0"], inp["I0"] = workloads.random_state(B, H, dv, dk, ip, seed=T + 3)
    gr = workloads.upstream_grads(B, T, H, dv, dk, dtype, seed=T + 5)
    g = to_device(inp, DEV)
    gg = to_device(gr, DEV)
    flags = (2 if per_entry else 0) | (1 if vstar else 0)
    nbytes = _pm().bwd_workspace_size(B, T, H, dk, dv, flags)
    ws = torch.full((nbytes,), 0x7F, dtype=torch.uint8, device=DEV)      # stale contents
    kw = dict(mu0=g.get("mu0"), I0=g.get("I0"), vstar=vstar)
    y0, mu0T, I0T = _pm().fwd_chunked(*gpu_args(g), **kw)
    y1, mu1T, I1T = _pm().fwd_chunked(*gpu_args(g), **kw, workspace=ws, save_checkpoints=True)
    bk = dict(mu0=g.get("mu0"), I0=g.get("I0"), gmuT=gg["gmuT"], gIT=gg["gIT"], vstar=vstar)
    ws_own = torch.empty_like(ws)
    a = _pm().bwd(*gpu_args(g), gg["gy"], **bk, workspace=ws_own)
    b = _pm().bwd(*gpu_args(g), gg["gy"], **bk, workspace=ws, checkpoints_saved=True)
    c = _pm().bwd(*gpu_args(g), gg["gy"], **bk, workspace=ws, checkpoints_saved=True)   # left in place
    torch.cuda.synchronize()
    assert torch.equal(y1, y0) and torch.equal(mu1T, mu0T) and torch.equal(I1T, I0T)
    ck_bytes = B * H * ((T + 15) // 16) * 2 * dv * dk * 4
    assert torch.equal(ws[:ck_bytes], ws_own[:ck_bytes]), "checkpoint bytes differ"
    for n in BWD_NAMES:
        assert torch.equal(b[n], a[n]), n
        assert torch.equal(c[n], a[n]), n
    ref = oracle.bwd(**inp, gy=gr["gy"], gmuT=gr["gmuT"], gIT=gr["gIT"], vstar=vstar)
    _compare_bwd(b, ref, TOL_BWD)


def test_training_forward_layer760m_matches_plain_forward_and_backward():
    """At the 760M layer's full size: the checkpointing forward and the backward
    that reuses its checkpoints equal the plain forward and backward bit for bit."""
    w = workloads.WORKLOADS[2]
    _announce("training fwd 760M layer bf16", B=w.B, H=w.H, T=w.T, d=w.dk)
    inp = workloads.make_inputs(w)
    gr = workloads.upstream_grads(w.B, w.T, w.H, w.dv, w.dk, w.dtype, seed=2)
    g = to_device(inp, DEV)
    gg = to_device(gr, DEV)
    ws = torch.empty(_pm().bwd_workspace_size(w.B, w.T, w.H, w.dk, w.dv), dtype=torch.uint8, device=DEV)
    y0, mu0T, I0T = _pm().fwd_chunked(*gpu_args(g))
    y1, mu1T, I1T = _pm().fwd_chunked(*gpu_args(g), workspace=ws, save_checkpoints=True)
    torch.cuda.synchronize()
    assert torch.equal(y1, y0) and torch.equal(mu1T, mu0T) and torch.equal(I1T, I0T)
    del y0, mu0T, I0T
    b = _pm().bwd(*gpu_args(g), gg["gy"], gmuT=gg["gmuT"], gIT=gg["gIT"], workspace=ws, checkpoints_saved=True)
    b = {n: b[n].clone() for n in ("gq", "gk", "gv", "gdt", "gA", "gIp")}
    a = _pm().bwd(*gpu_args(g), gg["gy"], gmuT=gg["gmuT"], gIT=gg["gIT"], workspace=ws)
    torch.cuda.synchronize()
    for n in b:
        assert torch.equal(b[n], a[n]), n


# ---------------------------------------------------------------------------
# generalised boundary: value expansion / any dv multiple of 16, v* input,
# a prior per state entry
# ---------------------------------------------------------------------------

DV_SHAPES = [(128, 256, torch.float32), (128, 256, torch.bfloat16), (64, 48, torch.float32),
             (32, 16, torch.float32), (128, 512, torch.bfloat16), (64, 176, torch.float32),
             # the widest value dimension the path takes
             (128, 1024, torch.bfloat16), (32, 1024, torch.float32)]


@pytest.mark.parametrize("dk,dv,dtype", DV_SHAPES)
def test_value_expansion_forward_step_backward(dk, dv, dtype):
    w = workloads.WORKLOADS[0].with_(B=2, H=2, dk=dk, dv=dv, dtype=dtype, A_mode="logspace16")
    T = 45
    _announce("dv shapes fwd+step+bwd", B=w.B, H=w.H, T=T, dk=dk, dv=dv, dtype=dtype)
    inp = workloads.make_inputs(w, T=T, seed=dk + dv)
    inp["mu0"], inp["I0"] = workloads.random_state(w.B, w.H, dv, dk, inp["I_prior"], seed=dv)
    y, muT, IT = _run_fwd(inp)
    _compare_full(inp, y, muT, IT, tol_for(dtype))
    # one decode step from the final state
    d = {n: x.to(DEV) for n, x in workloads.decode_inputs(w, 0).items()}
    ref_y, ref_mu, ref_I = oracle.step(**{n: workloads_cpu(d[n]) for n in d}, A=inp["A"], I_prior=inp["I_prior"],
                                       mu=to_np(muT), I=to_np(IT))
    mu, I = muT.clone(), IT.clone()
    ys = _pm().step(d["q"], d["k"], d["v"], d["beta"], d["dt"], inp["A"].to(DEV), inp["I_prior"].to(DEV), mu, I)
    torch.cuda.synchronize()
    assert_close("step y", ys, ref_y, tol_for(dtype))
    assert_close("step mu", mu, ref_mu, TOL_F32)
    gr = workloads.upstream_grads(w.B, T, w.H, dv, dk, dtype, seed=dv)
    _compare_bwd(_run_bwd(inp, gr), _bwd_ref(inp, gr), TOL_BWD)


def workloads_cpu(x):
    return x.cpu() if isinstance(x, torch.Tensor) else x


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_vstar_input_forward_step_backward(dtype):
    """With PALIMPSA_VSTAR the v tensor is the write v* itself."""
    w = workloads.WORKLOADS[0].with_(B=2, H=3, dk=64, dv=64, dtype=dtype, A_mode="logspace16")
    T = 70
    _announce("v* fwd+step+bwd", B=w.B, H=w.H, T=T, d=64, dtype=dtype)
    inp = workloads.make_inputs(w, T=T, seed=77)
    g = to_device(inp, DEV)
    y, muT, IT = _pm().fwd_chunked(*gpu_args(g), vstar=True)
    torch.cuda.synchronize()
    y_ref, mu_ref, I_ref = oracle.fwd(**inp, vstar=True)
    assert_close("y (v*)", y, y_ref, tol_for(dtype))
    assert_close("muT (v*)", muT, mu_ref, TOL_F32)
    assert_close("IT (v*)", IT, I_ref, TOL_F32)
    d = {n: x.to(DEV) for n, x in workloads.decode_inputs(w, 1).items()}
    ref = oracle.step(**{n: d[n].cpu() for n in d}, A=inp["A"], I_prior=inp["I_prior"], mu=to_np(muT),
                      I=to_np(IT), vstar=True)
    ys = _pm().step(d["q"], d["k"], d["v"], d["beta"], d["dt"], g["A"], g["I_prior"], muT, IT, vstar=True)
    torch.cuda.synchronize()
    assert_close("step y (v*)", ys, ref[0], tol_for(dtype))
    assert_close("step mu (v*)", muT, ref[1], TOL_F32)
    gr = workloads.upstream_grads(w.B, T, w.H, 64, 64, dtype, seed=78)
    gg = to_device(gr, DEV)
    got = _pm().bwd(*gpu_args(g), gg["gy"], gmuT=gg["gmuT"], gIT=gg["gIT"], vstar=True)
    torch.cuda.synchronize()
    ref = oracle.bwd(**inp, gy=gr["gy"], gmuT=gr["gmuT"], gIT=gr["gIT"], vstar=True)
    _compare_bwd(got, ref, TOL_BWD)


@pytest.mark.parametrize("dk,dv,state", [(128, 128, False), (64, 32, True), (32, 64, False), (128, 256, True)])
def test_per_entry_prior_forward_step_backward(dk, dv, state):
    w = workloads.WORKLOADS[0].with_(B=2, H=2, dk=dk, dv=dv, A_mode="logspace16")
    T = 200    # long enough for the 3-segment split below (segments are multiples of 64 tokens)
    _announce("per-entry prior fwd+split+step+bwd", B=w.B, H=w.H, T=T, dk=dk, dv=dv, state=state)
    inp = workloads.make_inputs(w, T=T, seed=dk * 3 + dv)
    inp["I_prior"] = workloads.per_entry_prior(w.H, dv, dk, seed=dk + dv)
    if state:
        inp["mu0"], inp["I0"] = workloads.random_state(w.B, w.H, dv, dk, torch.ones(w.H), seed=5)
    y, muT, IT = _run_fwd(inp)
    _compare_full(inp, y, muT, IT, TOL_F32)
    g = to_device(inp, DEV)
    ys, mus, Is = _pm().fwd_chunked(*gpu_args(g), mu0=g.get("mu0"), I0=g.get("I0"), segments=3)
    torch.cuda.synchronize()
    assert rel_err(ys, y) <= 1e-5 and rel_err(mus, muT) <= 1e-5 and rel_err(Is, IT) <= 1e-6
    d = {n: x.to(DEV) for n, x in workloads.decode_inputs(w, 2).items()}
    ref = oracle.step(**{n: d[n].cpu() for n in d}, A=inp["A"], I_prior=inp["I_prior"], mu=to_np(muT), I=to_np(IT))
    ys1 = _pm().step(d["q"], d["k"], d["v"], d["beta"], d["dt"], g["A"], g["I_prior"], muT, IT)
    torch.cuda.synchronize()
    assert_close("step y (per-entry prior)", ys1, ref[0], TOL_F32)
    assert_close("step I (per-entry prior)", IT, ref[2], TOL_F32)
    gr = workloads.upstream_grads(w.B, T, w.H, dv, dk, w.dtype, seed=dk)
    got = _run_bwd(inp, gr)
    assert tuple(got["gIp"].shape) == (w.H, dv, dk)
    _compare_bwd(got, _bwd_ref(inp, gr), TOL_BWD)


@pytest.mark.parametrize("dv", [256, 192, 1024])
def test_frozen_value_expansion(dv):
    w = workloads.WORKLOADS[0].with_(B=1, H=3, dk=128, dv=dv, dtype=torch.bfloat16, A_mode="logspace16")
    _announce("frozen dv", B=1, H=3, T=130, dk=128, dv=dv)
    inp = workloads.make_inputs(w, T=130, seed=dv)
    g = to_device(inp, DEV)
    y, muT = _pm().fwd_frozen(*gpu_args(g))
    torch.cuda.synchronize()
    y_ref, mu_ref = _frozen_ref(inp)
    assert_close("frozen y (dv=%d)" % dv, y, y_ref, 2e-2)
    assert_close("frozen muT (dv=%d)" % dv, muT, mu_ref, 2e-2)


# ---------------------------------------------------------------------------
# block-diagonal precision (2x2 blocks along the key axis)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dk,dv,dtype,state,T", [(32, 32, torch.float32, False, 37), (64, 48, torch.float32, True, 100),
                                                 (128, 128, torch.bfloat16, True, 70), (128, 64, torch.float32, False, 1),
                                                 (64, 128, torch.bfloat16, False, 160),
                                                 (128, 1024, torch.bfloat16, True, 45), (32, 1024, torch.float32, False, 45)])
def test_blockdiag_matches_oracle(dk, dv, dtype, state, T):
    w = workloads.WORKLOADS[0].with_(B=2, H=2, dk=dk, dv=dv, dtype=dtype, A_mode="logspace16")
    _announce("blockdiag fwd", B=w.B, H=w.H, T=T, dk=dk, dv=dv, dtype=dtype, state=state)
    inp = workloads.make_inputs(w, T=T, seed=dk + dv + T)
    mu0 = P0 = None
    if state:
        mu0, P0 = workloads.random_block_state(w.B, w.H, dv, dk, 2, inp["I_prior"], seed=T)
    g = to_device(inp, DEV)
    y, muT, PT = _pm().fwd_blockdiag(*gpu_args(g), block=2, mu0=None if mu0 is None else mu0.to(DEV),
                                     P0=None if P0 is None else P0.to(DEV))
    torch.cuda.synchronize()
    y_ref, mu_ref, P_ref = oracle.fwd_blockdiag(**{n: inp[n] for n in ("q", "k", "v", "beta", "dt", "A", "I_prior")},
                                                block=2, mu0=mu0, P0=P0)
    assert_close("blockdiag y", y, y_ref, tol_for(dtype))
    assert_close("blockdiag muT", muT, mu_ref, TOL_F32)
    assert_close("blockdiag PT", PT, P_ref, TOL_F32)


def test_blockdiag_empty_sequence_copies_state():
    w = workloads.WORKLOADS[0].with_(B=1, H=2, dk=32, dv=32)
    _announce("blockdiag T=0", B=1, H=2, dk=32, dv=32)
    inp = workloads.make_inputs(w, T=0)
    mu0, P0 = workloads.random_block_state(1, 2, 32, 32, 2, inp["I_prior"], seed=3)
    g = to_device(inp, DEV)
    _, muT, PT = _pm().fwd_blockdiag(*gpu_args(g), block=2, mu0=mu0.to(DEV), P0=P0.to(DEV))
    torch.cuda.synchronize()
    assert torch.equal(muT.cpu(), mu0)
    assert torch.equal(PT.cpu()[..., 0, 0], P0[..., 0, 0]) and torch.equal(PT.cpu()[..., 0, 1], P0[..., 0, 1])


def test_blockdiag_layer760m_sampled():
    w = workloads.WORKLOADS[2]
    heads = [(0, 0), (7, 11)]
    _announce("blockdiag 760M layer", B=w.B, H=w.H, T=w.T, d=w.dk, sampled=heads)
    inp = workloads.make_inputs(w)
    g = to_device(inp, DEV)
    y, muT, PT = _pm().fwd_blockdiag(*gpu_args(g), block=2)
    torch.cuda.synchronize()
    sub = oracle.select_heads(inp, heads)
    y_ref, mu_ref, P_ref = oracle.fwd_blockdiag(**{n: sub[n] for n in ("q", "k", "v", "beta", "dt", "A", "I_prior")},
                                                block=2)
    bs = [b for b, _ in heads]
    hs = [h for _, h in heads]
    assert_close("blockdiag y (sampled)", to_np(y)[bs, :, hs, :].transpose(1, 0, 2)[None], y_ref, tol_for(w.dtype))
    assert_close("blockdiag muT (sampled)", to_np(muT)[bs, hs][None], mu_ref, TOL_F32)
    assert_close("blockdiag PT (sampled)", to_np(PT)[bs, hs][None], P_ref, TOL_F32)


@pytest.mark.parametrize("dk,dv,dtype", [(32, 32, torch.float32), (64, 48, torch.bfloat16), (128, 128, torch.float32),
                                         (128, 1024, torch.bfloat16)])
def test_blockdiag_step_matches_oracle(dk, dv, dtype):
    """One decode token from a random SPD block state against the oracle's
    block-diagonal forward over that one token."""
    w = workloads.WORKLOADS[0].with_(B=2, H=3, dk=dk, dv=dv, dtype=dtype, A_mode="logspace16")
    _announce("blockdiag step", B=w.B, H=w.H, dk=dk, dv=dv, dtype=dtype)
    inp = workloads.make_inputs(w, T=1, seed=dk + dv)
    mu0, P0 = workloads.random_block_state(w.B, w.H, dv, dk, 2, inp["I_prior"], seed=dv)
    d = {n: inp[n][:, 0].contiguous().to(DEV) for n in ("q", "k", "v", "beta", "dt")}
    mu, P = mu0.to(DEV), P0.to(DEV)
    y = _pm().step_blockdiag(d["q"], d["k"], d["v"], d["beta"], d["dt"], inp["A"].to(DEV), inp["I_prior"].to(DEV),
                             mu, P)
    torch.cuda.synchronize()
    y_ref, mu_ref, P_ref = oracle.fwd_blockdiag(**{n: inp[n] for n in ("q", "k", "v", "beta", "dt", "A", "I_prior")},
                                                block=2, mu0=mu0, P0=P0)
    assert_close("bd step y", y, y_ref[:, 0], tol_for(dtype))
    assert_close("bd step mu", mu, mu_ref, TOL_F32)
    assert_close("bd step P", P, P_ref, TOL_F32)


def test_blockdiag_steps_follow_the_forward():
    """T decode steps from the default state reproduce the block-diagonal
    forward's readouts and final state (up to float32 rounding: the step
    re-forms P mu each token, the forward carries it)."""
    w = workloads.WORKLOADS[0].with_(B=2, H=2, dk=64, dv=64, dtype=torch.float32, A_mode="logspace16")
    T = 40
    _announce("blockdiag steps vs forward", T=T)
    inp = workloads.make_inputs(w, T=T, seed=77)
    g = to_device(inp, DEV)
    y_f, mu_f, P_f = _pm().fwd_blockdiag(*gpu_args(g), block=2)
    mu = torch.zeros(w.B, w.H, w.dv, w.dk, device=DEV)
    P = (g["I_prior"].view(1, w.H, 1, 1, 1, 1) * torch.eye(2, device=DEV)).expand(w.B, w.H, w.dv, w.dk // 2, 2, 2)
    P = P.contiguous()
    ys = []
    for t in range(T):
        ys.append(_pm().step_blockdiag(g["q"][:, t].contiguous(), g["k"][:, t].contiguous(), g["v"][:, t].contiguous(),
                                       g["beta"][:, t].contiguous(), g["dt"][:, t].contiguous(), g["A"], g["I_prior"],
                                       mu, P))
    torch.cuda.synchronize()
    assert_close("bd steps y", torch.stack(ys, 1), y_f, 1e-5)
    assert_close("bd steps mu", mu, mu_f, 1e-5)
    assert_close("bd steps P", P[..., 0, 1], P_f[..., 0, 1], 1e-5)


@pytest.mark.parametrize("dk,dv,dtype,state,T", [(64, 48, torch.float32, True, 37), (128, 128, torch.bfloat16, True, 70),
                                                 (128, 64, torch.float32, False, 1), (64, 128, torch.bfloat16, False, 100),
                                                 (128, 32, torch.float32, True, 0),
                                                 (64, 1024, torch.bfloat16, True, 45)])
def test_blockdiag4_matches_oracle(dk, dv, dtype, state, T):
    """4x4 precision blocks (Cholesky per block) against the oracle's block-diagonal forward."""
    w = workloads.WORKLOADS[0].with_(B=2, H=2, dk=dk, dv=dv, dtype=dtype, A_mode="logspace16")
    _announce("blockdiag4 fwd", B=w.B, H=w.H, T=T, dk=dk, dv=dv, dtype=dtype, state=state)
    inp = workloads.make_inputs(w, T=T, seed=dk + dv + T + 4)
    mu0 = P0 = None
    if state:
        mu0, P0 = workloads.random_block_state(w.B, w.H, dv, dk, 4, inp["I_prior"], seed=T + 4)
    g = to_device(inp, DEV)
    y, muT, PT = _pm().fwd_blockdiag(*gpu_args(g), block=4, mu0=None if mu0 is None else mu0.to(DEV),
                                     P0=None if P0 is None else P0.to(DEV))
    torch.cuda.synchronize()
    y_ref, mu_ref, P_ref = oracle.fwd_blockdiag(**{n: inp[n] for n in ("q", "k", "v", "beta", "dt", "A", "I_prior")},
                                                block=4, mu0=mu0, P0=P0)
    if T > 0:
        assert_close("blockdiag4 y", y, y_ref, tol_for(dtype))
    assert_close("blockdiag4 muT", muT, mu_ref, TOL_F32)
    assert_close("blockdiag4 PT", PT, P_ref, TOL_F32)


def test_blockdiag4_layer760m_sampled():
    w = workloads.WORKLOADS[2]
    heads = [(3, 2), (6, 9)]
    _announce("blockdiag4 760M layer", B=w.B, H=w.H, T=w.T, d=w.dk, sampled=heads)
    inp = workloads.make_inputs(w)
    g = to_device(inp, DEV)
    y, muT, PT = _pm().fwd_blockdiag(*gpu_args(g), block=4)
    torch.cuda.synchronize()
    sub = oracle.select_heads(inp, heads)
    y_ref, mu_ref, P_ref = oracle.fwd_blockdiag(**{n: sub[n] for n in ("q", "k", "v", "beta", "dt", "A", "I_prior")},
                                                block=4)
    bs = [b for b, _ in heads]
    hs = [h for _, h in heads]
    assert_close("blockdiag4 y (sampled)", to_np(y)[bs, :, hs, :].transpose(1, 0, 2)[None], y_ref, tol_for(w.dtype))
    assert_close("blockdiag4 muT (sampled)", to_np(muT)[bs, hs][None], mu_ref, TOL_F32)
    assert_close("blockdiag4 PT (sampled)", to_np(PT)[bs, hs][None], P_ref, TOL_F32)


@pytest.mark.parametrize("dk,dv,dtype", [(64, 64, torch.float32), (128, 96, torch.bfloat16)])
def test_blockdiag4_step_matches_oracle_and_forward(dk, dv, dtype):
    """One 4x4-block decode token against the oracle, then steps against the forward."""
    w = workloads.WORKLOADS[0].with_(B=2, H=2, dk=dk, dv=dv, dtype=dtype, A_mode="logspace16")
    _announce("blockdiag4 step", B=w.B, H=w.H, dk=dk, dv=dv, dtype=dtype)
    inp = workloads.make_inputs(w, T=1, seed=dk + dv + 5)
    mu0, P0 = workloads.random_block_state(w.B, w.H, dv, dk, 4, inp["I_prior"], seed=dv + 5)
    d = {n: inp[n][:, 0].contiguous().to(DEV) for n in ("q", "k", "v", "beta", "dt")}
    mu, P = mu0.to(DEV), P0.to(DEV)
    y = _pm().step_blockdiag(d["q"], d["k"], d["v"], d["beta"], d["dt"], inp["A"].to(DEV), inp["I_prior"].to(DEV),
                             mu, P, block=4)
    torch.cuda.synchronize()
    y_ref, mu_ref, P_ref = oracle.fwd_blockdiag(**{n: inp[n] for n in ("q", "k", "v", "beta", "dt", "A", "I_prior")},
                                                block=4, mu0=mu0, P0=P0)
    assert_close("bd4 step y", y, y_ref[:, 0], tol_for(dtype))
    assert_close("bd4 step mu", mu, mu_ref, TOL_F32)
    assert_close("bd4 step P", P, P_ref, TOL_F32)
    # 30 steps from the default state against the forward over the same tokens
    T = 30
    inp = workloads.make_inputs(w.with_(dtype=torch.float32), T=T, seed=88)
    g = to_device(inp, DEV)
    y_f, mu_f, P_f = _pm().fwd_blockdiag(*gpu_args(g), block=4)
    mu = torch.zeros(w.B, w.H, dv, dk, device=DEV)
    P = (g["I_prior"].view(1, w.H, 1, 1, 1, 1) * torch.eye(4, device=DEV)).expand(w.B, w.H, dv, dk // 4, 4, 4)
    P = P.contiguous()
    ys = [_pm().step_blockdiag(g["q"][:, t].contiguous(), g["k"][:, t].contiguous(), g["v"][:, t].contiguous(),
                               g["beta"][:, t].contiguous(), g["dt"][:, t].contiguous(), g["A"], g["I_prior"], mu, P,
                               block=4) for t in range(T)]
    torch.cuda.synchronize()
    assert_close("bd4 steps y", torch.stack(ys, 1), y_f, 1e-5)
    assert_close("bd4 steps mu", mu, mu_f, 1e-5)
    assert_close("bd4 steps P", P, P_f, 1e-5)


# ---------------------------------------------------------------------------
# block-diagonal precision: backward (2x2 blocks)
# ---------------------------------------------------------------------------

BD_BWD_NAMES = ("gq", "gk", "gv", "gbeta", "gdt", "gA", "gIp", "gmu0", "gP0")
BD_FWD_KEYS = ("q", "k", "v", "beta", "dt", "A", "I_prior")


def _sym_blocks(G):
    """The gradient for a symmetric P0: (G + G^T) / 2 per block."""
    G = np.asarray(G, dtype=np.float64)
    return 0.5 * (G + np.swapaxes(G, -1, -2))


def _bd_bwd_run(inp, gy, mu0=None, P0=None, gmuT=None, gPT=None, block=2):
    g = to_device(inp, DEV)
    dev = lambda t: None if t is None else t.to(DEV)
    out = _pm().bwd_blockdiag(*gpu_args(g), dev(gy), block=block, mu0=dev(mu0), P0=dev(P0), gmuT=dev(gmuT),
                              gPT=dev(gPT))
    torch.cuda.synchronize()
    return out


def _bd_bwd_ref(inp, gy, mu0=None, P0=None, gmuT=None, gPT=None, block=2):
    ref = oracle.bwd_blockdiag(**{n: inp[n] for n in BD_FWD_KEYS}, block=block, gy=gy, mu0=mu0, P0=P0,
                               gmuT=gmuT, gPT=gPT)
    ref["gP0"] = _sym_blocks(ref["gP0"])
    return ref


BD_BWD_CASES = [
    # block, B, T, H, dk, dv, dtype, gy dtype, start state given, final-state gradients
    (2, 1, 37, 2, 32, 32, torch.float32, torch.float32, True, True),
    (2, 2, 64, 3, 64, 64, torch.float32, torch.float32, False, False),
    (2, 1, 100, 2, 128, 128, torch.bfloat16, torch.bfloat16, True, True),
    (2, 2, 17, 2, 64, 48, torch.float32, torch.bfloat16, True, False),
    (2, 1, 9, 3, 128, 64, torch.bfloat16, torch.float32, False, True),
    (2, 1, 1, 2, 32, 64, torch.float32, torch.float32, True, True),
    (2, 2, 8, 1, 128, 32, torch.float32, torch.float32, False, True),
    (2, 1, 150, 1, 32, 128, torch.bfloat16, torch.bfloat16, False, False),
    (4, 1, 37, 2, 64, 32, torch.float32, torch.float32, True, True),
    (4, 2, 64, 2, 128, 64, torch.float32, torch.float32, False, False),
    (4, 1, 100, 2, 128, 128, torch.bfloat16, torch.bfloat16, True, True),
    (4, 2, 17, 1, 64, 48, torch.float32, torch.bfloat16, True, False),
    (4, 1, 1, 2, 128, 16, torch.float32, torch.float32, True, True),
    (4, 1, 9, 3, 64, 128, torch.bfloat16, torch.float32, False, True),
]


@pytest.mark.parametrize("block,B,T,H,dk,dv,dtype,gdtype,state,final", BD_BWD_CASES)
def test_blockdiag_bwd_matches_oracle(block, B, T, H, dk, dv, dtype, gdtype, state, final):
    w = workloads.WORKLOADS[0].with_(B=B, H=H, dk=dk, dv=dv, dtype=dtype, A_mode="logspace16")
    _announce("blockdiag bwd", block=block, B=B, T=T, H=H, dk=dk, dv=dv, dtype=dtype, gy=gdtype, state=state,
              final=final)
    inp = workloads.make_inputs(w, T=T, seed=T + dk + 5 * dv)
    mu0 = P0 = None
    if state:
        mu0, P0 = workloads.random_block_state(B, H, dv, dk, block, inp["I_prior"], seed=T + 2)
    gr = workloads.upstream_grads(B, T, H, dv, dk, gdtype, seed=T + dk + 1, final=final)
    gPT = workloads.block_state_grads(B, H, dv, dk, block, seed=T) if final else None
    got = _bd_bwd_run(inp, gr["gy"], mu0, P0, gr["gmuT"], gPT, block=block)
    ref = _bd_bwd_ref(inp, gr["gy"], mu0, P0, gr["gmuT"], gPT, block=block)
    for n in BD_BWD_NAMES:
        assert_close("bd%d %s" % (block, n), got[n], ref[n], TOL_BWD)


@pytest.mark.parametrize("block,dk,dtype", [(2, 128, torch.bfloat16), (2, 32, torch.float32), (4, 64, torch.bfloat16)])
def test_blockdiag_bwd_widest_value_dimension(block, dk, dtype):
    """dv = 1024, the widest the path takes (64 row blocks per head), from a
    random state with final-state gradients."""
    B, T, H, dv = 1, 45, 1, 1024
    w = workloads.WORKLOADS[0].with_(B=B, H=H, dk=dk, dv=dv, dtype=dtype, A_mode="logspace16")
    _announce("blockdiag bwd dv=1024", block=block, B=B, T=T, H=H, dk=dk, dv=dv, dtype=dtype)
    inp = workloads.make_inputs(w, T=T, seed=dk + block)
    mu0, P0 = workloads.random_block_state(B, H, dv, dk, block, inp["I_prior"], seed=dk)
    gr = workloads.upstream_grads(B, T, H, dv, dk, dtype, seed=dk + 3)
    gPT = workloads.block_state_grads(B, H, dv, dk, block, seed=dk)
    got = _bd_bwd_run(inp, gr["gy"], mu0, P0, gr["gmuT"], gPT, block=block)
    ref = _bd_bwd_ref(inp, gr["gy"], mu0, P0, gr["gmuT"], gPT, block=block)
    for n in BD_BWD_NAMES:
        assert_close("bd%d %s (dv=1024)" % (block, n), got[n], ref[n], TOL_BWD)


@pytest.mark.parametrize("block", [2, 4])
def test_blockdiag_bwd_no_forgetting(block):
    """dt = 0 everywhere: alpha = 1 and c = 0 at every token, so P only
    accumulates evidence and gI_prior keeps only the default start's share;
    gdt and gA are the derivatives at dt = 0."""
    B, T, H, dk, dv = 2, 50, 2, 64, 32
    w = workloads.WORKLOADS[0].with_(B=B, H=H, dk=dk, dv=dv)
    _announce("blockdiag bwd alpha=1", block=block, B=B, T=T, H=H, dk=dk, dv=dv)
    inp = workloads.make_inputs(w, T=T, seed=21)
    inp["dt"] = torch.zeros_like(inp["dt"])
    gr = workloads.upstream_grads(B, T, H, dv, dk, torch.float32, seed=21)
    got = _bd_bwd_run(inp, gr["gy"], gmuT=gr["gmuT"], block=block)
    ref = _bd_bwd_ref(inp, gr["gy"], gmuT=gr["gmuT"], block=block)
    for n in BD_BWD_NAMES:
        assert_close("bd%d %s (alpha=1)" % (block, n), got[n], ref[n], TOL_BWD)


@pytest.mark.parametrize("block,T,dk,dtype", [(2, 37, 128, torch.bfloat16), (2, 64, 32, torch.float32),
                                              (4, 41, 64, torch.float32), (4, 16, 128, torch.bfloat16),
                                              (2, 0, 64, torch.float32)])
def test_blockdiag_training_forward_saves_the_checkpoints(block, T, dk, dtype):
    """The forward with save_checkpoints writes the backward's checkpoints as
    the backward's own pass would: its outputs equal the plain forward's and
    the backward that reuses them equals the one that recomputes them, bitwise
    (T = 37 and 41 end mid-chunk, so the discard block takes a store)."""
    B, H, dv = 2, 2, 48
    w = workloads.WORKLOADS[0].with_(B=B, H=H, dk=dk, dv=dv, dtype=dtype, A_mode="logspace16")
    _announce("blockdiag training forward", block=block, B=B, T=T, H=H, dk=dk, dv=dv, dtype=dtype)
    inp = workloads.make_inputs(w, T=T, seed=T + block)
    mu0, P0 = workloads.random_block_state(B, H, dv, dk, block, inp["I_prior"], seed=T)
    gr = workloads.upstream_grads(B, T, H, dv, dk, dtype, seed=T + 1)
    g = to_device(inp, DEV)
    mu0, P0, gy, gmuT = mu0.to(DEV), P0.to(DEV), gr["gy"].to(DEV), gr["gmuT"].to(DEV)
    pm = _pm()
    ws = torch.empty(pm.bwd_blockdiag_workspace_size(B, T, H, dk, dv, block), dtype=torch.uint8, device=DEV)
    ref_fwd = pm.fwd_blockdiag(*gpu_args(g), block=block, mu0=mu0, P0=P0)
    ref_bwd = pm.bwd_blockdiag(*gpu_args(g), gy, block=block, mu0=mu0, P0=P0, gmuT=gmuT)
    ws.fill_(0xFF)          # any stale contents must be overwritten
    got_fwd = pm.fwd_blockdiag(*gpu_args(g), block=block, mu0=mu0, P0=P0, save_checkpoints=True, workspace=ws)
    got_bwd = pm.bwd_blockdiag(*gpu_args(g), gy, block=block, mu0=mu0, P0=P0, gmuT=gmuT, workspace=ws,
                               checkpoints_saved=True)
    torch.cuda.synchronize()
    for name, x, y in zip(("y", "muT", "PT"), got_fwd, ref_fwd):
        assert torch.equal(x, y), name
    for n in BD_BWD_NAMES:
        assert torch.equal(got_bwd[n], ref_bwd[n]), n


@pytest.mark.parametrize("block", [2, 4])
def test_blockdiag_bwd_empty_sequence(block):
    B, H, dk, dv = 2, 3, 64, 32
    w = workloads.WORKLOADS[0].with_(B=B, H=H, dk=dk, dv=dv)
    _announce("blockdiag bwd T=0", block=block, B=B, H=H, dk=dk, dv=dv)
    inp = workloads.make_inputs(w, T=0)
    mu0, P0 = workloads.random_block_state(B, H, dv, dk, block, inp["I_prior"], seed=6)
    gr = workloads.upstream_grads(B, 0, H, dv, dk, torch.float32, seed=6)
    gPT = workloads.block_state_grads(B, H, dv, dk, block, seed=6)
    got = _bd_bwd_run(inp, gr["gy"], mu0, P0, gr["gmuT"], gPT, block=block)
    assert torch.equal(got["gmu0"].cpu(), gr["gmuT"])
    assert torch.equal(got["gP0"].cpu(), 0.5 * (gPT + gPT.transpose(-1, -2)))
    assert float(got["gA"].abs().max()) == 0.0 and float(got["gIp"].abs().max()) == 0.0
    # the default start state: gI_prior collects tr(gP0) = tr(gPT)
    got = _bd_bwd_run(inp, gr["gy"], gmuT=gr["gmuT"], gPT=gPT, block=block)
    ref = _bd_bwd_ref(inp, gr["gy"], gmuT=gr["gmuT"], gPT=gPT, block=block)
    assert_close("bd%d gIp (T=0, default start)" % block, got["gIp"], ref["gIp"], TOL_F32)


@pytest.mark.parametrize("block", [2, 4])
def test_blockdiag_bwd_is_deterministic(block):
    B, T, H, dk, dv = 2, 77, 2, 128, 64
    w = workloads.WORKLOADS[0].with_(B=B, H=H, dk=dk, dv=dv, dtype=torch.bfloat16, A_mode="logspace16")
    _announce("blockdiag bwd determinism", block=block, B=B, T=T, H=H, dk=dk, dv=dv)
    inp = workloads.make_inputs(w, T=T, seed=9)
    gr = workloads.upstream_grads(B, T, H, dv, dk, torch.bfloat16, seed=9)
    a = _bd_bwd_run(inp, gr["gy"], gmuT=gr["gmuT"], block=block)
    b = _bd_bwd_run(inp, gr["gy"], gmuT=gr["gmuT"], block=block)
    for n in BD_BWD_NAMES:
        assert torch.equal(a[n], b[n]), n


@pytest.mark.parametrize("block", [2, 4])
def test_blockdiag_bwd_layer760m_sampled_head(block):
    """The full 760M-layer block-diagonal backward on the GPU; the oracle runs
    one (sequence, head) pair, whose per-token and per-sequence gradients
    compare directly."""
    w = workloads.WORKLOADS[2]
    b, h = (3, 7) if block == 2 else (6, 2)
    _announce("blockdiag bwd 760M layer bf16", block=block, B=w.B, H=w.H, T=w.T, d=w.dk, sampled=(b, h))
    inp = workloads.make_inputs(w)
    gr = workloads.upstream_grads(w.B, w.T, w.H, w.dv, w.dk, w.dtype, seed=12)
    gPT = workloads.block_state_grads(w.B, w.H, w.dv, w.dk, block, seed=12)
    got = _bd_bwd_run(inp, gr["gy"], gmuT=gr["gmuT"], gPT=gPT, block=block)
    sub = oracle.select_heads(inp, [(b, h)])
    ref = _bd_bwd_ref(sub, to_np(gr["gy"])[b:b + 1, :, h:h + 1], gmuT=to_np(gr["gmuT"])[b:b + 1, h:h + 1],
                      gPT=to_np(gPT)[b:b + 1, h:h + 1], block=block)
    for n in ("gq", "gk", "gv", "gbeta"):
        assert_close("bd %s (sampled)" % n, to_np(got[n])[b:b + 1, :, h:h + 1], ref[n], TOL_BWD)
    assert_close("bd gdt (sampled)", to_np(got["gdt"])[b:b + 1, :, h:h + 1], ref["gdt"], TOL_BWD)
    assert_close("bd gmu0 (sampled)", to_np(got["gmu0"])[b:b + 1, h:h + 1], ref["gmu0"], TOL_BWD)
    assert_close("bd gP0 (sampled)", to_np(got["gP0"])[b:b + 1, h:h + 1], ref["gP0"], TOL_BWD)


# ---------------------------------------------------------------------------
# heads as wide as the model (the pages' recurrent-kernel measurement, Fig. 7):
# dk in {256, 512, 1024, 2048}
# ---------------------------------------------------------------------------

WIDE_CASES = [
    # B, H, T, dk, dv, dtype, start state
    (2, 1, 45, 256, 256, torch.float32, True),
    (1, 2, 37, 512, 512, torch.float32, False),
    (2, 1, 21, 512, 48, torch.bfloat16, True),
    (1, 1, 30, 1024, 64, torch.float32, True),
    (1, 1, 19, 2048, 32, torch.float32, False),
    (1, 1, 9, 2048, 2048, torch.bfloat16, True),
    (2, 3, 11, 512, 16, torch.float32, True),      # two 8-row workgroups per head
    (1, 2, 66, 1024, 80, torch.bfloat16, False),   # ten 8-row workgroups, 33 chunks
    (1, 1, 0, 512, 16, torch.float32, True),       # empty sequence: the state is copied through
    (2, 1, 0, 2048, 32, torch.float32, False),     # empty sequence from the default state
    # the widest value dimensions the wide path takes
    (1, 1, 12, 256, 1024, torch.float32, True),
    (1, 1, 6, 512, 4096, torch.bfloat16, False),
    (1, 1, 4, 2048, 4096, torch.float32, True),
]


@pytest.mark.parametrize("B,H,T,dk,dv,dtype,state", WIDE_CASES)
def test_wide_heads_forward_and_step(B, H, T, dk, dv, dtype, state):
    w = workloads.WORKLOADS[0].with_(B=B, H=H, dk=dk, dv=dv, dtype=dtype, A_mode="logspace16")
    _announce("wide head fwd+step", B=B, H=H, T=T, dk=dk, dv=dv, dtype=dtype, state=state)
    inp = workloads.make_inputs(w, T=T, seed=dk + dv + T)
    if state:
        inp["mu0"], inp["I0"] = workloads.random_state(B, H, dv, dk, inp["I_prior"], seed=dk)
    y, muT, IT = _run_fwd(inp)
    _compare_full(inp, y, muT, IT, tol_for(dtype))
    d = {n: x.to(DEV) for n, x in workloads.decode_inputs(w, 3).items()}
    ref = oracle.step(**{n: d[n].cpu() for n in d}, A=inp["A"], I_prior=inp["I_prior"], mu=to_np(muT), I=to_np(IT))
    ys = _pm().step(d["q"], d["k"], d["v"], d["beta"], d["dt"], inp["A"].to(DEV), inp["I_prior"].to(DEV), muT, IT)
    torch.cuda.synchronize()
    assert_close("wide step y", ys, ref[0], tol_for(dtype))
    assert_close("wide step mu", muT, ref[1], TOL_F32)
    assert_close("wide step I", IT, ref[2], TOL_F32)


# Heads of 512 keys and wider run row-parallel (lanes on value rows, the
# column operands k, k^2, q as scalar operands, partial readouts of column
# slices added in a last pass) when the call has the workspace that
# workspace_size() reports; that is nonzero when d_v is a multiple of 64 and
# the grid of 64-row blocks x column slices covers every CU.
ROWS_CASES = [
    # B, H, T, dk, dv, dtype, start state
    (4, 1, 21, 512, 2048, torch.bfloat16, True),    # 16 columns per lane, 2 slices, ragged last 8-token block
    (2, 2, 9, 1024, 2048, torch.float32, False),    # 32 columns per lane, 2 slices
    (1, 2, 11, 2048, 2048, torch.bfloat16, True),   # 4 slices
    (1, 1, 3, 2048, 4096, torch.float32, True),     # the widest value dimension
    (2, 4, 17, 512, 1024, torch.float32, False),
    (4, 1, 1, 512, 2048, torch.bfloat16, True),     # one token: a single, partial reduction block
    (5, 13, 5, 2048, 64, torch.float32, True),      # one row block per head; 260 workgroups (no XCD remap)
]


@pytest.mark.parametrize("B,H,T,dk,dv,dtype,state", ROWS_CASES)
def test_wide_heads_row_parallel(B, H, T, dk, dv, dtype, state):
    """Every output against the oracle; against the column-parallel kernel
    (no workspace) the final state is the same bits (the same update, in the
    same order, per entry) and y differs only in the order of its sum."""
    pm = _pm()
    assert pm.workspace_size(B, T, H, dk, dv) > 0
    w = workloads.WORKLOADS[0].with_(B=B, H=H, dk=dk, dv=dv, dtype=dtype, A_mode="logspace16")
    _announce("wide head row-parallel fwd", B=B, H=H, T=T, dk=dk, dv=dv, dtype=dtype, state=state)
    inp = workloads.make_inputs(w, T=T, seed=3 * dk + dv + T)
    if state:
        inp["mu0"], inp["I0"] = workloads.random_state(B, H, dv, dk, inp["I_prior"], seed=dk + 1)
    y, muT, IT = _run_fwd(inp)
    _compare_full(inp, y, muT, IT, tol_for(dtype))
    g = to_device(inp, DEV)
    none = torch.empty(0, dtype=torch.uint8, device=DEV)
    y_c, mu_c, I_c = pm.fwd_chunked(*gpu_args(g), mu0=g.get("mu0"), I0=g.get("I0"), workspace=none,
                                    out_dtype=torch.float32)
    y_r, _, _ = pm.fwd_chunked(*gpu_args(g), mu0=g.get("mu0"), I0=g.get("I0"), out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(mu_c, muT) and torch.equal(I_c, IT)
    assert rel_err(y_r, y_c) <= 1e-5


def test_wide_heads_row_parallel_resume_in_place():
    """muT/IT aliasing mu0/I0: each lane reads its entries before the first
    token and writes the same entries after the last, so in place equals out
    of place bit for bit."""
    B, H, T, dk, dv = 1, 2, 13, 2048, 2048
    w = workloads.WORKLOADS[0].with_(B=B, H=H, dk=dk, dv=dv, dtype=torch.bfloat16, A_mode="logspace16")
    _announce("wide head row-parallel in-place resume", B=B, H=H, T=T, dk=dk, dv=dv)
    inp = workloads.make_inputs(w, T=T, seed=91)
    inp["mu0"], inp["I0"] = workloads.random_state(B, H, dv, dk, inp["I_prior"], seed=92)
    g = to_device(inp, DEV)
    pm = _pm()
    y1, mu1, I1 = pm.fwd_chunked(*gpu_args(g), mu0=g["mu0"], I0=g["I0"])
    mu, I = g["mu0"].clone(), g["I0"].clone()
    y2, mu2, I2 = pm.fwd_chunked(*gpu_args(g), mu0=mu, I0=I, muT=mu, IT=I)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2) and torch.equal(mu1, mu2) and torch.equal(I1, I2)
    assert mu2.data_ptr() == mu.data_ptr()


@pytest.mark.parametrize("D", [512, 2048])
def test_recurrent_shape_full_size_sampled_rows(D):
    """The recurrent-kernel shape the bench times (B=16, T=2048, H=1,
    d_k = d_v = D, bf16), through the same launch; the oracle runs on sampled
    value rows of sampled sequences (rows are independent: row i's state and
    y_i depend only on beta_i, v_i and the shared k, q, dt), every key column."""
    w = workloads.WORKLOADS[2].with_(B=16, T=2048, H=1, dk=D, dv=D)
    _announce("recurrent shape full size, sampled rows", B=16, T=2048, H=1, D=D)
    inp = workloads.make_inputs(w, seed=70 + D // 512)
    assert _pm().workspace_size(w.B, w.T, w.H, D, D) > 0
    y, muT, IT = _run_fwd(inp)
    bs = [0, 7, 15]
    rows = [0, 1, 63, 64, 255, 256, D // 2 + 5, D - 1]
    sub = {n: (x[bs] if n in ("q", "k", "dt") else x) for n, x in inp.items()}
    sub["v"] = inp["v"][bs][..., rows]
    sub["beta"] = inp["beta"][bs][..., rows]
    y_ref, mu_ref, I_ref = oracle.fwd(**sub, nthreads=len(bs))
    assert_close("y (sampled rows)", to_np(y)[bs][..., rows], y_ref, TOL_BF16)
    assert_close("muT (sampled rows)", to_np(muT)[bs][:, :, rows, :], mu_ref, TOL_F32)
    assert_close("IT (sampled rows)", to_np(IT)[bs][:, :, rows, :], I_ref, TOL_F32)


def test_wide_head_256_time_split_matches_single_pass():
    w = workloads.WORKLOADS[0].with_(B=1, H=1, dk=256, dv=64, A_mode="logspace16")
    _announce("dk=256 time split", T=700, dk=256, dv=64)
    inp = workloads.make_inputs(w, T=700, seed=256)
    g = to_device(inp, DEV)
    y1, mu1, I1 = _pm().fwd_chunked(*gpu_args(g), segments=1)
    y3, mu3, I3 = _pm().fwd_chunked(*gpu_args(g), segments=3)
    torch.cuda.synchronize()
    assert rel_err(y3, y1) <= 1e-5 and rel_err(mu3, mu1) <= 1e-5 and rel_err(I3, I1) <= 1e-6
    _compare_full(inp, y1, mu1, I1, TOL_F32)
