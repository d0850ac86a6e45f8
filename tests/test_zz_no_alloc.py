"""GPU test of palimpsa_fwd_chunked_noalloc, the forward for callers that
cannot allocate: it keeps a time split's segment summaries and start-state
copy in the library's fixed per-GPU scratch array instead of a workspace.
Its results must be those of palimpsa_fwd_chunked with a workspace (the same
split, so the same bits), call after call, whatever an earlier call left in
the shared array.
"""
import pytest
import torch

import oracle
import workloads
from parity_utils import TOL_F32, assert_close, gpu_args, to_device

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def _pm():
    import bayesian_metaplastic_memory_amd as pm
    return pm


def _announce(what, **shape):
    print("\n[case] %s %s" % (what, " ".join("%s=%s" % kv for kv in shape.items())), flush=True)


def _both(inp, segments, start):
    pm = _pm()
    g = to_device(inp, DEV)
    kw = dict(segments=segments)
    if start is not None:
        kw.update(mu0=start[0].to(DEV), I0=start[1].to(DEV))
    ref = pm.fwd_chunked(*gpu_args(g), **kw)
    out = pm.fwd_chunked_noalloc(*gpu_args(g), **kw)
    torch.cuda.synchronize()
    return ref, out


def test_noalloc_matches_the_workspace_forward_on_consecutive_calls():
    pm = _pm()
    assert pm.noalloc_scratch_bytes() == 64 << 20
    # first call: the long-context head count (auto split into 3 segments),
    # bf16, from a random start state
    w = workloads.WORKLOADS[4]
    T = 4096
    _announce("noalloc forward, call 1", B=w.B, H=w.H, T=T, d=w.dk, segments="auto")
    inp = workloads.make_inputs(w, T=T)
    start = workloads.random_state(w.B, w.H, w.dv, w.dk, inp["I_prior"], seed=21)
    print("  split workspace bytes: %d" % pm.workspace_size(w.B, T, w.H, w.dk, w.dv, 0), flush=True)
    assert pm.workspace_size(w.B, T, w.H, w.dk, w.dv, 0) > 0
    (y_r, mu_r, I_r), (y_n, mu_n, I_n) = _both(inp, 0, start)
    assert torch.equal(y_r, y_n) and torch.equal(mu_r, mu_n) and torch.equal(I_r, I_n)
    # second call, smaller: fp32, 5 explicit segments, default start state
    w2 = workloads.WORKLOADS[1].with_(B=1, H=3)
    T2 = 700
    _announce("noalloc forward, call 2 (smaller)", B=w2.B, H=w2.H, T=T2, d=w2.dk, segments=5)
    inp2 = workloads.make_inputs(w2, T=T2)
    assert 0 < pm.workspace_size(w2.B, T2, w2.H, w2.dk, w2.dv, 5) < pm.workspace_size(w.B, T, w.H, w.dk, w.dv, 0)
    (y_r, mu_r, I_r), (y_n, mu_n, I_n) = _both(inp2, 5, None)
    assert torch.equal(y_r, y_n) and torch.equal(mu_r, mu_n) and torch.equal(I_r, I_n)
    y_ref, mu_ref, I_ref = oracle.fwd(**inp2)
    assert_close("y", y_n, y_ref, TOL_F32)
    assert_close("muT", mu_n, mu_ref, TOL_F32)
    assert_close("IT", I_n, I_ref, TOL_F32)


def test_noalloc_in_place_resume_and_scratch_limit():
    pm = _pm()
    w = workloads.WORKLOADS[2].with_(B=2, H=16)
    T = 1024
    _announce("noalloc forward, in-place resume", B=w.B, H=w.H, T=T, d=w.dk, segments=4)
    inp = workloads.make_inputs(w, T=T)
    mu0, I0 = workloads.random_state(w.B, w.H, w.dv, w.dk, inp["I_prior"], seed=22)
    g = to_device(inp, DEV)
    y_r, mu_r, I_r = pm.fwd_chunked(*gpu_args(g), mu0=mu0.to(DEV), I0=I0.to(DEV), segments=4)
    mu, I = mu0.to(DEV), I0.to(DEV)
    y_n, mu_n, I_n = pm.fwd_chunked_noalloc(*gpu_args(g), mu0=mu, I0=I, muT=mu, IT=I, segments=4)
    torch.cuda.synchronize()
    assert mu_n.data_ptr() == mu.data_ptr()
    assert torch.equal(y_r, y_n) and torch.equal(mu_r, mu_n) and torch.equal(I_r, I_n)
    # a split that needs more than the fixed array: refused before any launch
    B, H, T3, d = 8, 32, 64 * 64, 128
    need = pm.workspace_size(B, T3, H, d, d, 64)
    print("  64-segment split needs %d bytes (limit %d)" % (need, pm.noalloc_scratch_bytes()), flush=True)
    assert need > pm.noalloc_scratch_bytes()
    x = torch.zeros(B, T3, H, d, dtype=torch.bfloat16, device=DEV)
    dt = torch.zeros(B, T3, H, dtype=torch.bfloat16, device=DEV)
    A, Ip = torch.ones(H, device=DEV), torch.ones(H, device=DEV)
    with pytest.raises(pm.PalimpsaError) as e:
        pm.fwd_chunked_noalloc(x, x, x, x, dt, A, Ip, segments=64)
    assert e.value.status == 5
    with pytest.raises(pm.PalimpsaError) as e:
        pm.fwd_chunked_noalloc(x, x, x, x, dt, A, Ip, segments=64, chunk=3)
    assert e.value.status == 1
