"""Pins of the oracle's block-diagonal backward (``oracle.bwd_blockdiag``).

The forward is the Gaussian update of each value row with the precision kept
block-diagonal along the key axis ("Learning to Remember, Learn, and Forget
in Attention-Based Models", slides, backup frame "dropping precision
correlations changes the mean", and the closing question on limited
cross-key correlations).  The pages print no backward, so the gradient is
fixed by calculus.  The pins:

* central finite differences of the oracle's forward ``fwd_blockdiag`` for
  every input (q, k, v, beta, dt, A, I_prior, mu0 and every entry of P0),
  blocks of 2 and 4, with and without a start state and final-state
  gradients;
* block 1 is Eq. (5): its gradients equal those of the C oracle's backward
  ``oracle.bwd`` (with I0 = P0 and gIT = gPT);
* T = 0: the start state's gradients are the final state's, nothing else moves;
* planted mistakes in a separate numpy transcription must each fail a pin.
"""
import math

import numpy as np
import pytest

import oracle

GRAD_OF = {"q": "gq", "k": "gk", "v": "gv", "beta": "gbeta", "dt": "gdt", "A": "gA",
           "I_prior": "gIp", "mu0": "gmu0", "P0": "gP0"}
FD_TOL = 1e-6


def _inputs(rng, B, T, H, dk, dv, block, state=True):
    nb = dk // block
    d = {
        "q": rng.normal(size=(B, T, H, dk)),
        "k": rng.normal(size=(B, T, H, dk)) / math.sqrt(dk),
        "v": rng.normal(size=(B, T, H, dv)),
        "beta": rng.uniform(0.1, 1.0, size=(B, T, H, dv)),
        "dt": rng.uniform(0.05, 0.8, size=(B, T, H)),
        "A": rng.uniform(0.5, 4.0, size=H),
        "I_prior": rng.uniform(0.5, 1.5, size=H),
        "mu0": None, "P0": None,
    }
    if state:
        L = 0.4 * rng.normal(size=(B, H, dv, nb, block, block))
        d["mu0"] = rng.normal(size=(B, H, dv, dk))
        d["P0"] = d["I_prior"][None, :, None, None, None, None] * np.eye(block) + L @ L.swapaxes(-1, -2)
    return d


def _loss(inp, block, gy, gmuT, gPT):
    y, m, P = oracle.fwd_blockdiag(**inp, block=block)
    L = float((y * gy).sum())
    if gmuT is not None:
        L += float((m * gmuT).sum())
    if gPT is not None:
        L += float((P * gPT).sum())
    return L


def _finite_differences(inp, block, gy, gmuT, gPT, h=1e-6):
    fd = {}
    for name, g in GRAD_OF.items():
        if inp[name] is None:
            continue
        base = inp[name]
        out = np.zeros_like(base)
        for idx in np.ndindex(base.shape):
            x = base.copy()
            step = h * max(1.0, abs(base[idx]))
            x[idx] = base[idx] + step
            lp = _loss(dict(inp, **{name: x}), block, gy, gmuT, gPT)
            x[idx] = base[idx] - step
            lm = _loss(dict(inp, **{name: x}), block, gy, gmuT, gPT)
            out[idx] = (lp - lm) / (2 * step)
        fd[g] = out
    return fd


def _normwise(a, b):
    return float(np.abs(np.asarray(a) - np.asarray(b)).max() / max(np.abs(b).max(), 1e-30))


def _case(seed, block, state, final, dk=4, T=4):
    rng = np.random.default_rng(seed)
    B, H, dv = 1, 2, 2
    inp = _inputs(rng, B, T, H, dk, dv, block, state=state)
    gy = rng.normal(size=(B, T, H, dv))
    gmuT = rng.normal(size=(B, H, dv, dk)) if final else None
    gPT = rng.normal(size=(B, H, dv, dk // block, block, block)) if final else None
    return inp, gy, gmuT, gPT


def _fd_errors(bwd, seed, block, state, final):
    inp, gy, gmuT, gPT = _case(seed, block, state, final)
    got = bwd(**inp, block=block, gy=gy, gmuT=gmuT, gPT=gPT)
    fd = _finite_differences(inp, block, gy, gmuT, gPT)
    return {g: _normwise(got[g], fd[g]) for g in fd}


@pytest.mark.parametrize("block,state,final", [(2, True, True), (2, False, True), (2, True, False),
                                               (4, True, True), (4, False, False)])
def test_blockdiag_bwd_matches_finite_differences(block, state, final):
    errs = _fd_errors(oracle.bwd_blockdiag, 11 + block + 2 * state + final, block, state, final)
    bad = {g: e for g, e in errs.items() if e > FD_TOL}
    assert not bad, bad


def test_blockdiag_bwd_block1_is_the_exact_backward():
    """Block 1 keeps only the diagonal: Eq. (5), whose backward the C oracle
    pins on its own; the two agree to float64 rounding."""
    rng = np.random.default_rng(5)
    B, T, H, dk, dv = 2, 9, 2, 3, 4
    inp = _inputs(rng, B, T, H, dk, dv, 1, state=True)
    gy = rng.normal(size=(B, T, H, dv))
    gmuT = rng.normal(size=(B, H, dv, dk))
    gPT = rng.normal(size=(B, H, dv, dk, 1, 1))
    got = oracle.bwd_blockdiag(**inp, block=1, gy=gy, gmuT=gmuT, gPT=gPT)
    I0 = np.ascontiguousarray(inp["P0"][..., 0, 0])
    ref = oracle.bwd(inp["q"], inp["k"], inp["v"], inp["beta"], inp["dt"], inp["A"], inp["I_prior"], gy,
                     mu0=inp["mu0"], I0=I0, gmuT=gmuT, gIT=np.ascontiguousarray(gPT[..., 0, 0]))
    for g in ("gq", "gk", "gv", "gbeta", "gdt", "gA", "gIp", "gmu0"):
        assert _normwise(got[g], ref[g]) < 1e-10, g
    assert _normwise(got["gP0"][..., 0, 0], ref["gI0"]) < 1e-10
    # the default start state too (gIp then collects the start state's share)
    got = oracle.bwd_blockdiag(**dict(inp, mu0=None, P0=None), block=1, gy=gy, gmuT=gmuT, gPT=gPT)
    ref = oracle.bwd(inp["q"], inp["k"], inp["v"], inp["beta"], inp["dt"], inp["A"], inp["I_prior"], gy,
                     gmuT=gmuT, gIT=np.ascontiguousarray(gPT[..., 0, 0]))
    for g in ("gq", "gk", "gv", "gbeta", "gdt", "gA", "gIp", "gmu0"):
        assert _normwise(got[g], ref[g]) < 1e-10, g


def test_blockdiag_bwd_empty_sequence():
    rng = np.random.default_rng(8)
    inp = _inputs(rng, 1, 0, 2, 4, 2, 2, state=True)
    gmuT = rng.normal(size=(1, 2, 2, 4))
    gPT = rng.normal(size=(1, 2, 2, 2, 2, 2))
    got = oracle.bwd_blockdiag(**inp, block=2, gy=np.zeros((1, 0, 2, 2)), gmuT=gmuT, gPT=gPT)
    assert np.allclose(got["gmu0"], gmuT, rtol=1e-12, atol=1e-12)
    assert np.allclose(got["gP0"], gPT, rtol=1e-12, atol=1e-12)
    assert not got["gA"].any() and not got["gIp"].any()


# ---------------------------------------------------------------------------
# planted mistakes: a separate transcription with switches, each of which the
# finite-difference pin must reject
# ---------------------------------------------------------------------------

def _bwd_copy(q, k, v, beta, dt, A, I_prior, block, gy, mu0=None, P0=None, gmuT=None, gPT=None, kind=None):
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    bs, nb = block, dk // block
    eye = np.eye(bs)
    out = {n: np.zeros(x.shape) for n, x in (("gq", q), ("gk", k), ("gv", v), ("gbeta", v), ("gdt", dt))}
    out["gA"], out["gIp"] = np.zeros(H), np.zeros(H)
    out["gmu0"], out["gP0"] = np.zeros((B, H, dv, dk)), np.zeros((B, H, dv, nb, bs, bs))
    sol = lambda M, x: np.linalg.solve(M, x[..., None])[..., 0]
    for b in range(B):
        for h in range(H):
            P = (np.broadcast_to(I_prior[h] * eye, (dv, nb, bs, bs)).copy() if mu0 is None else P0[b, h].copy())
            m0 = np.zeros((dv, nb, bs)) if mu0 is None else mu0[b, h].reshape(dv, nb, bs)
            hs = [np.einsum("rnij,rnj->rni", P, m0)]
            Ps = [P]
            for t in range(T):
                a = math.exp(-A[h] * dt[b, t, h])
                kb = k[b, t, h].reshape(nb, bs)
                Ps.append(a * Ps[-1] + (1 - a) * I_prior[h] * eye +
                          beta[b, t, h][:, None, None, None] * (kb[:, :, None] * kb[:, None, :])[None])
                hs.append(a * hs[-1] + (beta[b, t, h] * v[b, t, h])[:, None, None] * kb[None])
            Gh, GP = np.zeros((dv, nb, bs)), np.zeros((dv, nb, bs, bs))
            if gmuT is not None:
                w = sol(Ps[T], gmuT[b, h].reshape(dv, nb, bs))
                Gh += w
                GP -= w[..., :, None] * sol(Ps[T], hs[T])[..., None, :]
            if gPT is not None:
                GP += gPT[b, h]
            for t in range(T - 1, -1, -1):
                a = math.exp(-A[h] * dt[b, t, h])
                kb, qb = k[b, t, h].reshape(nb, bs), q[b, t, h].reshape(nb, bs)
                bt = beta[b, t, h]
                mu_t = sol(Ps[t + 1], hs[t + 1] if kind != "readout_old_state" else hs[t])
                out["gq"][b, t, h] += (gy[b, t, h][:, None, None] * mu_t).sum(0).reshape(dk)
                w = sol(Ps[t + 1], gy[b, t, h][:, None, None] * qb[None])
                Gh += w
                GP -= w[..., :, None] * mu_t[..., None, :]
                GPs = GP if kind == "gk_one_sided" else GP + GP.swapaxes(-1, -2)
                out["gk"][b, t, h] += ((bt * v[b, t, h])[:, None, None] * Gh).sum(0).reshape(dk)
                out["gk"][b, t, h] += (bt[:, None, None] * np.einsum("rnij,nj->rni", GPs, kb)).sum(0).reshape(dk)
                g_bv = (Gh * kb[None]).sum((1, 2))
                out["gv"][b, t, h] = g_bv * bt
                out["gbeta"][b, t, h] = g_bv * v[b, t, h] + np.einsum("rnij,ni,nj->r", GP, kb, kb)
                g_a = (Gh * hs[t]).sum() + (GP * Ps[t]).sum()
                g_c = np.trace(GP, axis1=-2, axis2=-1).sum()
                u = (I_prior[h] * g_c - g_a) if kind != "gate_sign" else (g_a - I_prior[h] * g_c)
                out["gdt"][b, t, h] = A[h] * a * u
                out["gA"][h] += dt[b, t, h] * a * u
                out["gIp"][h] += (1 - a) * g_c
                if kind != "adjoint_not_decayed":
                    Gh *= a
                    GP *= a
            out["gmu0"][b, h] = np.einsum("rnji,rnj->rni", Ps[0], Gh).reshape(dv, dk)
            out["gP0"][b, h] = GP + Gh[..., :, None] * m0[..., None, :]
            if mu0 is None and kind != "prior_share_missing":
                out["gIp"][h] += np.trace(out["gP0"][b, h], axis1=-2, axis2=-1).sum()
    return out


BD_MUTANTS = ["readout_old_state", "gk_one_sided", "gate_sign", "adjoint_not_decayed", "prior_share_missing"]


def test_unmutated_copy_agrees_with_oracle():
    inp, gy, gmuT, gPT = _case(3, 2, True, True, T=6)
    a = oracle.bwd_blockdiag(**inp, block=2, gy=gy, gmuT=gmuT, gPT=gPT)
    b = _bwd_copy(**inp, block=2, gy=gy, gmuT=gmuT, gPT=gPT)
    for g in a:
        assert _normwise(b[g], a[g]) < 1e-12, g


@pytest.mark.parametrize("kind", BD_MUTANTS)
def test_blockdiag_pins_catch_planted_mistake(kind):
    state = kind != "prior_share_missing"
    bwd = lambda **kw: _bwd_copy(**kw, kind=kind)
    errs = _fd_errors(bwd, 21, 2, state, True)
    assert max(errs.values()) > 1e-3, (kind, errs)
