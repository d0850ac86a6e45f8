"""Pins of the oracle's frozen-importance backward (``oracle.bwd_mamba2_limit``).

With the importance held at I_prior the recurrence is the Mamba2 limit of
Palimpsa ("Learning to Remember, Learn, and Forget in Attention-Based
Models", slides, frame "The Mamba2 limit enables a gradual model upgrade"):
m_t = alpha_t m_{t-1} + (beta_t v_t / I_prior) k_t^T, y_t = m_t q_t.  The pages
print no backward, so the gradient is fixed by calculus.  The pins:

* central finite differences of the oracle's forward ``fwd_mamba2_limit``
  for every input, with and without a start state and final-state
  gradients, and with v holding beta . v (beta None);
* a closed form at alpha = 1 (dt = 0), where the state is a plain running
  sum and so is the adjoint: m_t = m_0 + sum_{s<=t} w_s k_s^T and
  G_t = gmuT + sum_{u>=t} gy_u q_u^T give gq_t = m_t^T gy_t, gk_t = G_t^T w_t,
  gw_t = G_t k_t;
* T = 0: the gradient of the start state is gmuT and nothing else moves;
* heads and sequences are independent;
* planted mistakes in a separate numpy transcription must each fail a pin.
"""
import math

import numpy as np
import pytest

import oracle

GRAD_OF = {"q": "gq", "k": "gk", "v": "gv", "beta": "gbeta", "dt": "gdt", "A": "gA",
           "I_prior": "gIp", "mu0": "gmu0"}
FD_TOL = 1e-6


def _inputs(rng, B, T, H, dk, dv, state=True, vstar=False):
    d = {
        "q": rng.normal(size=(B, T, H, dk)),
        "k": rng.normal(size=(B, T, H, dk)) / math.sqrt(dk),
        "v": rng.normal(size=(B, T, H, dv)),
        "beta": None if vstar else rng.uniform(0.1, 1.0, size=(B, T, H, dv)),
        "dt": rng.uniform(0.05, 0.8, size=(B, T, H)),
        "A": rng.uniform(0.5, 4.0, size=H),
        "I_prior": rng.uniform(0.5, 1.5, size=H),
        "mu0": rng.normal(size=(B, H, dv, dk)) if state else None,
    }
    return d


def _fwd(inp):
    args = dict(inp)
    if args["beta"] is None:
        args["beta"] = np.ones(args["v"].shape)
    return oracle.fwd_mamba2_limit(**args)


def _loss(inp, gy, gmuT):
    y, m = _fwd(inp)
    L = float((y * gy).sum())
    if gmuT is not None:
        L += float((m * gmuT).sum())
    return L


def _finite_differences(inp, gy, gmuT, h=1e-6):
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
            lp = _loss(dict(inp, **{name: x}), gy, gmuT)
            x[idx] = base[idx] - step
            lm = _loss(dict(inp, **{name: x}), gy, gmuT)
            out[idx] = (lp - lm) / (2 * step)
        fd[g] = out
    return fd


def _normwise(a, b):
    return float(np.abs(np.asarray(a) - np.asarray(b)).max() / max(np.abs(b).max(), 1e-30))


def _fd_errors(bwd, seed, state, final, vstar=False, T=5):
    rng = np.random.default_rng(seed)
    inp = _inputs(rng, 2, T, 2, 3, 2, state=state, vstar=vstar)
    gy = rng.normal(size=(2, T, 2, 2))
    gmuT = rng.normal(size=(2, 2, 2, 3)) if final else None
    got = bwd(**inp, gy=gy, gmuT=gmuT)
    fd = _finite_differences(inp, gy, gmuT)
    return {g: _normwise(got[g], fd[g]) for g in fd}


@pytest.mark.parametrize("state,final", [(True, True), (False, True), (True, False), (False, False)])
def test_frozen_bwd_matches_finite_differences(state, final):
    err = _fd_errors(oracle.bwd_mamba2_limit, seed=7 + 2 * state + final, state=state, final=final)
    assert all(e < FD_TOL for e in err.values()), err


def test_frozen_bwd_vstar_matches_finite_differences():
    err = _fd_errors(oracle.bwd_mamba2_limit, seed=31, state=True, final=True, vstar=True)
    assert all(e < FD_TOL for e in err.values()), err
    rng = np.random.default_rng(31)
    inp = _inputs(rng, 2, 5, 2, 3, 2, vstar=True)
    assert oracle.bwd_mamba2_limit(**inp, gy=rng.normal(size=(2, 5, 2, 2)))["gbeta"] is None


def test_frozen_bwd_closed_form_without_decay():
    rng = np.random.default_rng(5)
    B, T, H, dk, dv = 1, 6, 2, 3, 4
    inp = _inputs(rng, B, T, H, dk, dv)
    inp["dt"] = np.zeros((B, T, H))
    gy = rng.normal(size=(B, T, H, dv))
    gmuT = rng.normal(size=(B, H, dv, dk))
    got = oracle.bwd_mamba2_limit(**inp, gy=gy, gmuT=gmuT)
    for h in range(H):
        w = inp["beta"][0, :, h] * inp["v"][0, :, h] / inp["I_prior"][h]
        writes = np.einsum("ti,tj->tij", w, inp["k"][0, :, h])
        m = inp["mu0"][0, h] + np.cumsum(writes, axis=0)                 # m_t, t = 0..T-1
        reads = np.einsum("ti,tj->tij", gy[0, :, h], inp["q"][0, :, h])
        G = gmuT[0, h] + np.cumsum(reads[::-1], axis=0)[::-1]             # G_t
        gw = np.einsum("tij,tj->ti", G, inp["k"][0, :, h])
        assert _normwise(got["gq"][0, :, h], np.einsum("tij,ti->tj", m, gy[0, :, h])) < 1e-12
        assert _normwise(got["gk"][0, :, h], np.einsum("tij,ti->tj", G, w)) < 1e-12
        assert _normwise(got["gv"][0, :, h], gw * inp["beta"][0, :, h] / inp["I_prior"][h]) < 1e-12
        assert _normwise(got["gmu0"][0, h], G[0]) < 1e-12


def test_frozen_bwd_empty_sequence():
    rng = np.random.default_rng(9)
    inp = _inputs(rng, 2, 0, 3, 4, 2)
    gmuT = rng.normal(size=(2, 3, 2, 4))
    got = oracle.bwd_mamba2_limit(**inp, gy=np.zeros((2, 0, 3, 2)), gmuT=gmuT)
    assert np.array_equal(got["gmu0"], gmuT)
    assert not got["gA"].any() and not got["gIp"].any() and got["gq"].size == 0


def test_frozen_bwd_heads_and_sequences_are_independent():
    rng = np.random.default_rng(21)
    inp = _inputs(rng, 2, 7, 3, 3, 2)
    gy = rng.normal(size=(2, 7, 3, 2))
    gmuT = rng.normal(size=(2, 3, 2, 3))
    full = oracle.bwd_mamba2_limit(**inp, gy=gy, gmuT=gmuT)
    b, h = 1, 2
    sub = {n: (None if x is None else (x[[h]] if n in ("A", "I_prior") else
                                       x[[b]][:, :, [h]] if x.ndim >= 3 and x.shape[1] == 7 else
                                       x[[b]][:, [h]])) for n, x in inp.items()}
    part = oracle.bwd_mamba2_limit(**sub, gy=gy[[b]][:, :, [h]], gmuT=gmuT[[b]][:, [h]])
    assert _normwise(part["gq"][0, :, 0], full["gq"][b, :, h]) < 1e-12
    assert _normwise(part["gdt"][0, :, 0], full["gdt"][b, :, h]) < 1e-12
    assert _normwise(part["gmu0"][0, 0], full["gmu0"][b, h]) < 1e-12


# A second transcription (all states kept, no checkpoints) with planted
# mistakes: each mutant must fail the finite-difference pins.
def _np_frozen_bwd(kind):
    def bwd(q, k, v, beta, dt, A, I_prior, gy, mu0=None, gmuT=None):
        vstar = beta is None
        beta = np.ones(v.shape) if vstar else beta
        B, T, H, dk = q.shape
        dv = v.shape[-1]
        out = {n: np.zeros(x.shape) for n, x in (("gq", q), ("gk", k), ("gv", v), ("gbeta", v), ("gdt", dt))}
        out["gA"], out["gIp"], out["gmu0"] = np.zeros(H), np.zeros(H), np.zeros((B, H, dv, dk))
        for b in range(B):
            for h in range(H):
                a = np.exp(-A[h] * dt[b, :, h])
                w = beta[b, :, h] * v[b, :, h] / (1.0 if kind == "w_not_scaled" else I_prior[h])
                ms = [np.zeros((dv, dk)) if mu0 is None else mu0[b, h]]
                for t in range(T):
                    ms.append(a[t] * ms[-1] + np.outer(w[t], k[b, t, h]))
                G = np.zeros((dv, dk)) if gmuT is None else gmuT[b, h].copy()
                for t in range(T - 1, -1, -1):
                    if kind == "readout_after_decay":
                        pass
                    else:
                        G = G + np.outer(gy[b, t, h], q[b, t, h])
                    out["gq"][b, t, h] = (ms[t] if kind == "gq_uses_old_state" else ms[t + 1]).T @ gy[b, t, h]
                    out["gk"][b, t, h] = G.T @ w[t]
                    gw = G @ k[b, t, h]
                    ga = float(np.sum(G * ms[t]))
                    out["gv"][b, t, h] = gw * beta[b, t, h] / I_prior[h]
                    out["gbeta"][b, t, h] = gw * v[b, t, h] / I_prior[h]
                    if kind != "gIp_missing":
                        out["gIp"][h] -= float(gw @ w[t]) / I_prior[h]
                    sgn = 1.0 if kind == "gdt_sign" else -1.0
                    out["gdt"][b, t, h] = sgn * A[h] * a[t] * ga
                    out["gA"][h] -= dt[b, t, h] * a[t] * ga
                    if kind != "adjoint_not_decayed":
                        G = a[t] * G
                    if kind == "readout_after_decay":
                        G = G + a[t] * np.outer(gy[b, t, h], q[b, t, h])
                out["gmu0"][b, h] = G
        if vstar:
            out["gbeta"] = None
        return out
    return bwd


FROZEN_MUTANTS = ["w_not_scaled", "readout_after_decay", "gq_uses_old_state", "gIp_missing",
                  "gdt_sign", "adjoint_not_decayed"]


def _pins_pass(bwd):
    for state, final in ((True, True), (False, False)):
        err = _fd_errors(bwd, seed=50 + state, state=state, final=final, T=4)
        if not all(e < FD_TOL for e in err.values()):
            return False
    return True


def test_numpy_transcription_agrees_with_oracle():
    rng = np.random.default_rng(17)
    inp = _inputs(rng, 2, 9, 2, 3, 4)
    gy = rng.normal(size=(2, 9, 2, 4))
    gmuT = rng.normal(size=(2, 2, 4, 3))
    a = oracle.bwd_mamba2_limit(**inp, gy=gy, gmuT=gmuT)
    b = _np_frozen_bwd("none")(**inp, gy=gy, gmuT=gmuT)
    for g in GRAD_OF.values():
        assert _normwise(a[g], b[g]) < 1e-12, g


def test_unmutated_frozen_copy_passes_pins():
    assert _pins_pass(_np_frozen_bwd("none"))


@pytest.mark.parametrize("kind", FROZEN_MUTANTS)
def test_frozen_pins_catch_planted_mistake(kind):
    assert not _pins_pass(_np_frozen_bwd(kind))
