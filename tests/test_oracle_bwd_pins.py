"""Pins of the oracle's backward (``oracle.bwd``) against facts other than itself.

The pages train through the recurrence but print no backward, so the
gradient is fixed by calculus on Eq. (5) and the gate of Eq. (9) ("Learning
to Remember, Learn, and Forget in Attention-Based Models", slides, frames
"Palimpsa updates content and importance together" and "Forgetting
discounts evidence and restores the prior").  The pins:

* central finite differences of the oracle's forward, for every input
  (tokens, gate parameters, prior, initial state), with and without
  final-state gradients and with the default start state;
* a closed form at alpha = 1 (dt = 0), where the recurrence is a plain sum:
  I_T = I_0 + sum_t beta_t k_t^2 and mu_T = (I_0 mu_0 + sum_t beta_t v_t k_t) / I_T;
* an exact cancellation: one token from the default state gives
  I_1 = I_prior + beta k^2 and mu_1 = beta v k / I_1 whatever alpha is, so the
  gradient with respect to dt and A is zero;
* T = 0: the final state is the initial state;
* planted mistakes in a separate numpy transcription must each fail a pin.
"""
import math

import numpy as np
import pytest

import oracle


def _inputs(rng, B, T, H, dk, dv, state=True):
    d = {
        "q": rng.normal(size=(B, T, H, dk)),
        "k": rng.normal(size=(B, T, H, dk)) / math.sqrt(dk),
        "v": rng.normal(size=(B, T, H, dv)),
        "beta": rng.uniform(0.1, 1.0, size=(B, T, H, dv)),
        "dt": rng.uniform(0.05, 0.6, size=(B, T, H)),
        "A": rng.uniform(0.5, 4.0, size=H),
        "I_prior": rng.uniform(0.5, 1.5, size=H),
        "mu0": None, "I0": None,
    }
    if state:
        d["mu0"] = rng.normal(size=(B, H, dv, dk))
        d["I0"] = rng.uniform(0.5, 3.0, size=(B, H, dv, dk))
    return d


def _loss(fwd, inp, gy, gmuT, gIT, **kw):
    y, mu, I = fwd(**inp, **kw)
    L = float((y * gy).sum())
    if gmuT is not None:
        L += float((mu * gmuT).sum())
    if gIT is not None:
        L += float((I * gIT).sum())
    return L


GRAD_OF = {"q": "gq", "k": "gk", "v": "gv", "beta": "gbeta", "dt": "gdt", "A": "gA",
           "I_prior": "gIp", "mu0": "gmu0", "I0": "gI0"}


def _finite_differences(fwd, inp, gy, gmuT, gIT, h=1e-6, **kw):
    """Central differences of L for every element of every input."""
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
            lp = _loss(fwd, dict(inp, **{name: x}), gy, gmuT, gIT, **kw)
            x[idx] = base[idx] - step
            lm = _loss(fwd, dict(inp, **{name: x}), gy, gmuT, gIT, **kw)
            out[idx] = (lp - lm) / (2 * step)
        fd[g] = out
    return fd


def _normwise(a, b):
    scale = max(np.abs(b).max(), 1e-30)
    return np.abs(a - b).max() / scale


def _fd_pin_errors(bwd, seed, state, final_grads, T=7, per_entry=False, vstar=False):
    rng = np.random.default_rng(seed)
    B, H, dk, dv = 2, 2, 3, 2
    inp = _inputs(rng, B, T, H, dk, dv, state=state)
    if per_entry:
        inp["I_prior"] = rng.uniform(0.5, 1.5, size=(H, dv, dk))
    gy = rng.normal(size=(B, T, H, dv))
    gmuT = rng.normal(size=(B, H, dv, dk)) if final_grads else None
    gIT = rng.normal(size=(B, H, dv, dk)) if final_grads else None
    kw = {"vstar": True} if vstar else {}
    got = bwd(**inp, gy=gy, gmuT=gmuT, gIT=gIT, **kw)
    fd = _finite_differences(oracle.fwd, inp, gy, gmuT, gIT, **kw)
    return {g: _normwise(got[g], ref) for g, ref in fd.items()}


# central differences with h = 1e-6 are accurate to about h^2 * f''' / f' plus
# rounding of about 1e-16 / h: a few 1e-9 relative on these inputs
FD_TOL = 1e-6


@pytest.mark.parametrize("state,final_grads", [(True, True), (False, False), (True, False), (False, True)])
def test_oracle_bwd_matches_finite_differences(state, final_grads):
    err = _fd_pin_errors(oracle.bwd, seed=3 + 2 * state + final_grads, state=state,
                         final_grads=final_grads)
    bad = {g: e for g, e in err.items() if not e < FD_TOL}
    assert not bad, bad


@pytest.mark.parametrize("per_entry,vstar,state", [(True, False, False), (True, False, True),
                                                  (False, True, True), (True, True, False)])
def test_oracle_bwd_options_match_finite_differences(per_entry, vstar, state):
    """A prior per state entry (gIp then has the state's shape) and the v*
    input (gv is then the gradient with respect to v* itself)."""
    err = _fd_pin_errors(oracle.bwd, seed=60 + per_entry + 2 * vstar + 4 * state, state=state,
                         final_grads=True, per_entry=per_entry, vstar=vstar)
    bad = {g: e for g, e in err.items() if not e < FD_TOL}
    assert not bad, bad


def test_oracle_bwd_alpha_one_closed_form():
    """dt = 0: with gy = 0, L = <gmuT, mu_T> + <gIT, I_T> and
    mu_T = (I0 mu0 + sum_t (beta v)_t k_t) / I_T,  I_T = I0 + sum_t beta_t k_t^2, so
      dL/dv_t[i]    = sum_j gmuT_ij beta_t[i] k_t[j] / I_T
      dL/dk_t[j]    = sum_i [gmuT_ij ((beta v)_t[i] - 2 mu_T beta_t[i] k_t[j]) / I_T
                             + gIT_ij 2 beta_t[i] k_t[j]]
      dL/dbeta_t[i] = sum_j [gmuT_ij (v_t[i] k_t[j] - mu_T k_t[j]^2) / I_T + gIT_ij k_t[j]^2]
      dL/dmu0 = gmuT I0 / I_T,   dL/dI0 = gmuT (mu0 - mu_T) / I_T + gIT."""
    rng = np.random.default_rng(21)
    B, T, H, dk, dv = 1, 6, 2, 4, 3
    inp = _inputs(rng, B, T, H, dk, dv)
    inp["dt"] = np.zeros((B, T, H))
    gmuT = rng.normal(size=(B, H, dv, dk))
    gIT = rng.normal(size=(B, H, dv, dk))
    got = oracle.bwd(**inp, gy=np.zeros((B, T, H, dv)), gmuT=gmuT, gIT=gIT)
    k, v, beta = inp["k"][0], inp["v"][0], inp["beta"][0]            # [T, H, d]
    I_T = inp["I0"][0] + np.einsum("thi,thj->hij", beta, k * k)
    M_T = inp["I0"][0] * inp["mu0"][0] + np.einsum("thi,thj->hij", beta * v, k)
    mu_T = M_T / I_T
    G, GI = gmuT[0], gIT[0]
    gv = np.einsum("hij,thi,thj->thi", G / I_T, beta, k)
    gk = (np.einsum("hij,thi->thj", G / I_T, beta * v)
          - 2 * np.einsum("hij,thi,thj->thj", G * mu_T / I_T, beta, k)
          + 2 * np.einsum("hij,thi,thj->thj", GI, beta, k))
    gbeta = (np.einsum("hij,thi,thj->thi", G / I_T, v, k)
             - np.einsum("hij,thj->thi", G * mu_T / I_T, k * k)
             + np.einsum("hij,thj->thi", GI, k * k))
    for name, ref in [("gv", gv), ("gk", gk), ("gbeta", gbeta)]:
        assert _normwise(got[name][0], ref) < 1e-12, name
    assert _normwise(got["gmu0"][0], G * inp["I0"][0] / I_T) < 1e-12
    assert _normwise(got["gI0"][0], G * (inp["mu0"][0] - mu_T) / I_T + GI) < 1e-12
    assert np.abs(got["gq"]).max() == 0.0


def test_oracle_bwd_single_token_from_default_state_has_no_gate_gradient():
    rng = np.random.default_rng(5)
    inp = _inputs(rng, 2, 1, 3, 4, 3, state=False)
    g = oracle.bwd(**inp, gy=rng.normal(size=(2, 1, 3, 3)))
    scale = np.abs(g["gv"]).max()
    assert np.abs(g["gdt"]).max() < 1e-14 * scale
    assert np.abs(g["gA"]).max() < 1e-14 * scale
    assert np.abs(g["gq"]).max() > 0


def test_oracle_bwd_empty_sequence_passes_final_gradients_through():
    rng = np.random.default_rng(8)
    inp = _inputs(rng, 1, 0, 2, 3, 2)
    gmuT, gIT = rng.normal(size=(1, 2, 2, 3)), rng.normal(size=(1, 2, 2, 3))
    g = oracle.bwd(**inp, gy=np.zeros((1, 0, 2, 2)), gmuT=gmuT, gIT=gIT)
    assert np.array_equal(g["gmu0"], gmuT) and np.array_equal(g["gI0"], gIT)
    assert g["gq"].shape == (1, 0, 2, 3) and np.all(g["gA"] == 0) and np.all(g["gIp"] == 0)


def test_oracle_bwd_heads_are_independent():
    """A sampled head's gradients equal its slice of a full run (the per-token
    gradients; gA and gIp are summed over the batch)."""
    rng = np.random.default_rng(9)
    inp = _inputs(rng, 2, 9, 3, 4, 4)
    gy = rng.normal(size=(2, 9, 3, 4))
    full = oracle.bwd(**inp, gy=gy)
    sub = oracle.select_heads(inp, [(1, 2)])
    part = oracle.bwd(**sub, gy=gy[1:2, :, 2:3])
    for g in ("gq", "gk", "gv", "gbeta", "gdt"):
        np.testing.assert_array_equal(part[g][0, :, 0], full[g][1, :, 2])


# ---------------------------------------------------------------------------
# planted mistakes: a numpy transcription of the same reverse-mode steps with
# switches; the unmutated copy passes the pins and agrees with the C oracle,
# and every mutant fails at least one pin.
# ---------------------------------------------------------------------------

def _np_bwd(kind):
    def bwd(q, k, v, beta, dt, A, I_prior, gy, mu0=None, I0=None, gmuT=None, gIT=None):
        B, T, H, dk = q.shape
        dv = v.shape[-1]
        default = mu0 is None
        out = {n: np.zeros_like(x) for n, x in (("gq", q), ("gk", k), ("gv", v), ("gbeta", beta), ("gdt", dt))}
        out["gA"], out["gIp"] = np.zeros(H), np.zeros(H)
        out["gmu0"], out["gI0"] = np.zeros((B, H, dv, dk)), np.zeros((B, H, dv, dk))
        for b in range(B):
            for h in range(H):
                Ip = I_prior[h]
                m = np.zeros((dv, dk)) if default else mu0[b, h].copy()
                P = np.full((dv, dk), Ip) if default else I0[b, h].copy()
                states = [(m, P)]
                for t in range(T):
                    a = math.exp(-A[h] * dt[b, t, h])
                    oma = -math.expm1(-A[h] * dt[b, t, h])
                    kk = k[b, t, h]
                    Pn = a * P + oma * Ip + np.outer(beta[b, t, h], kk * kk)
                    m = a * (P / Pn) * m + np.outer(beta[b, t, h] * v[b, t, h], kk) / Pn
                    P = Pn
                    states.append((m, P))
                gm = np.zeros((dv, dk)) if gmuT is None else gmuT[b, h].copy()
                gI = np.zeros((dv, dk)) if gIT is None else gIT[b, h].copy()
                for t in range(T - 1, -1, -1):
                    (mo, Io), (mn, In) = states[t], states[t + 1]
                    a = math.exp(-A[h] * dt[b, t, h])
                    oma = -math.expm1(-A[h] * dt[b, t, h])
                    kk, qq, bb, vv, yy = k[b, t, h], q[b, t, h], beta[b, t, h], v[b, t, h], gy[b, t, h]
                    read_mu = mo if kind == "gq_uses_old_mu" else mn
                    out["gq"][b, t, h] = yy @ read_mu
                    g_mn = gm + np.outer(yy, qq)
                    g_In = gI if kind == "no_readout_term_on_I" else gI - g_mn * mn / In
                    keep = 1.0 if kind == "adjoint_not_decayed" else a
                    g_mo = g_mn * keep * Io / In
                    g_Io = g_mn * a * mo / In + g_In * a
                    ga = (g_mn * (Io / In) * mo).sum() + (g_In * Io).sum()
                    goma = (g_In * Ip).sum()
                    g_w = g_mn / In
                    gk = (g_w * (bb * vv)[:, None]).sum(0)
                    if kind != "gk_missing_importance_term":
                        gk = gk + (g_In * 2 * bb[:, None] * kk[None, :]).sum(0)
                    out["gk"][b, t, h] = gk
                    gw_sum = (g_w * kk[None, :]).sum(1)
                    out["gv"][b, t, h] = gw_sum if kind == "gv_missing_beta" else gw_sum * bb
                    gb = (g_In * (kk * kk)[None, :]).sum(1)
                    out["gbeta"][b, t, h] = gb if kind == "gbeta_missing_write" else gw_sum * vv + gb
                    sign = -1.0 if kind == "gdt_sign" else 1.0
                    out["gdt"][b, t, h] = sign * A[h] * a * (goma - ga)
                    out["gA"][h] += dt[b, t, h] * a * (goma - ga)
                    if kind != "gIp_missing_prior_term":
                        out["gIp"][h] += (g_In * oma).sum()
                    gm, gI = g_mo, g_Io
                out["gmu0"][b, h], out["gI0"][b, h] = gm, gI
        if default:
            out["gIp"] = out["gIp"] + out["gI0"].sum(axis=(0, 2, 3))
        return out
    return bwd


BWD_MUTANTS = ["gq_uses_old_mu", "no_readout_term_on_I", "adjoint_not_decayed",
               "gk_missing_importance_term", "gv_missing_beta", "gbeta_missing_write",
               "gdt_sign", "gIp_missing_prior_term"]


def _bwd_pins_pass(bwd):
    for state, final in ((True, True), (False, False)):
        err = _fd_pin_errors(bwd, seed=40 + state, state=state, final_grads=final, T=4)
        if not all(e < FD_TOL for e in err.values()):
            return False
    return True


def test_numpy_transcription_agrees_with_c_oracle():
    rng = np.random.default_rng(13)
    inp = _inputs(rng, 2, 11, 2, 3, 4)
    gy = rng.normal(size=(2, 11, 2, 4))
    gmuT, gIT = rng.normal(size=(2, 2, 4, 3)), rng.normal(size=(2, 2, 4, 3))
    a = oracle.bwd(**inp, gy=gy, gmuT=gmuT, gIT=gIT)
    b = _np_bwd("none")(**inp, gy=gy, gmuT=gmuT, gIT=gIT)
    for g in GRAD_OF.values():
        assert _normwise(a[g], b[g]) < 1e-12, g


def test_unmutated_bwd_copy_passes_pins():
    assert _bwd_pins_pass(_np_bwd("none"))


@pytest.mark.parametrize("kind", BWD_MUTANTS)
def test_bwd_pins_catch_planted_mistake(kind):
    assert not _bwd_pins_pass(_np_bwd(kind))
