"""Pins for the float64 oracle, independent of the oracle's own formulas.

Each test checks the oracle against something the pages or mathematics fix:
printed worked examples (``tests/golden``), closed forms, limits, invariants
and brute-force sums or posteriors on tiny inputs.  The last group plants
plausible mistakes in a copy of the recurrence and checks that the pins
catch every one of them.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _rand_inputs(rng, B, T, H, dk, dv, dt_scale=1.0, alpha_one=False):
    q = rng.standard_normal((B, T, H, dk))
    k = rng.standard_normal((B, T, H, dk))
    q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, H, dv))
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal((B, T, H, dv))))
    dt = np.zeros((B, T, H)) if alpha_one else dt_scale * np.log1p(np.exp(rng.standard_normal((B, T, H))))
    A = np.exp(np.linspace(0.0, math.log(4.0), H))
    Ip = np.linspace(0.5, 2.0, H)
    return dict(q=q, k=k, v=v, beta=beta, dt=dt, A=A, I_prior=Ip)


def _scalar_inputs(mu_prev, I_prev, v, k, beta, Ip, alpha):
    """One token, one head, d_k = d_v = 1, with alpha given through dt = -ln(alpha) / A."""
    A = 1.0
    dt = -math.log(alpha) / A
    one = lambda x: np.array(x, dtype=np.float64).reshape(1, 1, 1, 1)
    return dict(q=one(1.0), k=one(k), v=one(v), beta=one(beta),
                dt=np.array(dt).reshape(1, 1, 1), A=np.array([A]), I_prior=np.array([Ip]),
                mu0=one(mu_prev), I0=one(I_prev))


# ---------------------------------------------------------------------------
# printed worked examples
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("impl", ["c", "numpy"])
def test_scalar_teaching_example(impl):
    g = _golden("scalar_example.json")
    x = g["inputs"]
    tol = 0.5 * 10 ** (-g["printed_decimals"])
    fn = oracle.fwd if impl == "c" else oracle.fwd_numpy
    for row in g["rows"]:
        inp = _scalar_inputs(x["mu_prev"], row["I_prev"], x["v"], x["k"], x["beta"],
                             x["I_prior"], x["alpha"])
        y, mu, I = fn(**inp)
        assert abs(I.item() - row["I_new"]) <= 1e-12
        assert abs(mu.item() - row["mu_new"]) <= tol
        # with q = 1 the readout is the new mean itself
        assert abs(y.item() - mu.item()) <= 1e-15


def test_full_versus_diagonal_2d_example():
    g = _golden("full_vs_diagonal_2d.json")
    x = g["inputs"]
    k = np.array([x["k"]])
    v = np.array([[x["v"]]])
    beta = np.array([[x["beta"]]])
    P_prior = np.array(x["P_prior"])
    for alpha in (1.0, 0.7, 0.2):
        mu_full, P_full, _ = oracle.fwd_full_gaussian(k, v, beta, np.array([alpha]), P_prior,
                                                      mu0=np.array([x["mu_prev"]]))
        np.testing.assert_allclose(P_full[0], g["P_new"], atol=1e-14)
        np.testing.assert_allclose(mu_full[0], g["mu_full"], atol=1e-14)
        mu_diag, _, _ = oracle.fwd_full_gaussian(k, v, beta, np.array([alpha]), P_prior,
                                                 mu0=np.array([x["mu_prev"]]), diagonal=True)
        np.testing.assert_allclose(mu_diag[0], g["mu_diag"], atol=1e-14)
        # the Palimpsa recurrence (C oracle) gives the diagonal answer
        dt = -math.log(alpha) if alpha < 1 else 0.0
        _, mu, I = oracle.fwd(q=np.ones((1, 1, 1, 2)), k=k.reshape(1, 1, 1, 2),
                              v=v.reshape(1, 1, 1, 1), beta=beta.reshape(1, 1, 1, 1),
                              dt=np.array(dt).reshape(1, 1, 1), A=np.array([1.0]),
                              I_prior=np.array([1.0]))
        np.testing.assert_allclose(mu[0, 0, 0], g["mu_diag"], atol=1e-14)
        np.testing.assert_allclose(I[0, 0, 0], np.diag(g["P_new"]), atol=1e-14)


def test_correlated_keys_example():
    g = _golden("correlated_keys.json")
    keys = np.array(g["inputs"]["keys"])
    vals = np.array(g["inputs"]["values"])
    # full posterior with no forgetting and a vanishing ridge -> regression map
    lam = 1e-10
    mu, _, _ = oracle.fwd_full_gaussian(keys, vals[:, None], np.ones((2, 1)), np.ones(2),
                                        lam * np.eye(2))
    np.testing.assert_allclose(mu[0], g["regression_map_lambda_to_0"], atol=1e-6)
    np.testing.assert_allclose(keys @ mu[0], g["regression_reads"], atol=1e-6)
    # the additive natural-parameter state of the recurrence (alpha = 1, beta = 1)
    _, muT, IT = oracle.fwd(q=np.ones((1, 2, 1, 2)), k=keys.reshape(1, 2, 1, 2),
                            v=vals.reshape(1, 2, 1, 1), beta=np.ones((1, 2, 1, 1)),
                            dt=np.zeros((1, 2, 1)), A=np.array([1.0]), I_prior=np.array([0.3]))
    M = (IT * muT)[0, 0, 0]
    np.testing.assert_allclose(M, g["additive_map"], atol=1e-14)
    np.testing.assert_allclose(keys @ M, g["additive_reads"], atol=1e-14)


# ---------------------------------------------------------------------------
# closed forms and brute force
# ---------------------------------------------------------------------------

def _brute_force(inp, mu0=None, I0=None):
    """Explicit sums of discounted writes, written as double loops over tokens:
    M_t = (prod_{u<=t} a_u) M_0 + sum_{s<=t} (prod_{s<u<=t} a_u) (beta_s v_s) (x) k_s
    Ibar_t likewise with beta_s (x) k_s^2; I_t = I_prior + Ibar_t; y_t = (M_t / I_t) q_t.
    """
    q, k, v, beta, dt, A, Ip = (inp[n] for n in ("q", "k", "v", "beta", "dt", "A", "I_prior"))
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    y = np.zeros((B, T, H, dv))
    muT = np.zeros((B, H, dv, dk))
    IT = np.zeros((B, H, dv, dk))
    for b in range(B):
        for h in range(H):
            alpha = np.exp(-A[h] * dt[b, :, h])
            m0 = np.zeros((dv, dk)) if mu0 is None else mu0[b, h]
            i0 = np.full((dv, dk), Ip[h]) if I0 is None else I0[b, h]
            for t in range(T):
                M = np.prod(alpha[: t + 1]) * (i0 * m0)
                Ibar = np.prod(alpha[: t + 1]) * (i0 - Ip[h])
                for s in range(t + 1):
                    w = np.prod(alpha[s + 1: t + 1])
                    M = M + w * np.outer(beta[b, s, h] * v[b, s, h], k[b, s, h])
                    Ibar = Ibar + w * np.outer(beta[b, s, h], k[b, s, h] ** 2)
                I = Ip[h] + Ibar
                y[b, t, h] = (M / I) @ q[b, t, h]
            muT[b, h], IT[b, h] = M / I, I
    return y, muT, IT


@pytest.mark.parametrize("with_state", [False, True])
def test_brute_force_discounted_sums(with_state):
    rng = np.random.default_rng(11)
    inp = _rand_inputs(rng, B=2, T=9, H=2, dk=3, dv=2)
    mu0 = I0 = None
    if with_state:
        mu0 = rng.standard_normal((2, 2, 2, 3))
        I0 = inp["I_prior"][None, :, None, None] * (1 + rng.exponential(size=(2, 2, 2, 3)))
    y_ref, mu_ref, I_ref = _brute_force(inp, mu0, I0)
    for fn in (oracle.fwd, oracle.fwd_numpy):
        y, mu, I = fn(**inp, mu0=mu0, I0=I0)
        np.testing.assert_allclose(y, y_ref, rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(mu, mu_ref, rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(I, I_ref, rtol=1e-13, atol=1e-13)


def test_no_evidence_excess_importance_decays():
    """beta = 0: I_t - I_prior = alpha_t (I_{t-1} - I_prior) and M_t = alpha_t M_{t-1}."""
    rng = np.random.default_rng(3)
    inp = _rand_inputs(rng, B=1, T=20, H=2, dk=4, dv=3)
    inp["beta"] = np.zeros_like(inp["beta"])
    mu0 = rng.standard_normal((1, 2, 3, 4))
    I0 = inp["I_prior"][None, :, None, None] + rng.exponential(size=(1, 2, 3, 4))
    mu, I = mu0.copy(), I0.copy()
    for t in range(20):
        a = np.exp(-inp["A"] * inp["dt"][:, t])[:, :, None, None]
        y, mu_n, I_n = oracle.step(inp["q"][:, t], inp["k"][:, t], inp["v"][:, t],
                                   inp["beta"][:, t], inp["dt"][:, t], inp["A"],
                                   inp["I_prior"], mu, I)
        Ip = inp["I_prior"][None, :, None, None]
        np.testing.assert_allclose(I_n - Ip, a * (I - Ip), rtol=1e-14, atol=1e-15)
        np.testing.assert_allclose(I_n * mu_n, a * (I * mu), rtol=1e-13, atol=1e-15)
        mu, I = mu_n, I_n


def test_stationary_precision_closed_form():
    """Constant alpha, beta, k: I_t = I_prior + alpha^t (I_0 - I_prior)
    + beta k^2 (1 - alpha^t) / (1 - alpha), tending to I_prior + N beta k^2."""
    T, alpha, beta, kk, Ip, I_0 = 400, 0.97, 0.6, 0.8, 1.5, 1.5
    dt = -math.log(alpha)
    inp = dict(q=np.ones((1, T, 1, 1)), k=np.full((1, T, 1, 1), kk), v=np.ones((1, T, 1, 1)),
               beta=np.full((1, T, 1, 1), beta), dt=np.full((1, T, 1), dt),
               A=np.array([1.0]), I_prior=np.array([Ip]))
    for t in (1, 2, 10, 100, T):
        sub = {n: (x[:, :t] if n in ("q", "k", "v", "beta", "dt") else x) for n, x in inp.items()}
        _, _, I = oracle.fwd(**sub)
        a_t = math.exp(-dt * t)
        expect = Ip + a_t * (I_0 - Ip) + beta * kk ** 2 * (1 - a_t) / (1 - math.exp(-dt))
        assert abs(I.item() - expect) <= 1e-12 * expect
    N = 1.0 / (1.0 - alpha)
    assert abs(I.item() - (Ip + N * beta * kk ** 2)) < 1e-4


def test_geometric_evidence_weight_bounded_by_N():
    """beta k^2 = 1 from Ibar_0 = 0: Ibar_t = sum_{j<t} alpha^j = (1 - alpha^t)/(1 - alpha) <= N."""
    for alpha in (0.5, 0.9, 0.999):
        T = 200
        inp = dict(q=np.ones((1, T, 1, 1)), k=np.ones((1, T, 1, 1)), v=np.zeros((1, T, 1, 1)),
                   beta=np.ones((1, T, 1, 1)), dt=np.full((1, T, 1), -math.log(alpha)),
                   A=np.array([1.0]), I_prior=np.array([1.0]))
        _, _, I = oracle.fwd(**inp)
        weight = I.item() - 1.0
        assert abs(weight - (1 - alpha ** T) / (1 - alpha)) <= 1e-12 * weight
        assert weight <= 1.0 / (1.0 - alpha)


def test_alpha_one_is_pure_accumulation():
    """dt = 0: M_T = M_0 + sum_t (beta.v) (x) k, I_T = I_0 + sum_t beta (x) k^2, with an
    inclusive running readout (cumulative sums)."""
    rng = np.random.default_rng(5)
    inp = _rand_inputs(rng, B=2, T=30, H=3, dk=5, dv=4, alpha_one=True)
    y, mu, I = oracle.fwd(**inp)
    bv = inp["beta"] * inp["v"]
    M_cum = np.cumsum(np.einsum("bthi,bthj->bthij", bv, inp["k"]), axis=1)
    I_cum = inp["I_prior"][None, None, :, None, None] + np.cumsum(
        np.einsum("bthi,bthj->bthij", inp["beta"], inp["k"] ** 2), axis=1)
    y_ref = np.einsum("bthij,bthj->bthi", M_cum / I_cum, inp["q"])
    np.testing.assert_allclose(y, y_ref, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(I, I_cum[:, -1], rtol=1e-13)
    np.testing.assert_allclose(I * mu, M_cum[:, -1], rtol=1e-11, atol=1e-12)


def test_natural_parameter_scans_agree():
    rng = np.random.default_rng(7)
    inp = _rand_inputs(rng, B=2, T=40, H=2, dk=6, dv=5)
    mu0 = rng.standard_normal((2, 2, 5, 6))
    I0 = inp["I_prior"][None, :, None, None] * (1 + rng.exponential(size=(2, 2, 5, 6)))
    a = oracle.fwd(**inp, mu0=mu0, I0=I0)
    b = oracle.fwd_natural(**inp, mu0=mu0, I0=I0)
    for x, z in zip(a, b):
        np.testing.assert_allclose(x, z, rtol=1e-11, atol=1e-12)


# ---------------------------------------------------------------------------
# the full Gaussian posterior on tiny d_k
# ---------------------------------------------------------------------------

def test_full_gaussian_alpha_one_is_weighted_ridge():
    """No forgetting: the full posterior mean of each value row solves the
    weighted normal equations (P_prior + sum_t beta_t k k^T) m = sum_t beta_t v_t k."""
    rng = np.random.default_rng(9)
    T, dk, dv = 12, 3, 2
    k = rng.standard_normal((T, dk))
    v = rng.standard_normal((T, dv))
    beta = rng.uniform(0.1, 1.0, (T, dv))
    P_prior = 0.7 * np.eye(dk)
    mu, P, _ = oracle.fwd_full_gaussian(k, v, beta, np.ones(T), P_prior)
    for i in range(dv):
        G = P_prior + (beta[:, i, None, None] * k[:, :, None] * k[:, None, :]).sum(0)
        r = (beta[:, i, None] * v[:, i, None] * k).sum(0)
        np.testing.assert_allclose(P[i], G, rtol=1e-13)
        np.testing.assert_allclose(mu[i], np.linalg.solve(G, r), rtol=1e-10)


def test_axis_aligned_keys_full_equals_diagonal():
    """One-hot keys leave every precision diagonal, so the full posterior and
    the recurrence coincide."""
    rng = np.random.default_rng(13)
    T, dk, dv = 25, 4, 3
    idx = rng.integers(0, dk, T)
    k = np.eye(dk)[idx] * rng.uniform(0.5, 1.5, (T, 1))
    v = rng.standard_normal((T, dv))
    beta = rng.uniform(0.1, 1.0, (T, dv))
    dt = np.log1p(np.exp(rng.standard_normal(T)))
    alpha = np.exp(-dt)
    Ip = 1.3
    mu_full, P_full, _ = oracle.fwd_full_gaussian(k, v, beta, alpha, Ip * np.eye(dk))
    _, mu, I = oracle.fwd(q=np.ones((1, T, 1, dk)), k=k[None, :, None], v=v[None, :, None],
                          beta=beta[None, :, None], dt=dt[None, :, None],
                          A=np.array([1.0]), I_prior=np.array([Ip]))
    np.testing.assert_allclose(mu[0, 0], mu_full, rtol=1e-12, atol=1e-14)
    for i in range(dv):
        np.testing.assert_allclose(np.diag(P_full[i]), I[0, 0, i], rtol=1e-13)
        assert np.abs(P_full[i] - np.diag(np.diag(P_full[i]))).max() == 0.0


def test_diagonal_gaussian_equals_recurrence():
    """Keeping only diag(P) in the coupled Gaussian solution at every token is Eq. (5)."""
    rng = np.random.default_rng(17)
    inp = _rand_inputs(rng, B=1, T=30, H=1, dk=3, dv=2)
    alpha = np.exp(-inp["A"][0] * inp["dt"][0, :, 0])
    Ip = inp["I_prior"][0]
    mu_d, P_d, mus = oracle.fwd_full_gaussian(inp["k"][0, :, 0], inp["v"][0, :, 0],
                                              inp["beta"][0, :, 0], alpha, Ip * np.eye(3),
                                              diagonal=True)
    y, mu, I = oracle.fwd(**inp)
    np.testing.assert_allclose(mu[0, 0], mu_d, rtol=1e-12)
    np.testing.assert_allclose(I[0, 0], np.stack([np.diag(p) for p in P_d]), rtol=1e-13)
    np.testing.assert_allclose(y[0, :, 0], np.einsum("tij,tj->ti", mus, inp["q"][0, :, 0]),
                               rtol=1e-11, atol=1e-13)
    # and it differs from the full posterior once keys are correlated
    mu_f, _, _ = oracle.fwd_full_gaussian(inp["k"][0, :, 0], inp["v"][0, :, 0],
                                          inp["beta"][0, :, 0], alpha, Ip * np.eye(3))
    assert np.abs(mu_f - mu_d).max() > 1e-3


# ---------------------------------------------------------------------------
# limits and invariants
# ---------------------------------------------------------------------------

def test_mamba2_limit():
    """With the write v* = beta.v held fixed and beta -> 0, the excess precision
    vanishes and y approaches the frozen-importance recurrence linearly in beta."""
    rng = np.random.default_rng(19)
    base = _rand_inputs(rng, B=1, T=64, H=2, dk=8, dv=6)
    vstar = base["beta"] * base["v"]
    errs = []
    for eps in (1e-2, 1e-4, 1e-6):
        inp = dict(base)
        inp["beta"] = eps * base["beta"]
        inp["v"] = vstar / inp["beta"]
        y, _, I = oracle.fwd(**inp)
        y_lim, _ = oracle.fwd_mamba2_limit(**inp)
        excess = (I / inp["I_prior"][None, :, None, None] - 1).max()
        assert excess < 100 * eps
        errs.append(np.abs(y - y_lim).max() / np.abs(y_lim).max())
    assert errs[0] > 1e-4                      # the limit is not exact at finite beta
    assert errs[1] < 2e-2 * errs[0] and errs[2] < 2e-2 * errs[1]
    assert errs[2] < 1e-5


def test_importance_invariants():
    """I_t >= I_prior whenever I_0 >= I_prior, and
    Ibar_t <= max(Ibar_0, max_s beta_s k_s^2 / (1 - alpha_s)) for alpha < 1."""
    rng = np.random.default_rng(23)
    inp = _rand_inputs(rng, B=2, T=60, H=2, dk=4, dv=3)
    Ip = inp["I_prior"][None, :, None, None]
    mu = rng.standard_normal((2, 2, 3, 4))
    I = Ip * (1 + rng.exponential(size=(2, 2, 3, 4)))
    alpha = np.exp(-inp["A"][None, None, :] * inp["dt"])        # [B, T, H]
    ratio = inp["beta"][..., :, None] * inp["k"][..., None, :] ** 2 / (1 - alpha)[..., None, None]
    bound = np.maximum(I - Ip, ratio.max(axis=1))
    for t in range(60):
        _, mu, I = oracle.step(inp["q"][:, t], inp["k"][:, t], inp["v"][:, t],
                               inp["beta"][:, t], inp["dt"][:, t], inp["A"],
                               inp["I_prior"], mu, I)
        assert (I >= Ip).all()
        assert (I - Ip <= bound * (1 + 1e-12)).all()
        assert np.isfinite(mu).all()


def test_step_composes_to_fwd():
    rng = np.random.default_rng(29)
    inp = _rand_inputs(rng, B=2, T=17, H=3, dk=4, dv=4)
    y, mu_f, I_f = oracle.fwd(**inp)
    Ip = inp["I_prior"]
    mu = np.zeros((2, 3, 4, 4))
    I = np.broadcast_to(Ip[None, :, None, None], mu.shape).copy()
    for t in range(17):
        yt, mu, I = oracle.step(inp["q"][:, t], inp["k"][:, t], inp["v"][:, t],
                                inp["beta"][:, t], inp["dt"][:, t], inp["A"], Ip, mu, I)
        assert np.array_equal(yt, y[:, t])
    assert np.array_equal(mu, mu_f) and np.array_equal(I, I_f)


def test_c_and_numpy_transcriptions_agree_on_tiny_workload():
    import workloads
    w = workloads.WORKLOADS[0]
    inp = workloads.make_inputs(w, T=64)
    a = oracle.fwd(**inp)
    b = oracle.fwd_numpy(**inp)
    for x, z in zip(a, b):
        np.testing.assert_allclose(x, z, rtol=1e-12, atol=1e-13)


def test_select_heads_matches_full_run():
    import workloads
    w = workloads.WORKLOADS[0].with_(B=2, H=3)
    inp = workloads.make_inputs(w, T=40)
    mu0, I0 = workloads.random_state(2, 3, 32, 32, inp["I_prior"], seed=1)
    inp["mu0"], inp["I0"] = mu0, I0
    y, mu, I = oracle.fwd(**inp)
    heads = [(1, 2), (0, 0), (1, 0)]
    sub = oracle.select_heads(inp, heads)
    ys, mus, Is = oracle.fwd(**sub)
    for s, (b, h) in enumerate(heads):
        assert np.array_equal(ys[0, :, s], y[b, :, h])
        assert np.array_equal(mus[0, s], mu[b, h]) and np.array_equal(Is[0, s], I[b, h])


def test_empty_sequence_returns_initial_state():
    rng = np.random.default_rng(31)
    inp = _rand_inputs(rng, B=1, T=0, H=2, dk=3, dv=3)
    mu0 = rng.standard_normal((1, 2, 3, 3))
    I0 = 1 + rng.exponential(size=(1, 2, 3, 3))
    y, mu, I = oracle.fwd(**inp, mu0=mu0, I0=I0)
    assert y.shape == (1, 0, 2, 3)
    assert np.array_equal(mu, mu0) and np.array_equal(I, I0)


# ---------------------------------------------------------------------------
# planted mistakes: every mutant of the recurrence must fail some pin
# ---------------------------------------------------------------------------

def _mutant_fwd(kind):
    def fwd(q, k, v, beta, dt, A, I_prior, mu0=None, I0=None):
        B, T, H, dk = q.shape
        dv = v.shape[-1]
        mu = np.zeros((B, H, dv, dk)) if mu0 is None else np.array(mu0, dtype=float)
        I = np.broadcast_to(np.asarray(I_prior)[None, :, None, None], (B, H, dv, dk)).copy() \
            if I0 is None else np.array(I0, dtype=float)
        y = np.zeros((B, T, H, dv))
        for b in range(B):
            for h in range(H):
                m, P = mu[b, h], I[b, h]
                for t in range(T):
                    a = math.exp(-A[h] * dt[b, t, h])
                    kk = k[b, t, h]
                    prior = 0.0 if kind == "no_prior_restore" else (1 - a) * I_prior[h]
                    k2 = kk if kind == "k_not_squared" else kk * kk
                    P_new = a * P + prior + np.outer(beta[b, t, h], k2)
                    ratio = (P_new / P_new) if kind == "ratio_uses_new" else (P / P_new)
                    keep = 1.0 if kind == "no_alpha_on_mean" else a
                    bv = v[b, t, h] if kind == "beta_dropped_in_write" else beta[b, t, h] * v[b, t, h]
                    m_new = keep * ratio * m + np.outer(bv, kk) / P_new
                    if kind == "readout_exclusive":
                        y[b, t, h] = m @ q[b, t, h]
                    elif kind == "readout_transposed":
                        y[b, t, h] = m_new.T @ q[b, t, h][: dv]
                    else:
                        y[b, t, h] = m_new @ q[b, t, h]
                    m, P = m_new, P_new
                mu[b, h], I[b, h] = m, P
        return y, mu, I
    return fwd


MUTANTS = ["no_prior_restore", "k_not_squared", "ratio_uses_new", "no_alpha_on_mean",
           "beta_dropped_in_write", "readout_exclusive", "readout_transposed"]


def _pins_pass(fn):
    """Re-run the example, brute-force and closed-form pins on ``fn``."""
    try:
        g = _golden("scalar_example.json")
        x = g["inputs"]
        for row in g["rows"]:
            inp = _scalar_inputs(x["mu_prev"], row["I_prev"], x["v"], x["k"], x["beta"],
                                 x["I_prior"], x["alpha"])
            _, mu, I = fn(**inp)
            if abs(I.item() - row["I_new"]) > 1e-12 or abs(mu.item() - row["mu_new"]) > 5e-5:
                return False
        rng = np.random.default_rng(11)
        inp = _rand_inputs(rng, B=1, T=7, H=2, dk=3, dv=3)
        ref = _brute_force(inp)
        got = fn(**inp)
        return all(np.allclose(a, b, rtol=1e-10, atol=1e-12) for a, b in zip(got, ref))
    except Exception:
        return False


def test_unmutated_copy_passes_pins():
    assert _pins_pass(_mutant_fwd("none"))


@pytest.mark.parametrize("kind", MUTANTS)
def test_pins_catch_planted_mistake(kind):
    assert not _pins_pass(_mutant_fwd(kind))


# ---------------------------------------------------------------------------
# options: a prior per state entry, and v* = beta . v as the write input
# ---------------------------------------------------------------------------

def _per_entry_prior(rng, H, dv, dk):
    return rng.uniform(0.3, 2.0, size=(H, dv, dk))


def test_per_entry_prior_c_and_numpy_agree():
    rng = np.random.default_rng(31)
    inp = _rand_inputs(rng, B=2, T=9, H=2, dk=3, dv=4)
    inp["I_prior"] = _per_entry_prior(rng, 2, 4, 3)
    for state in (False, True):
        if state:
            inp["mu0"] = rng.normal(size=(2, 2, 4, 3))
            inp["I0"] = rng.uniform(0.5, 2.0, size=(2, 2, 4, 3))
        a = oracle.fwd(**inp)
        b = oracle.fwd_numpy(**inp)
        for x, y in zip(a, b):
            np.testing.assert_allclose(x, y, rtol=1e-12, atol=1e-14)


def test_per_entry_prior_equal_to_the_head_prior_is_the_scalar_case():
    rng = np.random.default_rng(32)
    inp = _rand_inputs(rng, B=1, T=6, H=3, dk=4, dv=2)
    full = dict(inp, I_prior=np.broadcast_to(np.asarray(inp["I_prior"])[:, None, None], (3, 2, 4)).copy())
    for x, y in zip(oracle.fwd(**inp), oracle.fwd(**full)):
        np.testing.assert_array_equal(x, y)


def test_per_entry_prior_no_evidence_closed_form():
    """beta = 0: each entry relaxes to its own prior, I_T - Ip = (prod alpha)(I_0 - Ip),
    and the mean only decays, M_T = (prod alpha) M_0, so mu_T = (prod alpha) I_0 mu_0 / I_T."""
    rng = np.random.default_rng(33)
    B, T, H, dk, dv = 2, 7, 2, 3, 2
    inp = _rand_inputs(rng, B=B, T=T, H=H, dk=dk, dv=dv)
    inp["beta"] = np.zeros_like(inp["beta"])
    Ip = _per_entry_prior(rng, H, dv, dk)
    mu0 = rng.normal(size=(B, H, dv, dk))
    I0 = rng.uniform(0.5, 3.0, size=(B, H, dv, dk))
    _, mu, I = oracle.fwd(**dict(inp, I_prior=Ip, mu0=mu0, I0=I0))
    P = np.exp(-np.asarray(inp["A"])[None, :] * np.asarray(inp["dt"]).sum(axis=1))   # [B, H]
    I_ref = Ip[None] + P[:, :, None, None] * (I0 - Ip[None])
    np.testing.assert_allclose(I, I_ref, rtol=1e-12)
    np.testing.assert_allclose(mu, P[:, :, None, None] * I0 * mu0 / I_ref, rtol=1e-11)


def test_vstar_input_is_the_product_it_replaces():
    rng = np.random.default_rng(34)
    inp = _rand_inputs(rng, B=2, T=8, H=2, dk=3, dv=3)
    vstar = np.asarray(inp["beta"]) * np.asarray(inp["v"])
    a = oracle.fwd(**inp)
    b = oracle.fwd(**dict(inp, v=vstar), vstar=True)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)
    c = oracle.fwd_numpy(**dict(inp, v=vstar), vstar=True)
    for x, y in zip(a, c):
        np.testing.assert_allclose(x, y, rtol=1e-12, atol=1e-14)


# ---------------------------------------------------------------------------
# block-diagonal precision (limited cross-key correlations)
# ---------------------------------------------------------------------------

def test_blockdiag_block_one_is_the_recurrence():
    rng = np.random.default_rng(41)
    inp = _rand_inputs(rng, B=2, T=9, H=2, dk=4, dv=3)
    y, mu, P = oracle.fwd_blockdiag(**inp, block=1)
    y2, mu2, I2 = oracle.fwd(**inp)
    np.testing.assert_allclose(y, y2, rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(mu, mu2, rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(P[..., 0, 0], I2, rtol=1e-12)


def test_blockdiag_full_block_is_the_full_gaussian():
    rng = np.random.default_rng(42)
    inp = _rand_inputs(rng, B=1, T=7, H=1, dk=4, dv=2)
    y, mu, P = oracle.fwd_blockdiag(**inp, block=4)
    alpha = np.exp(-inp["A"][0] * inp["dt"][0, :, 0])
    mu_f, P_f, mus = oracle.fwd_full_gaussian(inp["k"][0, :, 0], inp["v"][0, :, 0], inp["beta"][0, :, 0],
                                              alpha, inp["I_prior"][0] * np.eye(4))
    np.testing.assert_allclose(mu[0, 0], mu_f, rtol=1e-10, atol=1e-13)
    np.testing.assert_allclose(P[0, 0, :, 0], P_f, rtol=1e-12)
    np.testing.assert_allclose(y[0, :, 0], np.einsum("tij,tj->ti", mus, inp["q"][0, :, 0]), rtol=1e-10, atol=1e-13)


def test_blockdiag_is_exact_when_every_key_lives_in_one_block():
    """Keys supported on one 2-block per token keep the full precision block-
    diagonal, so the block model equals the full update exactly."""
    rng = np.random.default_rng(43)
    inp = _rand_inputs(rng, B=1, T=10, H=1, dk=4, dv=2)
    kk = np.zeros_like(inp["k"])
    for t in range(10):
        blk = t % 2
        kk[0, t, 0, 2 * blk:2 * blk + 2] = rng.standard_normal(2)
    inp["k"] = kk
    _, mu, _ = oracle.fwd_blockdiag(**inp, block=2)
    alpha = np.exp(-inp["A"][0] * inp["dt"][0, :, 0])
    mu_f, _, _ = oracle.fwd_full_gaussian(kk[0, :, 0], inp["v"][0, :, 0], inp["beta"][0, :, 0], alpha,
                                          inp["I_prior"][0] * np.eye(4))
    np.testing.assert_allclose(mu[0, 0], mu_f, rtol=1e-10, atol=1e-13)
    _, mu_d, _ = oracle.fwd_blockdiag(**inp, block=1)
    assert np.abs(mu_d[0, 0] - mu_f).max() > 1e-3       # the diagonal model is not exact here


def test_blockdiag_axis_aligned_keys_agree_for_every_block_size():
    rng = np.random.default_rng(44)
    inp = _rand_inputs(rng, B=1, T=8, H=2, dk=4, dv=2)
    kk = np.zeros_like(inp["k"])
    idx = rng.integers(0, 4, size=(8, 2))
    for t in range(8):
        for h in range(2):
            kk[0, t, h, idx[t, h]] = rng.standard_normal()
    inp["k"] = kk
    ref = oracle.fwd(**inp)
    for bs in (1, 2, 4):
        y, mu, _ = oracle.fwd_blockdiag(**inp, block=bs)
        np.testing.assert_allclose(y, ref[0], rtol=1e-11, atol=1e-13)
        np.testing.assert_allclose(mu, ref[1], rtol=1e-11, atol=1e-13)


def test_blockdiag_teaching_example_two_by_two():
    """The backup frame's 2-D example: one key (1, 1), v = beta = 1, prior mean 0,
    identity prior precision (alpha = 1): the 2-block keeps the correlation and
    gives the full mean (1/3, 1/3); the diagonal model gives (1/2, 1/2)."""
    g = _golden("full_vs_diagonal_2d.json")
    x = g["inputs"]
    B = T = H = 1
    inp = dict(q=np.zeros((1, 1, 1, 2)), k=np.array(x["k"], float).reshape(1, 1, 1, 2),
               v=np.array([[[[x["v"]]]]], float), beta=np.array([[[[x["beta"]]]]], float),
               dt=np.zeros((1, 1, 1)), A=np.ones(1), I_prior=np.ones(1))
    _, mu2, P2 = oracle.fwd_blockdiag(**inp, block=2)
    _, mu1, _ = oracle.fwd_blockdiag(**inp, block=1)
    np.testing.assert_allclose(mu2[0, 0, 0], g["mu_full"], rtol=1e-12)
    np.testing.assert_allclose(mu1[0, 0, 0], g["mu_diag"], rtol=1e-12)
    np.testing.assert_allclose(P2[0, 0, 0, 0], g["P_new"], rtol=1e-12)
