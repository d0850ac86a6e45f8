"""Float64 CPU oracle for the Palimpsa dual-state recurrence.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the bench's
CPU-baseline leg may import this package; the product path
(``bayesian_metaplastic_memory_amd``) never does, and the two share no code.

Contents
--------
``fwd`` / ``step``
    Thin ctypes wrappers over ``palimpsa_oracle.c``: the sequential Eq. (5)
    recurrence of "Learning to Remember, Learn, and Forget in Attention-Based
    Models" (slides, frame "Palimpsa updates content and importance
    together") with the posterior-mean readout ``y_t = mu_t q_t``.
``fwd_numpy``
    The same definition written with numpy, vectorised over the state entries
    of one token; a second, independent transcription for small cases.
``fwd_natural``
    The natural-parameter affine scans ``M = I . mu``, ``Ibar = I - I_prior``
    (slides, frame "Natural parameters expose two affine scans", App. A.12).
``fwd_full_gaussian``
    The full-precision Gaussian update per value row (slides, backup frame
    "dropping precision correlations changes the mean", App. A.3-A.5), with
    an option that keeps only the diagonal of the precision at every token.
``bwd``
    The reverse-mode derivative of ``fwd`` (C oracle), for the training path.
``fwd_blockdiag`` / ``bwd_blockdiag``
    The Gaussian update with the precision kept block-diagonal along the key
    axis (limited cross-key correlations); block 1 is Eq. (5), block dk the
    full update; and its reverse-mode derivative.
``fwd_mamba2_limit`` / ``bwd_mamba2_limit``
    The frozen-importance recurrence of the Mamba2 limit (slides, frame "The
    Mamba2 limit enables a gradual model upgrade", Secs. 2.3-2.4), and its
    reverse-mode derivative.

All arrays use the library's layouts: q, k ``[B, T, H, dk]``; v, beta
``[B, T, H, dv]``; dt ``[B, T, H]``; A, I_prior ``[H]``; state
``[B, H, dv, dk]``; y ``[B, T, H, dv]``.

Every function here is pinned (``tests/test_oracle_pins.py`` and the
``test_oracle_*bwd_pins.py`` files) against the pages' worked examples,
closed forms, limits, a brute-force posterior and finite differences.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "palimpsa_oracle.c")
_LIB = os.path.join(_HERE, "libpalimpsa_oracle.so")
_lock = threading.Lock()
_handle = None

# -O2 without fast-math and without contraction: every product and sum is a
# separately rounded IEEE float64 operation.
GCC_FLAGS = ["-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
             "-shared", "-fPIC", "-std=c11"]


def build(force: bool = False) -> str:
    """Compile the C oracle with gcc (idempotent unless ``force``)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", *GCC_FLAGS, _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _lib():
    global _handle
    with _lock:
        if _handle is None:
            build()
            lib = ctypes.CDLL(_LIB)
            dp = ctypes.POINTER(ctypes.c_double)
            i = ctypes.c_int
            lib.oracle_fwd.argtypes = [i, i, i, i, i] + [dp] * 10 + [i, i]
            lib.oracle_fwd.restype = None
            lib.oracle_step.argtypes = [i, i, i, i] + [dp] * 10 + [i, i]
            lib.oracle_step.restype = None
            lib.oracle_bwd.argtypes = [i, i, i, i, i] + [dp] * 21 + [i, i]
            lib.oracle_bwd.restype = None
            lib.oracle_max_threads.argtypes = []
            lib.oracle_max_threads.restype = i
            _handle = lib
    return _handle


def max_threads() -> int:
    """Threads the OpenMP runtime would use by default."""
    return int(_lib().oracle_max_threads())


def _f64(x) -> np.ndarray:
    """Exact upcast to contiguous float64 (bf16 and fp32 values are exact)."""
    if hasattr(x, "detach"):  # a torch tensor; bf16 needs a float32 hop
        x = x.detach().cpu()
        if str(x.dtype) == "torch.bfloat16":
            x = x.float()
        x = x.numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


VSTAR, PRIOR_PER_ENTRY = 1, 2


def _opts(Ip, H, dv, dk, vstar):
    """Option bits of the C oracle: the prior is per head ``[H]`` or per
    state entry ``[H, dv, dk]``; ``vstar`` means v holds beta . v."""
    if Ip.shape == (H,):
        o = 0
    elif Ip.shape == (H, dv, dk):
        o = PRIOR_PER_ENTRY
    else:
        raise ValueError("I_prior must be [H] or [H, dv, dk]")
    return o | (VSTAR if vstar else 0)


def _prior_full(Ip, H, dv, dk):
    """The prior as [H, dv, dk] (a per-head prior broadcast to every entry)."""
    return Ip if Ip.shape == (H, dv, dk) else np.broadcast_to(Ip[:, None, None], (H, dv, dk))


def _init_state(B, H, dv, dk, Ip, mu0, I0):
    if (mu0 is None) != (I0 is None):
        raise ValueError("give both mu0 and I0, or neither")
    if mu0 is None:
        mu = np.zeros((B, H, dv, dk))
        I = np.broadcast_to(_prior_full(Ip, H, dv, dk)[None], (B, H, dv, dk)).copy()
    else:
        mu, I = _f64(mu0).copy(), _f64(I0).copy()
        if mu.shape != (B, H, dv, dk) or I.shape != (B, H, dv, dk):
            raise ValueError("state must be [B, H, dv, dk]")
    return mu, I


def fwd(q, k, v, beta, dt, A, I_prior, mu0=None, I0=None, nthreads: int = 0, vstar: bool = False):
    """Sequential float64 Eq. (5) over the whole sequence (C oracle).

    Returns ``(y [B,T,H,dv], muT [B,H,dv,dk], IT [B,H,dv,dk])`` as float64.
    ``mu0 = I0 = None`` means ``mu0 = 0`` and ``I0 = I_prior``.  ``I_prior``
    is ``[H]`` or ``[H, dv, dk]`` (one prior per state entry); with ``vstar``
    the ``v`` argument holds ``v* = beta . v``.
    """
    q, k, v, beta, dt = (_f64(x) for x in (q, k, v, beta, dt))
    A, Ip = _f64(A), _f64(I_prior)
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    if k.shape != q.shape or v.shape != (B, T, H, dv) or beta.shape != v.shape \
            or dt.shape != (B, T, H) or A.shape != (H,):
        raise ValueError("inconsistent shapes")
    opts = _opts(Ip, H, dv, dk, vstar)
    mu, I = _init_state(B, H, dv, dk, Ip, mu0, I0)
    y = np.zeros((B, T, H, dv))
    _lib().oracle_fwd(B, T, H, dk, dv, _ptr(q), _ptr(k), _ptr(v), _ptr(beta),
                      _ptr(dt), _ptr(A), _ptr(Ip), _ptr(mu), _ptr(I), _ptr(y),
                      opts, int(nthreads))
    return y, mu, I


def step(q, k, v, beta, dt, A, I_prior, mu, I, nthreads: int = 0, vstar: bool = False):
    """One decode token (C oracle).  q, k ``[B,H,dk]``; v, beta ``[B,H,dv]``;
    dt ``[B,H]``.  Returns ``(y [B,H,dv], mu', I')`` without touching inputs."""
    q, k, v, beta, dt = (_f64(x) for x in (q, k, v, beta, dt))
    A, Ip = _f64(A), _f64(I_prior)
    B, H, dk = q.shape
    dv = v.shape[-1]
    mu, I = _f64(mu).copy(), _f64(I).copy()
    if mu.shape != (B, H, dv, dk) or I.shape != mu.shape or dt.shape != (B, H):
        raise ValueError("inconsistent shapes")
    opts = _opts(Ip, H, dv, dk, vstar)
    y = np.zeros((B, H, dv))
    _lib().oracle_step(B, H, dk, dv, _ptr(q), _ptr(k), _ptr(v), _ptr(beta),
                       _ptr(dt), _ptr(A), _ptr(Ip), _ptr(mu), _ptr(I), _ptr(y),
                       opts, int(nthreads))
    return y, mu, I


def bwd(q, k, v, beta, dt, A, I_prior, gy, mu0=None, I0=None, gmuT=None, gIT=None,
        nthreads: int = 0, vstar: bool = False) -> dict:
    """Reverse-mode derivative of ``fwd`` (C oracle) for the scalar
    ``L = sum(gy * y) + sum(gmuT * muT) + sum(gIT * IT)``.

    Returns a dict of float64 arrays: ``gq, gk [B,T,H,dk]``, ``gv, gbeta
    [B,T,H,dv]``, ``gdt [B,T,H]``, ``gA, gIp [H]`` (summed over the batch),
    ``gmu0, gI0 [B,H,dv,dk]``.  With ``mu0 = I0 = None`` the start state is
    ``mu0 = 0, I0 = I_prior``; it then depends on ``I_prior``, so ``gIp``
    also collects the sum of ``gI0`` over the head's entries.  With a
    per-entry prior ``[H, dv, dk]``, ``gIp`` has that shape (and collects
    ``gI0`` entry by entry); with ``vstar``, ``gv`` is the gradient with
    respect to ``v* = beta . v`` and ``gbeta`` only has the importance term.
    """
    q, k, v, beta, dt, gy = (_f64(x) for x in (q, k, v, beta, dt, gy))
    A, Ip = _f64(A), _f64(I_prior)
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    if k.shape != q.shape or v.shape != (B, T, H, dv) or beta.shape != v.shape \
            or dt.shape != (B, T, H) or gy.shape != v.shape or A.shape != (H,):
        raise ValueError("inconsistent shapes")
    opts = _opts(Ip, H, dv, dk, vstar)
    per_entry = bool(opts & PRIOR_PER_ENTRY)
    default_state = mu0 is None
    mu, I = _init_state(B, H, dv, dk, Ip, mu0, I0)
    gmuT = None if gmuT is None else _f64(gmuT)
    gIT = None if gIT is None else _f64(gIT)
    for x in (gmuT, gIT):
        if x is not None and x.shape != (B, H, dv, dk):
            raise ValueError("final-state gradients must be [B, H, dv, dk]")
    out = {"gq": np.zeros((B, T, H, dk)), "gk": np.zeros((B, T, H, dk)),
           "gv": np.zeros((B, T, H, dv)), "gbeta": np.zeros((B, T, H, dv)),
           "gdt": np.zeros((B, T, H)), "gmu0": np.zeros((B, H, dv, dk)),
           "gI0": np.zeros((B, H, dv, dk))}
    gA_bh = np.zeros((B, H))
    gIp_bh = np.zeros((B, H, dv, dk)) if per_entry else np.zeros((B, H))
    null = ctypes.POINTER(ctypes.c_double)()
    _lib().oracle_bwd(B, T, H, dk, dv, _ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(dt),
                      _ptr(A), _ptr(Ip), _ptr(mu), _ptr(I), _ptr(gy),
                      null if gmuT is None else _ptr(gmuT), null if gIT is None else _ptr(gIT),
                      _ptr(out["gq"]), _ptr(out["gk"]), _ptr(out["gv"]), _ptr(out["gbeta"]),
                      _ptr(out["gdt"]), _ptr(gA_bh), _ptr(gIp_bh), _ptr(out["gmu0"]),
                      _ptr(out["gI0"]), opts, int(nthreads))
    out["gA"] = gA_bh.sum(axis=0)
    out["gIp"] = gIp_bh.sum(axis=0)
    if default_state:
        out["gIp"] = out["gIp"] + (out["gI0"].sum(axis=0) if per_entry else out["gI0"].sum(axis=(0, 2, 3)))
    return out


# ---------------------------------------------------------------------------
# numpy transcriptions (small cases and pins)
# ---------------------------------------------------------------------------

def _gate(A_h, dt):
    """alpha = exp(-A dt) and 1 - alpha = -expm1(-A dt) (Eq. (9) gate)."""
    return np.exp(-A_h * dt), -np.expm1(-A_h * dt)


def fwd_numpy(q, k, v, beta, dt, A, I_prior, mu0=None, I0=None, vstar: bool = False):
    """Eq. (5) token by token, vectorised over the (i, j) state entries.
    ``I_prior`` is ``[H]`` or ``[H, dv, dk]``; ``vstar`` as in ``fwd``."""
    q, k, v, beta, dt = (_f64(x) for x in (q, k, v, beta, dt))
    A, Ip = _f64(A), _f64(I_prior)
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    mu, I = _init_state(B, H, dv, dk, Ip, mu0, I0)
    prior = _prior_full(Ip, H, dv, dk)
    y = np.zeros((B, T, H, dv))
    for b in range(B):
        for h in range(H):
            m, P = mu[b, h], I[b, h]
            for t in range(T):
                a, oma = _gate(A[h], dt[b, t, h])
                kk = k[b, t, h]
                P_new = a * P + oma * prior[h] + np.outer(beta[b, t, h], kk * kk)
                wv = v[b, t, h] if vstar else beta[b, t, h] * v[b, t, h]
                m = a * (P / P_new) * m + np.outer(wv, kk) / P_new
                P = P_new
                y[b, t, h] = m @ q[b, t, h]
            mu[b, h], I[b, h] = m, P
    return y, mu, I


def fwd_natural(q, k, v, beta, dt, A, I_prior, mu0=None, I0=None):
    """Natural-parameter form: M_t = alpha M_{t-1} + (beta.v) (x) k,
    Ibar_t = alpha Ibar_{t-1} + beta (x) k^2, y_t = (M_t / (I_prior + Ibar_t)) q_t.
    Returns ``(y, muT, IT)`` like ``fwd``."""
    q, k, v, beta, dt = (_f64(x) for x in (q, k, v, beta, dt))
    A, Ip = _f64(A), _f64(I_prior)
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    mu, I = _init_state(B, H, dv, dk, Ip, mu0, I0)
    y = np.zeros((B, T, H, dv))
    for b in range(B):
        for h in range(H):
            M = I[b, h] * mu[b, h]
            Ibar = I[b, h] - Ip[h]
            for t in range(T):
                a, _ = _gate(A[h], dt[b, t, h])
                kk = k[b, t, h]
                M = a * M + np.outer(beta[b, t, h] * v[b, t, h], kk)
                Ibar = a * Ibar + np.outer(beta[b, t, h], kk * kk)
                y[b, t, h] = (M / (Ip[h] + Ibar)) @ q[b, t, h]
            I[b, h] = Ip[h] + Ibar
            mu[b, h] = M / I[b, h]
    return y, mu, I


def fwd_full_gaussian(k, v, beta, alpha, P_prior, mu0=None, P0=None,
                      diagonal: bool = False):
    """Full-precision Gaussian filter for ONE head, value rows independent.

    For each value row i (App. A.3-A.5):
        P_t = alpha_t P_{t-1} + (1 - alpha_t) P_prior + beta_{t,i} k_t k_t^T
        mu_t = P_t^{-1} [alpha_t P_{t-1} mu_{t-1} + beta_{t,i} v_{t,i} k_t]
    k ``[T, dk]``, v and beta ``[T, dv]``, alpha ``[T]``, P_prior ``[dk, dk]``.
    With ``diagonal=True`` only the diagonal of every new precision is kept
    (the off-diagonal precision terms are discarded from the coupled
    solution, which is how Eq. (5) is obtained).
    Returns ``(mu [dv, dk], P [dv, dk, dk], mus [T, dv, dk])``.
    """
    k, v, beta, alpha = (np.asarray(x, dtype=np.float64) for x in (k, v, beta, alpha))
    P_prior = np.asarray(P_prior, dtype=np.float64)
    T, dk = k.shape
    dv = v.shape[1]
    mu = np.zeros((dv, dk)) if mu0 is None else np.array(mu0, dtype=np.float64)
    P = np.broadcast_to(P_prior, (dv, dk, dk)).copy() if P0 is None \
        else np.array(P0, dtype=np.float64)
    if diagonal:
        P = np.stack([np.diag(np.diag(Pi)) for Pi in P])
    mus = np.zeros((T, dv, dk))
    for t in range(T):
        a = alpha[t]
        for i in range(dv):
            P_new = a * P[i] + (1.0 - a) * P_prior + beta[t, i] * np.outer(k[t], k[t])
            if diagonal:
                P_new = np.diag(np.diag(P_new))
            rhs = a * P[i] @ mu[i] + beta[t, i] * v[t, i] * k[t]
            mu[i] = np.linalg.solve(P_new, rhs)
            P[i] = P_new
        mus[t] = mu
    return mu, P, mus


def fwd_mamba2_limit(q, k, v, beta, dt, A, I_prior, mu0=None):
    """Frozen-importance recurrence mu_t = alpha_t mu_{t-1} + ((beta.v)/I_prior) (x) k_t
    with readout y_t = mu_t q_t (scalar I_prior per head)."""
    q, k, v, beta, dt = (_f64(x) for x in (q, k, v, beta, dt))
    A, Ip = _f64(A), _f64(I_prior)
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    mu = np.zeros((B, H, dv, dk)) if mu0 is None else _f64(mu0).copy()
    y = np.zeros((B, T, H, dv))
    for b in range(B):
        for h in range(H):
            m = mu[b, h]
            for t in range(T):
                a, _ = _gate(A[h], dt[b, t, h])
                m = a * m + np.outer(beta[b, t, h] * v[b, t, h] / Ip[h], k[b, t, h])
                y[b, t, h] = m @ q[b, t, h]
            mu[b, h] = m
    return y, mu


def bwd_mamba2_limit(q, k, v, beta, dt, A, I_prior, gy, mu0=None, gmuT=None):
    """Reverse-mode derivative of ``fwd_mamba2_limit`` for
    ``L = <gy, y> + <gmuT, muT>``; ``beta`` None means ``v`` holds beta . v.

    The frozen recurrence m_t = a_t m_{t-1} + w_t k_t^T, w_t = beta_t v_t / I_prior,
    y_t = m_t q_t, walked from t = T-1 down with G the adjoint of m_t:
    G += gy_t q_t^T (readout), then gq_t = m_t^T gy_t, gk_t = G^T w_t,
    gw_t = G k_t, ga_t = <G, m_{t-1}>, and G = a_t G for m_{t-1}.  States
    are recomputed from checkpoints every ceil(sqrt(T)) tokens.  Returns a
    dict of float64 arrays gq, gk, gv, gbeta (None without beta), gdt, gA,
    gIp, gmu0."""
    q, k, v, dt, gy = (_f64(x) for x in (q, k, v, dt, gy))
    vstar = beta is None
    beta = np.ones(v.shape) if vstar else _f64(beta)
    A, Ip = _f64(A), _f64(I_prior)
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    m0 = np.zeros((B, H, dv, dk)) if mu0 is None else _f64(mu0)
    gT = np.zeros((B, H, dv, dk)) if gmuT is None else _f64(gmuT)
    out = {n: np.zeros(x.shape) for n, x in (("gq", q), ("gk", k), ("gv", v), ("gbeta", v), ("gdt", dt))}
    out["gA"], out["gIp"], out["gmu0"] = np.zeros(H), np.zeros(H), np.zeros((B, H, dv, dk))
    seg = max(1, int(np.ceil(np.sqrt(max(T, 1)))))
    for b in range(B):
        for h in range(H):
            w = beta[b, :, h] * v[b, :, h] / Ip[h]                    # [T, dv]
            gates = [_gate(A[h], dt[b, t, h])[0] for t in range(T)]
            # checkpoints: the state before tokens 0, seg, 2 seg, ...
            cks, m = [], m0[b, h].copy()
            for t in range(T):
                if t % seg == 0:
                    cks.append(m.copy())
                m = gates[t] * m + np.outer(w[t], k[b, t, h])
            G = gT[b, h].copy()
            for s0 in (range(((T - 1) // seg) * seg, -1, -seg) if T else ()):
                # states before each token of the segment [s0, s1)
                s1 = min(T, s0 + seg)
                states = [cks[s0 // seg]]
                for t in range(s0, s1):
                    states.append(gates[t] * states[-1] + np.outer(w[t], k[b, t, h]))
                for t in range(s1 - 1, s0 - 1, -1):
                    m_t, m_p = states[t - s0 + 1], states[t - s0]
                    G = G + np.outer(gy[b, t, h], q[b, t, h])
                    out["gq"][b, t, h] = m_t.T @ gy[b, t, h]
                    out["gk"][b, t, h] = G.T @ w[t]
                    gw = G @ k[b, t, h]
                    ga = float(np.sum(G * m_p))
                    out["gv"][b, t, h] = gw * beta[b, t, h] / Ip[h]
                    out["gbeta"][b, t, h] = gw * v[b, t, h] / Ip[h]
                    out["gIp"][h] -= float(gw @ w[t]) / Ip[h]
                    a = gates[t]
                    out["gdt"][b, t, h] = -A[h] * a * ga
                    out["gA"][h] -= dt[b, t, h] * a * ga
                    G = a * G
            out["gmu0"][b, h] = G
    if vstar:
        out["gbeta"] = None
    return out


def fwd_blockdiag(q, k, v, beta, dt, A, I_prior, block: int, mu0=None, P0=None):
    """Palimpsa with limited cross-key precision: the full-precision Gaussian
    update of each value row (slides, backup frame "dropping precision
    correlations changes the mean", App. A.3-A.5)

        P_t = alpha_t P_{t-1} + (1 - alpha_t) I_prior Id + beta_{t,i} k_t k_t^T
        mu_t = P_t^{-1} [alpha_t P_{t-1} mu_{t-1} + beta_{t,i} v_{t,i} k_t]

    with P_t projected, at every token, onto the block-diagonal matrices of
    ``block`` x ``block`` blocks along the key axis (the slides' closing
    question on limited cross-key correlations).  ``block = 1`` is Eq. (5);
    ``block = dk`` is the full update.  The prior is one scalar per head.

    Layouts as ``fwd``; the precision state is ``[B, H, dv, dk/block, block,
    block]`` (full blocks).  Defaults: ``mu0 = 0``, ``P0 = I_prior Id``.
    Returns ``(y, muT, PT)`` as float64.
    """
    q, k, v, beta, dt = (_f64(x) for x in (q, k, v, beta, dt))
    A, Ip = _f64(A), _f64(I_prior)
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    bs = int(block)
    if bs < 1 or dk % bs:
        raise ValueError("block must divide dk")
    nb = dk // bs
    eye = np.eye(bs)
    mu = np.zeros((B, H, dv, dk)) if mu0 is None else _f64(mu0).copy()
    if P0 is None:
        P = np.broadcast_to(Ip[None, :, None, None, None, None] * eye, (B, H, dv, nb, bs, bs)).copy()
    else:
        P = _f64(P0).copy()
        if P.shape != (B, H, dv, nb, bs, bs):
            raise ValueError("P0 must be [B, H, dv, dk/block, block, block]")
    y = np.zeros((B, T, H, dv))
    for b in range(B):
        for h in range(H):
            m = mu[b, h].reshape(dv, nb, bs)
            Pb = P[b, h]
            for t in range(T):
                a, oma = _gate(A[h], dt[b, t, h])
                kb = k[b, t, h].reshape(nb, bs)
                outer = kb[:, :, None] * kb[:, None, :]                       # [nb, bs, bs]
                P_new = a * Pb + oma * Ip[h] * eye + beta[b, t, h][:, None, None, None] * outer[None]
                rhs = a * np.einsum("rnij,rnj->rni", Pb, m) + \
                    (beta[b, t, h] * v[b, t, h])[:, None, None] * kb[None]
                m = np.linalg.solve(P_new, rhs[..., None])[..., 0]
                Pb = P_new
                y[b, t, h] = m.reshape(dv, dk) @ q[b, t, h]
            mu[b, h] = m.reshape(dv, dk)
            P[b, h] = Pb
    return y, mu, P


def bwd_blockdiag(q, k, v, beta, dt, A, I_prior, block: int, gy, mu0=None, P0=None, gmuT=None, gPT=None):
    """Reverse-mode derivative of ``fwd_blockdiag`` for
    ``L = <gy, y> + <gmuT, muT> + <gPT, PT>``.

    The forward in its natural parameters, per value row i and key block b
    (slides, backup frame "dropping precision correlations changes the mean"):
        P_t = a_t P_{t-1} + c_t Id + beta_i k_b k_b^T,   c_t = (1 - a_t) I_prior
        h_t = a_t h_{t-1} + (beta_i v_i) k_b,            h_0 = P_0 mu0
        mu_t = P_t^{-1} h_t,   y_t[i] = sum_b q_b . mu_t[i, b]
    walked from t = T-1 down with (G_h, G_P) the adjoints of (h_t, P_t): the
    readout adds w = P_t^{-1} gmu to G_h and -w mu_t^T to G_P (gmu = gy_i q_b);
    then gk gets (beta v) G_h + beta (G_P + G_P^T) k, the row's write
    gradient is G_h . k, beta's importance term k^T G_P k, the gate takes
    <G_h, h_{t-1}> + <G_P, P_{t-1}> and trace(G_P), and both adjoints decay by
    a_t.  P is treated as a full matrix (``gP0`` is the gradient with respect to
    every entry of P0).  States are recomputed from checkpoints every
    ceil(sqrt(T)) tokens.  Defaults ``mu0 = 0, P0 = I_prior Id``; the start state
    then depends on I_prior, so ``gIp`` also collects trace(dL/dP0).  Returns
    a dict of float64 arrays gq, gk, gv, gbeta, gdt, gA, gIp, gmu0, gP0."""
    q, k, v, beta, dt, gy = (_f64(x) for x in (q, k, v, beta, dt, gy))
    A, Ip = _f64(A), _f64(I_prior)
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    bs = int(block)
    if bs < 1 or dk % bs:
        raise ValueError("block must divide dk")
    nb = dk // bs
    eye = np.eye(bs)
    out = {n: np.zeros(x.shape) for n, x in (("gq", q), ("gk", k), ("gv", v), ("gbeta", v), ("gdt", dt))}
    out["gA"], out["gIp"] = np.zeros(H), np.zeros(H)
    out["gmu0"], out["gP0"] = np.zeros((B, H, dv, dk)), np.zeros((B, H, dv, nb, bs, bs))
    seg = max(1, int(np.ceil(np.sqrt(max(T, 1)))))
    solve = lambda M, x: np.linalg.solve(M, x[..., None])[..., 0]
    for b in range(B):
        for h in range(H):
            if mu0 is None:
                Pst = np.broadcast_to(Ip[h] * eye, (dv, nb, bs, bs)).copy()
                m0 = np.zeros((dv, nb, bs))
            else:
                Pst = _f64(P0)[b, h].copy()
                m0 = _f64(mu0)[b, h].reshape(dv, nb, bs)
            hst = np.einsum("rnij,rnj->rni", Pst, m0)
            gates = [_gate(A[h], dt[b, t, h]) for t in range(T)]

            def step(hh, PP, t):
                a, oma = gates[t]
                kb = k[b, t, h].reshape(nb, bs)
                bt = beta[b, t, h]
                PP = a * PP + oma * Ip[h] * eye + bt[:, None, None, None] * (kb[:, :, None] * kb[:, None, :])[None]
                hh = a * hh + (bt * v[b, t, h])[:, None, None] * kb[None]
                return hh, PP

            cks, hh, PP = [], hst.copy(), Pst.copy()
            for t in range(T):
                if t % seg == 0:
                    cks.append((hh.copy(), PP.copy()))
                hh, PP = step(hh, PP, t)
            Gh, GP = np.zeros((dv, nb, bs)), np.zeros((dv, nb, bs, bs))
            if gmuT is not None:
                w = solve(PP, _f64(gmuT)[b, h].reshape(dv, nb, bs))
                Gh += w
                GP -= w[..., :, None] * solve(PP, hh)[..., None, :]
            if gPT is not None:
                GP += _f64(gPT)[b, h]
            for s0 in (range(((T - 1) // seg) * seg, -1, -seg) if T else ()):
                s1 = min(s0 + seg, T)
                states = [cks[s0 // seg]]
                for t in range(s0, s1):
                    states.append(step(*states[-1], t))
                for t in range(s1 - 1, s0 - 1, -1):
                    (h_prev, P_prev), (h_t, P_t) = states[t - s0], states[t - s0 + 1]
                    a, oma = gates[t]
                    kb = k[b, t, h].reshape(nb, bs)
                    qb = q[b, t, h].reshape(nb, bs)
                    bt = beta[b, t, h]
                    bvv = bt * v[b, t, h]
                    mu_t = solve(P_t, h_t)
                    out["gq"][b, t, h] += (gy[b, t, h][:, None, None] * mu_t).sum(0).reshape(dk)
                    w = solve(P_t, gy[b, t, h][:, None, None] * qb[None])
                    Gh += w
                    GP -= w[..., :, None] * mu_t[..., None, :]
                    g_bv = (Gh * kb[None]).sum((1, 2))
                    GPs = GP + GP.swapaxes(-1, -2)
                    out["gk"][b, t, h] += (bvv[:, None, None] * Gh).sum(0).reshape(dk)
                    out["gk"][b, t, h] += (bt[:, None, None] * np.einsum("rnij,nj->rni", GPs, kb)).sum(0).reshape(dk)
                    out["gv"][b, t, h] = g_bv * bt
                    out["gbeta"][b, t, h] = g_bv * v[b, t, h] + np.einsum("rnij,ni,nj->r", GP, kb, kb)
                    g_a = (Gh * h_prev).sum() + (GP * P_prev).sum()
                    g_c = np.trace(GP, axis1=-2, axis2=-1).sum()
                    u = Ip[h] * g_c - g_a
                    out["gdt"][b, t, h] = A[h] * a * u
                    out["gA"][h] += dt[b, t, h] * a * u
                    out["gIp"][h] += oma * g_c
                    Gh *= a
                    GP *= a
            # start state h_0 = P_0 mu0
            out["gmu0"][b, h] = np.einsum("rnji,rnj->rni", Pst, Gh).reshape(dv, dk)
            out["gP0"][b, h] = GP + Gh[..., :, None] * m0[..., None, :]
            if mu0 is None:
                out["gIp"][h] += np.trace(out["gP0"][b, h], axis1=-2, axis2=-1).sum()
    return out


# ---------------------------------------------------------------------------
# head sampling for full-size parity checks
# ---------------------------------------------------------------------------

def select_heads(inputs: dict, heads) -> dict:
    """Gather the listed (b, h) heads of API-layout inputs into a batch of
    shape B=1, H=len(heads), so the oracle runs only on those heads.  Heads are
    independent, so the result equals the corresponding slice of a full run."""
    bs = np.array([b for b, _ in heads])
    hs = np.array([h for _, h in heads])
    out = {}
    for name in ("q", "k", "v", "beta"):
        x = _f64(inputs[name])                   # [B, T, H, d]
        out[name] = np.ascontiguousarray(x[bs, :, hs, :].transpose(1, 0, 2)[None])
    dt = _f64(inputs["dt"])                      # [B, T, H]
    out["dt"] = np.ascontiguousarray(dt[bs, :, hs].T[None])
    out["A"] = _f64(inputs["A"])[hs]
    out["I_prior"] = _f64(inputs["I_prior"])[hs]
    for name in ("mu0", "I0"):
        if inputs.get(name) is not None:
            out[name] = np.ascontiguousarray(_f64(inputs[name])[bs, hs][None])
        else:
            out[name] = None
    return out
