"""Seeded synthetic inputs for the Palimpsa recurrence.

This module only draws random inputs; it contains none of the recurrence's
arithmetic, and both the HIP path and the oracle consume exactly what it
returns.  Inputs are CPU torch tensors in the library layouts
(q, k ``[B, T, H, dk]``; v, beta ``[B, T, H, dv]``; dt ``[B, T, H]``;
A, I_prior ``[H]`` float32).

Distributions follow the workloads described for the layer:
  * q, k ~ N(0, 1), then L2-normalised per token (in float32, before any
    rounding to bfloat16);
  * v ~ N(0, 1);
  * beta = sigmoid(N(0, 1)) per value channel;
  * dt = softplus(N(mean, 1)) with mean 0 (mean -2 for the long-context case);
  * A = 1 per head, or log-spaced on [1, 16] across heads;
  * I_prior = 1 per head; the initial state is mu0 = 0, I0 = I_prior.

Draw order from one CPU ``torch.Generator``: q, k, v, beta logits, dt raw,
then (key-pool case only) the pool and the per-token pool indices.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, replace

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    T: int
    dk: int
    dv: int
    chunk: int
    dtype: torch.dtype          # input/output storage type (state is float32)
    seed: int
    A_mode: str = "ones"        # "ones" or "logspace16"
    dt_mean: float = 0.0
    key_pool: int = 0           # > 0: keys drawn from a fixed pool of unit vectors
    beta_const: float | None = None   # overrides beta with a constant

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


WORKLOADS = {
    # tiny fp32 reference case
    0: Workload("tiny-fp32 B1 H2 T256 d32", 1, 2, 256, 32, 32, 32, torch.float32, 0),
    # MQAR-scale layer with keys reused from a 512-vector pool
    1: Workload("mqar-fp32 B4 H8 T2048 d64", 4, 8, 2048, 64, 64, 64, torch.float32, 1,
                key_pool=512),
    # 760M-model layer shape, bf16 inputs
    2: Workload("layer760m-bf16 B8 H12 T4096 d128", 8, 12, 4096, 128, 128, 64,
                torch.bfloat16, 2, A_mode="logspace16"),
    # recurrent decode: B64 H32 d128; T is the prefill length, steps separate
    3: Workload("decode-bf16 B64 H32 d128 prefill2048", 64, 32, 2048, 128, 128, 64,
                torch.bfloat16, 3, A_mode="logspace16"),
    # long context, bf16, long memory windows
    4: Workload("longctx-bf16 B1 H32 T32768 d128", 1, 32, 32768, 128, 128, 64,
                torch.bfloat16, 4, A_mode="logspace16", dt_mean=-2.0),
}
# the frozen-importance variant of the long-context case
WORKLOADS["4b"] = WORKLOADS[4].with_(name="longctx-bf16-beta1e-6 B1 H32 T32768 d128",
                                     beta_const=1e-6)

DECODE_STEPS = 1024


def head_constants(w: Workload):
    """Per-head A and I_prior (float32)."""
    if w.A_mode == "ones":
        A = torch.ones(w.H, dtype=torch.float32)
    elif w.A_mode == "logspace16":
        A = torch.exp(torch.linspace(0.0, math.log(16.0), w.H, dtype=torch.float64)).float()
    else:
        raise ValueError(w.A_mode)
    return A, torch.ones(w.H, dtype=torch.float32)


def _unit(x: torch.Tensor) -> torch.Tensor:
    return x / x.norm(dim=-1, keepdim=True)


def make_inputs(w: Workload, T: int | None = None, seed: int | None = None,
                device: str | torch.device = "cpu") -> dict:
    """Draw one sequence batch for workload ``w`` (``T`` overrides its length).

    With ``device`` a GPU the numbers come from that device's generator (a
    different stream than the CPU's, used for inputs too large to draw on
    the host quickly); both sides of a comparison then read the same tensors.
    """
    T = w.T if T is None else T
    g = torch.Generator(device=device).manual_seed(w.seed if seed is None else seed)
    B, H, dk, dv = w.B, w.H, w.dk, w.dv
    kw = dict(generator=g, device=device)
    q = _unit(torch.randn(B, T, H, dk, **kw))
    k = _unit(torch.randn(B, T, H, dk, **kw))
    v = torch.randn(B, T, H, dv, **kw)
    beta = torch.sigmoid(torch.randn(B, T, H, dv, **kw))
    dt = torch.nn.functional.softplus(torch.randn(B, T, H, **kw) + w.dt_mean)
    if w.key_pool:
        pool = _unit(torch.randn(w.key_pool, dk, **kw))
        idx = torch.randint(0, w.key_pool, (B, T, H), **kw)
        k = pool[idx]
    if w.beta_const is not None:
        beta = torch.full_like(beta, w.beta_const)
    A, Ip = head_constants(w)
    cast = (lambda x: x.to(w.dtype).contiguous())
    return {"q": cast(q), "k": cast(k), "v": cast(v), "beta": cast(beta), "dt": cast(dt),
            "A": A.to(device), "I_prior": Ip.to(device), "mu0": None, "I0": None}


def decode_inputs(w: Workload, step: int, device: str | torch.device = "cpu") -> dict:
    """Fresh single-token inputs for decode step ``step`` (0-based); each step
    has its own seed, so any step can be regenerated on its own."""
    g = torch.Generator(device=device).manual_seed(1_000_000 * (w.seed + 1) + step)
    B, H, dk, dv = w.B, w.H, w.dk, w.dv
    kw = dict(generator=g, device=device)
    q = _unit(torch.randn(B, H, dk, **kw))
    k = _unit(torch.randn(B, H, dk, **kw))
    v = torch.randn(B, H, dv, **kw)
    beta = torch.sigmoid(torch.randn(B, H, dv, **kw))
    dt = torch.nn.functional.softplus(torch.randn(B, H, **kw) + w.dt_mean)
    cast = (lambda x: x.to(w.dtype).contiguous())
    return {"q": cast(q), "k": cast(k), "v": cast(v), "beta": cast(beta), "dt": cast(dt)}


def random_state(B: int, H: int, dv: int, dk: int, I_prior: torch.Tensor, seed: int):
    """A non-trivial initial state: mu0 ~ 0.5 N(0, 1), I0 = I_prior * (1 + Exp(1))."""
    g = torch.Generator().manual_seed(seed)
    mu0 = 0.5 * torch.randn(B, H, dv, dk, generator=g)
    excess = torch.empty(B, H, dv, dk).exponential_(1.0, generator=g)
    I0 = I_prior.view(1, H, 1, 1) * (1.0 + excess)
    return mu0.float().contiguous(), I0.float().contiguous()


def upstream_grads(B: int, T: int, H: int, dv: int, dk: int, dtype: torch.dtype, seed: int,
                   final: bool = True) -> dict:
    """Seeded upstream gradients for the backward: gy ~ N(0, 1) in the
    output dtype, and (if ``final``) gmuT, gIT ~ 0.1 N(0, 1) in float32."""
    g = torch.Generator().manual_seed(10_000 + seed)
    out = {"gy": torch.randn(B, T, H, dv, generator=g).to(dtype).contiguous(), "gmuT": None, "gIT": None}
    if final:
        out["gmuT"] = (0.1 * torch.randn(B, H, dv, dk, generator=g)).contiguous()
        out["gIT"] = (0.1 * torch.randn(B, H, dv, dk, generator=g)).contiguous()
    return out


def per_entry_prior(H: int, dv: int, dk: int, seed: int) -> torch.Tensor:
    """A seeded prior precision per state entry, I_prior[h, i, j] ~ U[0.5, 2]."""
    g = torch.Generator().manual_seed(20_000 + seed)
    return (0.5 + 1.5 * torch.rand(H, dv, dk, generator=g)).contiguous()


def random_block_state(B: int, H: int, dv: int, dk: int, block: int, I_prior: torch.Tensor, seed: int):
    """A non-trivial start state for the block-diagonal forward: mu0 ~ 0.5 N(0, 1)
    and each precision block I_prior Id + L L^T with L ~ 0.5 N(0, 1) (symmetric
    positive definite), layout [B, H, dv, dk/block, block, block]."""
    g = torch.Generator().manual_seed(30_000 + seed)
    mu0 = 0.5 * torch.randn(B, H, dv, dk, generator=g)
    L = 0.5 * torch.randn(B, H, dv, dk // block, block, block, generator=g)
    P0 = I_prior.view(1, H, 1, 1, 1, 1) * torch.eye(block) + L @ L.transpose(-1, -2)
    return mu0.float().contiguous(), P0.float().contiguous()


def block_state_grads(B: int, H: int, dv: int, dk: int, block: int, seed: int) -> torch.Tensor:
    """A seeded upstream gradient of the final precision blocks for the
    block-diagonal backward, gPT ~ 0.1 N(0, 1) in every entry (not symmetric),
    layout [B, H, dv, dk/block, block, block], float32."""
    g = torch.Generator().manual_seed(40_000 + seed)
    return (0.1 * torch.randn(B, H, dv, dk // block, block, block, generator=g)).contiguous()
