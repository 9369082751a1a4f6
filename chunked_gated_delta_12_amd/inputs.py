"""Seeded synthetic inputs for the KDA operator.

This module is shared by the tests, the benchmark and the smoke check, and it
holds none of the operator's arithmetic: it only draws random tensors with the
shapes and distributions of the workloads below and rounds them to their
storage dtypes.  Both the HIP path and the oracle consume the very tensors it
returns (the oracle after an exact widening to float64).

Workloads follow the pages' long-context setting: 16-token chunks, a 64K
training-length prefill, a decay-bound stress case and a 1M-token prefill
(the context curriculum of "Architecture Deep Dive: Kimi K3...", section 5.1,
and the "Kimi K3" explainer, "Training the whole system").

Distributions (the second parameter of N is the standard deviation):
  q, v ~ N(0, 1);  k ~ N(0, 1) then L2-normalised per token and head;
  theta ~ N(mu, sigma) per channel;  beta = sigmoid(N(0, 1)) per token and head;
  S0 ~ N(0, s0_sigma) in fp32 (or absent).
Draw order: q, k, v, theta, beta, S0, all from one torch.Generator seeded with
the workload's seed on the device the tensors are made on.  q, k, v are
rounded to bf16 (round-to-nearest-even) unless the workload is fp32.

The output gate's pre-activation z ~ N(0, 2), in the storage dtype, comes from
a generator of its own (seed + 1000), so adding it leaves the draws above
unchanged.  With a standard deviation of 2 the gate sigmoid(z) spans about
0.02 .. 0.98 over the central 95% of draws.
"""
from __future__ import annotations

from dataclasses import dataclass, replace
from typing import Optional

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    T: int
    dk: int
    dv: int
    dtype: str            # "bf16" or "f32": storage of q, k, v and o
    theta_mu: float
    theta_sigma: float
    s0_sigma: Optional[float]
    seed: int


# Six workloads; the index doubles as the seed.  long_memory sits at the slow end of
# the bounded gate: theta ~ N(-8, 1) gives g of about -3e-3 per token, a chunk keeps
# about 95% of the state and a 512-token segment about a quarter, so every chunk's
# output depends on many chunks before it and segments hand a large part of the
# state on (the other workloads forget most of it within a chunk).
WORKLOADS = {
    "tiny": Workload("tiny", 1, 1, 64, 16, 16, "f32", 0.0, 1.0, None, 0),
    "small": Workload("small", 2, 4, 1024, 64, 64, "bf16", 0.0, 1.0, 0.1, 1),
    "prefill_64k": Workload("prefill_64k", 1, 16, 65536, 128, 128, "bf16", 0.0, 2.0, None, 2),
    "decay_stress": Workload("decay_stress", 1, 16, 8192, 128, 128, "bf16", 8.0, 1.0, None, 3),
    "prefill_1m": Workload("prefill_1m", 1, 16, 1 << 20, 128, 128, "bf16", 0.0, 2.0, None, 4),
    "long_memory": Workload("long_memory", 1, 16, 8192, 128, 128, "bf16", -8.0, 1.0, 0.1, 5),
}


@dataclass(frozen=True)
class DecodeWorkload:
    name: str
    B: int
    H: int
    dk: int
    dv: int
    steps: int
    dtype: str
    theta_mu: float
    theta_sigma: float
    s_sigma: float
    seed: int


DECODE_WORKLOADS = {
    "decode_b256": DecodeWorkload("decode_b256", 256, 16, 128, 128, 1024, "bf16", 0.0, 2.0, 0.1, 4),
}


def scaled(w: Workload, **kw) -> Workload:
    """Same distributions, other sizes (for tests that need a smaller case)."""
    return replace(w, **kw)


def torch_dtype(name: str) -> torch.dtype:
    return {"bf16": torch.bfloat16, "f32": torch.float32}[name]


def _normal(shape, gen, device, mu=0.0, sigma=1.0):
    x = torch.randn(*shape, generator=gen, device=device, dtype=torch.float32)
    if sigma != 1.0:
        x.mul_(sigma)
    if mu != 0.0:
        x.add_(mu)
    return x


def chunk_inputs(w: Workload, device="cpu"):
    """Returns dict q, k, v (storage dtype), theta, beta (fp32), S0 (fp32 or None)."""
    gen = torch.Generator(device=device)
    gen.manual_seed(w.seed)
    dt = torch_dtype(w.dtype)
    B, T, H, dk, dv = w.B, w.T, w.H, w.dk, w.dv
    q = _normal((B, T, H, dk), gen, device).to(dt)
    k = _normal((B, T, H, dk), gen, device)
    k = (k / k.norm(dim=-1, keepdim=True)).to(dt)
    v = _normal((B, T, H, dv), gen, device).to(dt)
    theta = _normal((B, T, H, dk), gen, device, w.theta_mu, w.theta_sigma)
    beta = torch.sigmoid(_normal((B, T, H), gen, device))
    S0 = None
    if w.s0_sigma is not None:
        S0 = _normal((B, H, dk, dv), gen, device, 0.0, w.s0_sigma)
    return dict(q=q, k=k, v=v, theta=theta, beta=beta, S0=S0)


def decode_state(w: DecodeWorkload, device="cpu"):
    """Initial fp32 state S ~ N(0, s_sigma), shape [B, H, dk, dv], and the generator
    that then yields the per-step tokens (pass it to decode_token)."""
    gen = torch.Generator(device=device)
    gen.manual_seed(w.seed)
    S = _normal((w.B, w.H, w.dk, w.dv), gen, device, 0.0, w.s_sigma)
    return S, gen


def decode_token(w: DecodeWorkload, gen, device="cpu", steps: int = 1):
    """The next `steps` tokens: q, k, v [steps, B, H, d] (storage dtype), theta
    [steps, B, H, dk], beta [steps, B, H] (fp32)."""
    dt = torch_dtype(w.dtype)
    B, H, dk, dv = w.B, w.H, w.dk, w.dv
    q = _normal((steps, B, H, dk), gen, device).to(dt)
    k = _normal((steps, B, H, dk), gen, device)
    k = (k / k.norm(dim=-1, keepdim=True)).to(dt)
    v = _normal((steps, B, H, dv), gen, device).to(dt)
    theta = _normal((steps, B, H, dk), gen, device, w.theta_mu, w.theta_sigma)
    beta = torch.sigmoid(_normal((steps, B, H), gen, device))
    return dict(q=q, k=k, v=v, theta=theta, beta=beta)


def output_gate_preact(shape, dtype: str, seed: int, device="cpu", sigma: float = 2.0):
    """Pre-activation z of the output gate: N(0, sigma) of the given shape, rounded
    to the storage dtype, drawn from a generator seeded with seed + 1000."""
    gen = torch.Generator(device=device)
    gen.manual_seed(seed + 1000)
    return _normal(tuple(shape), gen, device, 0.0, sigma).to(torch_dtype(dtype))
