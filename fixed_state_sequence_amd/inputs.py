"""Seeded synthetic inputs for causal linear attention.

This module only draws and rounds random numbers; it holds none of the
method's arithmetic.  Both the GPU path's tests/bench and the fp64 oracle
consume what it returns, so it is the one piece of code they share.

Workloads (shapes and distributions follow the pages' worked example and the
five measured configurations):

* ``tiny_worked_example`` -- T=8, d=4, fp32, Q, K, V drawn as three
  ``randn(8, 4)`` calls after seeding the generator with 0, in that order
  (efficient-attention lesson "Linear attention", Developer level, "The
  regrouping, and the recurrence it implies").
* ``prefill_inputs`` -- Q, K, V ~ N(0, 1) * scale, drawn in fp32 and rounded
  to the storage dtype with round-to-nearest-even; optional per-token
  per-head decay ``a = sigmoid(x)``, ``x ~ N(mean, 1)``, or RFA gate
  ``g = sigmoid(N(0, 1))``, or mLSTM gate pre-activations (input
  ``N(0, 1)``, forget ``N(3, 1)``: sigmoid(3) ~ 0.95, the SSD workload's
  typical decay); optional RFF projection ``W ~ N(0, I)``.
* ``rfa_decode_step_inputs`` -- unit-norm q, k (normalised in fp64, stored
  fp32), v ~ N(0, 1), gate g = sigmoid(N(0, 1)); ``W`` drawn once per head.

Random numbers come from ``torch.Generator`` (CPU unless a CUDA device is
asked for; the CUDA stream of numbers differs from the CPU one).
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import torch

DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}


def _gen(seed: int, device="cpu") -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def tiny_worked_example():
    """Q, K, V of the pages' worked example: seed 0, randn(8, 4) x 3, fp32."""
    g = _gen(0)
    q = torch.randn(8, 4, generator=g)
    k = torch.randn(8, 4, generator=g)
    v = torch.randn(8, 4, generator=g)
    return q, k, v


@dataclass
class PrefillInputs:
    q: torch.Tensor            # [B, H, T, d_h], storage dtype
    k: torch.Tensor            # [B, H, T, d_h]
    v: torch.Tensor            # [B, H, T, d_v]
    decay: Optional[torch.Tensor] = None   # [B, H, T] fp32 (SSD decay a_t)
    gate: Optional[torch.Tensor] = None    # [B, H, T] fp32 (RFA gate g_t)
    W: Optional[torch.Tensor] = None       # [H, D, d_h] fp32 (RFF projection)
    igate: Optional[torch.Tensor] = None   # [B, H, T] fp32 (mLSTM input pre-activation)
    fgate: Optional[torch.Tensor] = None   # [B, H, T] fp32 (mLSTM forget pre-activation)
    meta: dict = field(default_factory=dict)


def prefill_inputs(B: int, H: int, T: int, d_h: int, d_v: Optional[int] = None,
                   dtype: str = "bf16", seed: int = 0, scale: float = 1.0,
                   decay: Optional[str] = None, decay_mean: float = 3.0,
                   rff_D: Optional[int] = None, unit_norm_qk: bool = False,
                   device="cpu") -> PrefillInputs:
    """Draw Q, K, V (in that order), then the decay/gate input, then W.

    ``decay``: None, "ssd" (a = sigmoid(x), x ~ N(decay_mean, 1)), "rfa"
    (g = sigmoid(N(0, 1))) or "mlstm" (input pre-activations ~ N(0, 1), then
    forget pre-activations ~ N(decay_mean, 1)).  Values are drawn in fp32,
    scaled in fp32 and then rounded once to ``dtype`` (round to nearest even).
    """
    d_v = d_h if d_v is None else d_v
    g = _gen(seed, device)
    sd = DTYPES[dtype]
    q = torch.randn(B, H, T, d_h, generator=g, device=device)
    k = torch.randn(B, H, T, d_h, generator=g, device=device)
    v = torch.randn(B, H, T, d_v, generator=g, device=device)
    if unit_norm_qk:
        q = (q.double() / q.double().norm(dim=-1, keepdim=True)).float()
        k = (k.double() / k.double().norm(dim=-1, keepdim=True)).float()
    if scale != 1.0:
        q, k, v = q * scale, k * scale, v * scale
    out = PrefillInputs(q.to(sd), k.to(sd), v.to(sd),
                        meta=dict(B=B, H=H, T=T, d_h=d_h, d_v=d_v, dtype=dtype,
                                  seed=seed, scale=scale, decay=decay))
    if decay == "ssd":
        x = torch.randn(B, H, T, generator=g, device=device) + decay_mean
        out.decay = torch.sigmoid(x).float()
    elif decay == "rfa":
        out.gate = torch.sigmoid(torch.randn(B, H, T, generator=g, device=device)).float()
    elif decay == "mlstm":
        out.igate = torch.randn(B, H, T, generator=g, device=device)
        out.fgate = torch.randn(B, H, T, generator=g, device=device) + decay_mean
    elif decay is not None:
        raise ValueError(f"unknown decay kind {decay!r}")
    if rff_D is not None:
        out.W = torch.randn(H, rff_D, d_h, generator=g, device=device)
    return out


def rff_projection(H: int, D: int, d_h: int, seed: int = 0, device="cpu") -> torch.Tensor:
    """W ~ N(0, I), one [D, d_h] matrix per head, fp32: [H, D, d_h]."""
    return torch.randn(H, D, d_h, generator=_gen(seed, device), device=device)


@dataclass
class DecodeStep:
    q: torch.Tensor   # [N, H, d_h] fp32, unit norm
    k: torch.Tensor   # [N, H, d_h] fp32, unit norm
    v: torch.Tensor   # [N, H, d_v] fp32
    gate: torch.Tensor  # [N, H] fp32 in (0, 1)


def rfa_decode_step_inputs(N: int, H: int, d_h: int, d_v: Optional[int] = None,
                           step: int = 0, seed: int = 0, device="cpu") -> DecodeStep:
    """One decode step's inputs, from a generator seeded with (seed, step).

    q and k are normalised to unit L2 norm in fp64 and stored fp32; v is
    N(0, 1); the gate is sigmoid(N(0, 1)).
    """
    d_v = d_h if d_v is None else d_v
    g = _gen(1_000_003 * (seed + 1) + step, device)
    q = torch.randn(N, H, d_h, generator=g, device=device, dtype=torch.float64)
    k = torch.randn(N, H, d_h, generator=g, device=device, dtype=torch.float64)
    v = torch.randn(N, H, d_v, generator=g, device=device)
    gate = torch.sigmoid(torch.randn(N, H, generator=g, device=device))
    q = (q / q.norm(dim=-1, keepdim=True)).float()
    k = (k / k.norm(dim=-1, keepdim=True)).float()
    return DecodeStep(q, k, v, gate.float())


def rfa_decode_batch(steps: int, N: int, H: int, d_h: int, d_v: Optional[int] = None,
                     seed: int = 1, device="cpu") -> DecodeStep:
    """Inputs of `steps` decode steps drawn at once (for timing runs): q, k
    [steps, N, H, d_h] unit norm (fp64 normalisation, stored fp32), v
    [steps, N, H, d_v] ~ N(0, 1), gate [steps, N, H] = sigmoid(N(0, 1)).
    Same distributions as ``rfa_decode_step_inputs``; one generator."""
    d_v = d_h if d_v is None else d_v
    g = _gen(seed, device)
    q = torch.randn(steps, N, H, d_h, generator=g, device=device, dtype=torch.float64)
    k = torch.randn(steps, N, H, d_h, generator=g, device=device, dtype=torch.float64)
    v = torch.randn(steps, N, H, d_v, generator=g, device=device)
    gate = torch.sigmoid(torch.randn(steps, N, H, generator=g, device=device))
    q = (q / q.norm(dim=-1, keepdim=True)).float()
    k = (k / k.norm(dim=-1, keepdim=True)).float()
    return DecodeStep(q, k, v, gate.float().contiguous())


# --- the measured workloads, named by what they are --------------------------

WORKLOADS = {
    "tiny_causal_t8_d4": dict(kind="prefill", B=1, H=1, T=8, d_h=4, dtype="f32",
                              decay=None, tiny=True),
    "elu_prefill_b4_h8_t2048_d64": dict(kind="prefill", B=4, H=8, T=2048, d_h=64,
                                        dtype="bf16", decay=None),
    "ssd_prefill_b2_h16_t8192_d128": dict(kind="prefill", B=2, H=16, T=8192, d_h=128,
                                          dtype="bf16", decay="ssd"),
    "long_prefill_b1_h8_t102400_d128": dict(kind="prefill", B=1, H=8, T=102400, d_h=128,
                                            dtype="bf16", decay=None,
                                            scale=2.0 ** -0.5),
    "rfa_decode_n256_h16_d64_D64": dict(kind="decode", N=256, H=16, d_h=64, D=64,
                                        steps=1024),
    # the long-context shape with the mLSTM gates and identity features
    "mlstm_prefill_b1_h8_t102400_d128": dict(kind="prefill", B=1, H=8, T=102400, d_h=128,
                                             dtype="bf16", decay="mlstm",
                                             scale=2.0 ** -0.5),
}


def workload_inputs(name: str, seed: int = 0, device="cpu", **override):
    """Prefill inputs for one of the named prefill workloads."""
    w = dict(WORKLOADS[name])
    w.update(override)
    if w["kind"] != "prefill":
        raise ValueError(f"{name} is not a prefill workload")
    if w.get("tiny"):
        q, k, v = tiny_worked_example()
        return PrefillInputs(q.view(1, 1, 8, 4), k.view(1, 1, 8, 4), v.view(1, 1, 8, 4),
                             meta=dict(B=1, H=1, T=8, d_h=4, d_v=4, dtype="f32", seed=0))
    return prefill_inputs(w["B"], w["H"], w["T"], w["d_h"], dtype=w["dtype"], seed=seed,
                          scale=w.get("scale", 1.0), decay=w.get("decay"), device=device)
