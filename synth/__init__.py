"""Seeded synthetic inputs for the ReplaySSM decode workloads.

This module is shared by the HIP path's tests/benchmark and by the oracle's
tests.  It holds no arithmetic of the method: only the workload shapes and the
random draws that stand in for the activations of a hybrid model's SSM layers
(the article's evaluated models and datasets are not available, so inputs are
synthetic with the shapes and settings the article names: batch 256/512,
16-token intervals, 4 draft tokens, fp32 state).

Distributions (one draw per element, seeded per (workload seed, layer, stream)):
    x, B, C       ~ N(0, 1)
    dt            = softplus(N(0, 1) - 2)           (already post-softplus)
    A  (per head) = -exp(U[0, ln 16))               so A in (-16, -1]
    D  (per head) ~ N(0, 1)
    S0            ~ N(0, 0.1^2)                     (std 0.1)
    accepted drafts a ~ U{0..T-1}; positions kept n_keep = 1 + a
bf16 inputs are drawn in fp32 and rounded once (round-to-nearest-even, by
torch's cast) to bf16; A and D stay fp32.  Both sides consume the identical
stored values.
"""
from __future__ import annotations

import dataclasses
import math

import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    layers: int
    heads: int
    groups: int
    head_dim: int = 64      # P
    d_state: int = 128      # N
    interval: int = 16      # L
    steps: int = 512
    in_dtype: str = "bf16"  # "f32" | "bf16"
    drafts: int = 0         # draft tokens per speculative round (T = drafts + 1)
    rounds: int = 0
    seed: int = 0

    @property
    def max_draft(self) -> int:
        return self.drafts + 1 if self.drafts else 1

    def describe(self) -> str:
        return (f"{self.name}: B={self.batch} layers={self.layers} H={self.heads} "
                f"G={self.groups} P={self.head_dim} N={self.d_state} L={self.interval} "
                f"in={self.in_dtype}")


WORKLOADS = {
    # replay-vs-recurrence check: everything fp32, 4 intervals
    "tiny": Workload("tiny", batch=4, layers=1, heads=8, groups=1, steps=64,
                     in_dtype="f32", seed=0),
    # 4B-class hybrid model SSM layers
    "4b": Workload("4b", batch=256, layers=4, heads=96, groups=8, steps=512, seed=1),
    # 120B-class hybrid model SSM layers
    "120b": Workload("120b", batch=256, layers=8, heads=128, groups=8, steps=256, seed=2),
    # speculative verify + rollback on the 120B-class shape, 4 drafts
    "spec": Workload("spec", batch=512, layers=4, heads=128, groups=8, drafts=4,
                     rounds=200, seed=3),
    # precision split on the 4B-class shape
    "split": Workload("split", batch=256, layers=4, heads=96, groups=8, steps=512, seed=4),
}


def _dtype(name: str):
    return {"f32": torch.float32, "bf16": torch.bfloat16}[name]


def _gen(device, *key) -> torch.Generator:
    """A generator seeded from a tuple of small non-negative integers."""
    s = 0x9E3779B97F4A7C15
    for k in key:
        s = (s * 1000003 + int(k) + 1) % (1 << 63)
    g = torch.Generator(device=device)
    g.manual_seed(s)
    return g


def _softplus(z: torch.Tensor) -> torch.Tensor:
    # ln(1 + e^z), the positive transform that produces dt from a raw draw
    return torch.nn.functional.softplus(z)


def layer_params(w: Workload, layer: int, device="cpu"):
    """A [H] and D [H], fp32."""
    g = _gen(device, w.seed, layer, 0)
    u = torch.rand(w.heads, generator=g, device=device, dtype=torch.float32)
    A = -torch.exp(u * math.log(16.0))
    D = torch.randn(w.heads, generator=g, device=device, dtype=torch.float32)
    return A.contiguous(), D.contiguous()


def init_state(w: Workload, layer: int, device="cpu", batch: int | None = None):
    """S0 [batch, H, P, N] fp32 ~ N(0, 0.1^2)."""
    b = w.batch if batch is None else batch
    g = _gen(device, w.seed, layer, 1)
    S = torch.randn(b, w.heads, w.head_dim, w.d_state, generator=g, device=device,
                    dtype=torch.float32)
    return (S * 0.1).contiguous()


def token_inputs(w: Workload, layer: int, steps: int, device="cpu", stream: int = 0,
                 batch: int | None = None, tokens: int | None = None):
    """Inputs of ``steps`` consecutive calls.

    Returns x [steps, (tokens,) batch, H, P], Bm/Cm [steps, (tokens,) batch, G, N],
    dt [steps, (tokens,) batch, H] in the workload's input dtype.  ``tokens``
    adds a per-call token axis (speculative rounds); ``stream`` separates
    independent input streams of one layer."""
    b = w.batch if batch is None else batch
    lead = (steps,) if tokens is None else (steps, tokens)
    g = _gen(device, w.seed, layer, 2, stream)
    f32 = torch.float32
    x = torch.randn(*lead, b, w.heads, w.head_dim, generator=g, device=device, dtype=f32)
    Bm = torch.randn(*lead, b, w.groups, w.d_state, generator=g, device=device, dtype=f32)
    Cm = torch.randn(*lead, b, w.groups, w.d_state, generator=g, device=device, dtype=f32)
    z = torch.randn(*lead, b, w.heads, generator=g, device=device, dtype=f32)
    dt = _softplus(z - 2.0)
    dt_ = _dtype(w.in_dtype)
    return (x.to(dt_).contiguous(), Bm.to(dt_).contiguous(), Cm.to(dt_).contiguous(),
            dt.to(dt_).contiguous())


def n_keep(w: Workload, rounds: int, device="cpu", batch: int | None = None,
           stream: int = 0):
    """[rounds, batch] int32 positions kept per speculative round: 1 + a with
    a ~ U{0..drafts}.  Acceptance belongs to the sequence, so every layer of
    a model sees the same values."""
    b = w.batch if batch is None else batch
    g = _gen(device, w.seed, 3, stream)
    a = torch.randint(0, w.drafts + 1, (rounds, b), generator=g, device=device,
                      dtype=torch.int64)
    return (a + 1).to(torch.int32).contiguous()
