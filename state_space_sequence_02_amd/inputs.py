"""Seeded synthetic inputs for the Mamba-3 SSM recurrence.

This module only draws random tensors; it holds none of the recurrence's
arithmetic.  Both the HIP path (through the binding) and the CPU oracle are fed
from here, so the two sides always see the same values.

Distributions (the five workload descriptions shipped with this repository):
  x ~ N(0, 1)                      layout [b, L, H, R, P]
  B, C ~ N(0, 1/N)                 layout [b, L, H, R, N]
  dt = softplus(N(0, 1) - 3)       layout [b, L, H]
  A = -exp(U(0, ln 16))            layout [H]   (one scalar per head)
  lam = sigmoid(N(0, 1))           layout [b, L, H]   (U[0, 1] for "long")
  theta = dt * U(-pi, pi)          layout [b, L, H, N/2] (per-step angle per pair)

Draw order: A, x, B, C, dt-pre, lam-pre, theta-pre, from one generator seeded
with `seed`.  x, B and C are rounded to bfloat16 (round to nearest even) when
the workload's dtype is bf16, and that rounded tensor *is* the input both sides
consume.

Shapes follow the Mamba-3 pages: the 1.5B-layer geometry (model width 2048 =
32 heads x P=64, state N=64/128) of the decode-latency and prefill timing
tables (Mamba-3 paper page, Table 6 as quoted in section 4.4, Table 7 and
App. G.2), with the MIMO rank R=4 of section 3.3.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, replace
from typing import Optional

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    seqlen: int
    nheads: int
    headdim: int      # P
    dstate: int       # N
    rank: int         # R
    chunk: int        # tokens per chunk requested from the prefill (0 = library default)
    dtype: str        # "fp32" or "bf16": dtype of x, B, C and y
    lam_dist: str = "sigmoid"   # "sigmoid" -> sigmoid(N(0,1)); "uniform" -> U[0,1]
    rotation: bool = True
    steps: int = 0    # decode workloads: number of successive single-token steps

    @property
    def torch_dtype(self) -> torch.dtype:
        return torch.float32 if self.dtype == "fp32" else torch.bfloat16


WORKLOADS = {
    # tiny SISO case the oracle finishes instantly
    "tiny": Workload("tiny", 1, 64, 1, 16, 16, 1, 64, "fp32"),
    # SISO prefill at the 1.5B-layer shape
    "siso": Workload("siso", 4, 4096, 32, 64, 64, 1, 64, "bf16"),
    # MIMO prefill, rank 4, N=128, rotations on
    "mimo": Workload("mimo", 4, 4096, 32, 64, 128, 4, 64, "bf16"),
    # MIMO decode: 128 sequences x 32 heads, 256 successive steps
    "decode": Workload("decode", 128, 1, 32, 64, 128, 4, 0, "bf16", steps=256),
    # long-context MIMO prefill, lambda ~ U[0,1]
    "long": Workload("long", 1, 65536, 32, 64, 128, 4, 128, "bf16", lam_dist="uniform"),
}


def workload(name: str, **overrides) -> Workload:
    w = WORKLOADS[name]
    return replace(w, **overrides) if overrides else w


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def _lam(g, shape, dist, device):
    if dist == "sigmoid":
        return torch.sigmoid(torch.randn(shape, generator=g, device=device))
    if dist == "uniform":
        return torch.rand(shape, generator=g, device=device)
    raise ValueError(f"unknown lambda distribution {dist!r}")


def _cast(t: torch.Tensor, w: Workload) -> torch.Tensor:
    return t.to(w.torch_dtype).contiguous()


def make_prefill_inputs(w: Workload, seed: int = 0, device="cpu",
                        seqlen: Optional[int] = None, batch: Optional[int] = None) -> dict:
    """Draws one prefill problem.  Returns a dict of tensors on `device`.

    x, B, C are in w.dtype; dt, A, lam, theta are float32.  `theta` is None when
    the workload has rotation off.
    """
    b = w.batch if batch is None else batch
    L = w.seqlen if seqlen is None else seqlen
    H, P, N, R = w.nheads, w.headdim, w.dstate, w.rank
    g = _gen(seed, device)
    f32 = dict(dtype=torch.float32, device=device)
    A = -torch.exp(torch.rand((H,), generator=g, **f32) * math.log(16.0))
    x = torch.randn((b, L, H, R, P), generator=g, **f32)
    B = torch.randn((b, L, H, R, N), generator=g, **f32) / math.sqrt(N)
    C = torch.randn((b, L, H, R, N), generator=g, **f32) / math.sqrt(N)
    dt = torch.nn.functional.softplus(torch.randn((b, L, H), generator=g, **f32) - 3.0)
    lam = _lam(g, (b, L, H), w.lam_dist, device)
    theta = None
    if w.rotation:
        u = (torch.rand((b, L, H, N // 2), generator=g, **f32) * 2.0 - 1.0) * math.pi
        theta = (dt.unsqueeze(-1) * u).contiguous()
    return dict(x=_cast(x, w), B=_cast(B, w), C=_cast(C, w), dt=dt.contiguous(),
                A=A.contiguous(), lam=lam.contiguous(), theta=theta)


def make_decode_step_inputs(w: Workload, g: torch.Generator, device="cpu") -> dict:
    """Draws one decode step's per-token tensors (x, B, C, dt, lam, theta)."""
    b, H, P, N, R = w.batch, w.nheads, w.headdim, w.dstate, w.rank
    f32 = dict(dtype=torch.float32, device=device)
    x = torch.randn((b, H, R, P), generator=g, **f32)
    B = torch.randn((b, H, R, N), generator=g, **f32) / math.sqrt(N)
    C = torch.randn((b, H, R, N), generator=g, **f32) / math.sqrt(N)
    dt = torch.nn.functional.softplus(torch.randn((b, H), generator=g, **f32) - 3.0)
    lam = _lam(g, (b, H), w.lam_dist, device)
    theta = None
    if w.rotation:
        u = (torch.rand((b, H, N // 2), generator=g, **f32) * 2.0 - 1.0) * math.pi
        theta = (dt.unsqueeze(-1) * u).contiguous()
    return dict(x=_cast(x, w), B=_cast(B, w), C=_cast(C, w), dt=dt.contiguous(),
                lam=lam.contiguous(), theta=theta)


def make_decode_inputs(w: Workload, seed: int = 0, device="cpu", steps: Optional[int] = None) -> dict:
    """Draws A once, then `steps` successive decode steps stacked on a leading axis.

    Returns dict(A=[H], x=[S,b,H,R,P], B=[S,b,H,R,N], C=..., dt=[S,b,H],
    lam=[S,b,H], theta=[S,b,H,N/2] or None).
    """
    S = w.steps if steps is None else steps
    g = _gen(seed, device)
    A = -torch.exp(torch.rand((w.nheads,), generator=g, dtype=torch.float32, device=device)
                   * math.log(16.0))
    per = [make_decode_step_inputs(w, g, device) for _ in range(S)]
    out = dict(A=A.contiguous())
    for k in ("x", "B", "C", "dt", "lam", "theta"):
        if per and per[0][k] is not None:
            out[k] = torch.stack([p[k] for p in per]).contiguous()
        else:
            out[k] = None
    return out


def random_carry(w: Workload, seed: int = 1, device="cpu", batch: Optional[int] = None) -> dict:
    """A random incoming carry (h0, B_prev, x_prev) for continuation tests."""
    b = w.batch if batch is None else batch
    H, P, N, R = w.nheads, w.headdim, w.dstate, w.rank
    g = _gen(seed, device)
    f32 = dict(dtype=torch.float32, device=device)
    h0 = torch.randn((b, H, N, P), generator=g, **f32) * 0.5
    Bp = torch.randn((b, H, R, N), generator=g, **f32) / math.sqrt(N)
    xp = torch.randn((b, H, R, P), generator=g, **f32)
    return dict(h0=h0.contiguous(), B_prev=_cast(Bp, w), x_prev=_cast(xp, w))
