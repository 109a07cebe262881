"""Seeded synthetic workloads for the selective-scan forward pass.

This module only draws random inputs; it holds none of the scan's arithmetic
and is shared by the tests, the smoke check and the benchmark (both the GPU
path and the CPU oracle see exactly the tensors it returns).

Five workloads, by name:

  tiny    b=1  d=64   n=16 L=256    float32, gated, D ~ N(0,1),
          raw delta ~ N(0,1) with delta_bias = -2 and softplus on.
  130m    b=8  d=1536 n=16 L=2048   float32, gated, D = 1, softplus on,
          delta_bias[d] = log(expm1(dt0[d])), dt0 ~ U[1e-3, 1e-1]
          (the Mamba-130m layer shape: d_model 768, expand 2).
  1.4b    b=8  d=4096 n=16 L=2048   bfloat16 u/delta/B/C/z/y, float32 A, D,
          bias and state; otherwise as 130m.
  long    b=1  d=2048 n=16 L=65536  float32, no gate, no D, delta_bias = -4
          (slow decay), softplus on.
  varlen  b=16 d=5120 n=16 L=8192   bfloat16 I/O as 1.4b, per-row lengths
          ~ U{512..8192}; steps past a row's length are identity steps: raw
          delta = -inf there, so softplus(-inf + bias) = 0 exactly and
          a = exp(0) = 1, b = 0.

Every workload: u, z ~ N(0,1) [b,d,L]; A[d,n] = -(n+1) (S4D-real); B, C ~
N(0,1) [b,n,L].  Draw order with one torch.Generator seeded with ``seed``
(default 0) on ``device``: u, delta, z, B, C, D, dt0 (bias), lengths.
Values are drawn in float32 and cast to bfloat16 (round to nearest even)
where the workload stores bfloat16.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, replace
from typing import Dict, Optional

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    dim: int
    dstate: int
    L: int
    dtype: str            # "f32" or "bf16": storage of u, delta, B, C, z, y
    gated: bool           # z present
    D_kind: Optional[str] # None, "normal" or "ones"
    bias_kind: str        # "const" or "dt_init"
    bias_value: float = 0.0
    softplus: bool = True
    varlen: bool = False

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    def with_sizes(self, **kw) -> "Workload":
        """Same recipe at other sizes (batch, dim, dstate, L)."""
        return replace(self, **kw)

    # Bytes the method must move at minimum: every input element once, y and
    # last_state once (no (a, b) pairs and no per-step states).
    def algorithmic_bytes(self) -> int:
        s = 4 if self.dtype == "f32" else 2
        g = 1 if self.gated else 0
        per_ch = self.L * (s + s + g * s + s)        # u, delta, z, y
        bc = 2 * self.batch * self.dstate * self.L * s
        params = 4 * self.dim * self.dstate + 4 * self.dim * (int(self.D_kind is not None) +
                                                              int(self.bias_kind is not None))
        last = 4 * self.batch * self.dim * self.dstate
        return self.batch * self.dim * per_ch + bc + params + last

    def state_steps(self) -> int:
        return self.batch * self.dim * self.dstate * self.L


WORKLOADS: Dict[str, Workload] = {
    "tiny": Workload("tiny", 1, 64, 16, 256, "f32", True, "normal", "const", -2.0),
    "130m": Workload("130m", 8, 1536, 16, 2048, "f32", True, "ones", "dt_init"),
    "1.4b": Workload("1.4b", 8, 4096, 16, 2048, "bf16", True, "ones", "dt_init"),
    "long": Workload("long", 1, 2048, 16, 65536, "f32", False, None, "const", -4.0),
    "varlen": Workload("varlen", 16, 5120, 16, 8192, "bf16", True, "ones", "dt_init", varlen=True),
}


def make_inputs(w: Workload, device="cpu", seed: int = 0) -> dict:
    """Draw the inputs of workload ``w`` on ``device``.

    Returns a dict with u, delta, z (or None), A, B, C, D (or None),
    delta_bias, delta_softplus, lengths (varlen only, int64 [b]) and the
    workload itself under "workload".
    """
    dev = torch.device(device)
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    b, d, n, L = w.batch, w.dim, w.dstate, w.L
    f32 = dict(device=dev, dtype=torch.float32)
    u = torch.randn((b, d, L), generator=g, **f32)
    delta = torch.randn((b, d, L), generator=g, **f32)
    z = torch.randn((b, d, L), generator=g, **f32) if w.gated else None
    B = torch.randn((b, n, L), generator=g, **f32)
    C = torch.randn((b, n, L), generator=g, **f32)
    if w.D_kind == "normal":
        D = torch.randn((d,), generator=g, **f32)
    elif w.D_kind == "ones":
        D = torch.ones((d,), **f32)
    else:
        D = None
    if w.bias_kind == "const":
        delta_bias = torch.full((d,), w.bias_value, **f32)
    else:
        # Mamba's dt initialisation: dt0 ~ U[1e-3, 1e-1], bias = log(expm1(dt0)),
        # evaluated in float64 (log(-expm1(-x)) + x is the stable form).
        dt0 = torch.rand((d,), generator=g, **f32).to(torch.float64) * (0.1 - 1e-3) + 1e-3
        delta_bias = (dt0 + torch.log(-torch.expm1(-dt0))).to(torch.float32)
    lengths = None
    if w.varlen:
        lengths = torch.randint(512, L + 1, (b,), generator=g, device=dev, dtype=torch.int64)
        t = torch.arange(L, device=dev)[None, None, :]
        pad = t >= lengths[:, None, None]
        delta = torch.where(pad, torch.full_like(delta, -math.inf), delta)
    A = -torch.arange(1, n + 1, **f32)[None, :].expand(d, n).contiguous()
    cast = w.torch_dtype
    out = dict(
        u=u.to(cast).contiguous(),
        delta=delta.to(cast).contiguous(),
        z=None if z is None else z.to(cast).contiguous(),
        A=A,
        B=B.to(cast).contiguous(),
        C=C.to(cast).contiguous(),
        D=D,
        delta_bias=delta_bias,
        delta_softplus=w.softplus,
        lengths=lengths,
        workload=w,
    )
    return out


def random_A(d: int, n: int, device="cpu", seed: int = 1) -> torch.Tensor:
    """A random negative A[d, n] = -exp(N(0,1)) (not the S4D-real pattern),
    for tests that must not depend on A's structure."""
    g = torch.Generator(device=torch.device(device))
    g.manual_seed(seed)
    return -torch.exp(torch.randn((d, n), generator=g, device=device, dtype=torch.float32))


def make_grads(w: Workload, device="cpu", seed: int = 0) -> dict:
    """Incoming gradients for the backward pass of workload ``w``: dy ~ N(0,1)
    [b, d, L] in the workload's storage type and dlast ~ N(0,1) [b, d, n]
    float32, drawn in that order with a generator seeded with ``seed + 1000``
    (so that they do not repeat the input draws)."""
    dev = torch.device(device)
    g = torch.Generator(device=dev)
    g.manual_seed(seed + 1000)
    f32 = dict(device=dev, dtype=torch.float32)
    dy = torch.randn((w.batch, w.dim, w.L), generator=g, **f32).to(w.torch_dtype).contiguous()
    dlast = torch.randn((w.batch, w.dim, w.dstate), generator=g, **f32)
    return dict(dy=dy, dlast=dlast)


def d_model_of(w: Workload) -> int:
    """Model width of workload ``w``'s layer: d_inner / 2 (Mamba's expand = 2;
    768 for 130m, 2048 for 1.4b)."""
    return w.dim // 2


def make_proj_inputs(batch: int, d_inner: int, d_model: int, L: int, dtype=torch.float32, device="cpu",
                     seed: int = 0) -> dict:
    """Inputs of the output projection: y ~ N(0,1) [batch, d_inner, L] (the
    scan's output layout) and W ~ N(0,1)/sqrt(d_inner) [d_model, d_inner] (a
    Linear weight at its usual scale), drawn in that order in float32 with a
    generator seeded with ``seed + 2000`` and cast to ``dtype``."""
    dev = torch.device(device)
    g = torch.Generator(device=dev)
    g.manual_seed(seed + 2000)
    f32 = dict(device=dev, dtype=torch.float32)
    y = torch.randn((batch, d_inner, L), generator=g, **f32).to(dtype).contiguous()
    W = (torch.randn((d_model, d_inner), generator=g, **f32) / math.sqrt(d_inner)).to(dtype).contiguous()
    return dict(y=y, W=W)
