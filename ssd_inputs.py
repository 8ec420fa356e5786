"""Seeded synthetic inputs for the Mamba-2 SSD forward pass.

This module is shared by the CPU oracle's tests and by the HIP path's tests
and benchmark.  It holds no part of the method's arithmetic: it only draws
random tensors with a fixed recipe.

Recipe (one CPU ``torch.Generator`` per draw, seed fixed per workload, draws
in this order, all drawn in float32 and then rounded to nearest-even into the
workload's dtype):

* ``x``, ``B``, ``C`` ~ N(0, 1)
* ``z`` ~ N(0, 1); ``u_bias`` ~ U(ln 1e-3, ln 1e-1) per head;
  ``dt_bias = softplus^-1(exp(u_bias))``; ``dt = softplus(0.5 z + dt_bias)``
  (dt is rounded to the workload dtype after the softplus)
* ``A = -exp(U(ln 1, ln 16))`` per head, float32
* ``D``: ones for the all-float32 workload, N(0, 1) float32 otherwise
* initial state: ``0.1 * N(0, 1)`` float32 where the workload has one

Softplus and the bias are part of how dt is produced, not of the forward
pass: the kernels receive dt as given.
"""
from __future__ import annotations

import dataclasses
import math

import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    seqlen: int
    nheads: int
    headdim: int
    dstate: int
    ngroups: int
    chunk_size: int
    dtype: str            # "f32" (every tensor float32) or "bf16" (x, dt, B, C, y bfloat16)
    d_ones: bool          # D = 1 (else N(0, 1))
    init_state: bool      # initial state drawn (else none)
    seed: int

    @property
    def nchunks(self) -> int:
        return -(-self.seqlen // self.chunk_size)

    @property
    def tokens(self) -> int:
        return self.batch * self.seqlen


# The five workloads of the pages' sweep (1K-256K tokens, state size 64-512),
# plus the tiny all-float32 case.
WORKLOADS = {
    w.name: w
    for w in (
        Workload("tiny_fp32_L256_N16", 1, 256, 2, 16, 16, 1, 64, "f32", True, False, 1000),
        Workload("small_L1k_N64", 1, 1024, 8, 64, 64, 1, 256, "bf16", False, True, 1001),
        Workload("mid_L8k_N128", 2, 8192, 24, 64, 128, 1, 256, "bf16", False, False, 1002),
        Workload("long_L64k_N256", 1, 65536, 32, 64, 256, 1, 256, "bf16", False, False, 1003),
        Workload("longest_L256k_N512", 1, 262144, 32, 64, 512, 4, 256, "bf16", False, False, 1004),
    )
}
WORKLOAD_ORDER = list(WORKLOADS)


def custom(name="custom", *, batch=1, seqlen=256, nheads=2, headdim=16, dstate=16, ngroups=1,
           chunk_size=64, dtype="bf16", d_ones=False, init_state=False, seed=7) -> Workload:
    return Workload(name, batch, seqlen, nheads, headdim, dstate, ngroups, chunk_size, dtype,
                    d_ones, init_state, seed)


def _softplus(v: torch.Tensor) -> torch.Tensor:
    return torch.nn.functional.softplus(v)


def _inv_softplus(v: torch.Tensor) -> torch.Tensor:
    # softplus^-1(y) = y + log(-expm1(-y))
    return v + torch.log(-torch.expm1(-v))


def make_inputs(w: Workload) -> dict:
    """Draws the workload's tensors on the CPU.

    Returns a dict with ``x[B,L,H,P]``, ``dt[B,L,H]``, ``A[H]``, ``B[B,L,G,N]``,
    ``C[B,L,G,N]``, ``D[H]`` and ``init_state[B,H,P,N]`` (or None).
    """
    g = torch.Generator(device="cpu")
    g.manual_seed(w.seed)
    Bn, L, H, P, N, G = w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.ngroups
    io = torch.float32 if w.dtype == "f32" else torch.bfloat16
    x = torch.randn((Bn, L, H, P), generator=g, dtype=torch.float32).to(io)
    B = torch.randn((Bn, L, G, N), generator=g, dtype=torch.float32).to(io)
    C = torch.randn((Bn, L, G, N), generator=g, dtype=torch.float32).to(io)
    z = torch.randn((Bn, L, H), generator=g, dtype=torch.float32)
    u_bias = torch.rand((H,), generator=g, dtype=torch.float32)
    u_bias = math.log(1e-3) + (math.log(1e-1) - math.log(1e-3)) * u_bias
    dt_bias = _inv_softplus(torch.exp(u_bias))
    dt = _softplus(0.5 * z + dt_bias).to(io)
    del z
    u_A = torch.rand((H,), generator=g, dtype=torch.float32)
    A = -torch.exp(math.log(16.0) * u_A)
    if w.d_ones:
        D = torch.ones((H,), dtype=torch.float32)
    else:
        D = torch.randn((H,), generator=g, dtype=torch.float32)
    h0 = None
    if w.init_state:
        h0 = 0.1 * torch.randn((Bn, H, P, N), generator=g, dtype=torch.float32)
    return {"x": x, "dt": dt, "A": A.contiguous(), "B": B, "C": C, "D": D, "init_state": h0}


def make_cotangents(w: Workload) -> dict:
    """Seeded upstream gradients for the backward pass: ``dy[B,L,H,P]`` in the
    workload's dtype and ``dfinal[B,H,P,N]`` float32, both standard normal
    (their own stream, seed + 1000003, so the forward inputs are unchanged)."""
    g = torch.Generator(device="cpu")
    g.manual_seed(w.seed + 1000003)
    io = torch.float32 if w.dtype == "f32" else torch.bfloat16
    dy = torch.randn((w.batch, w.seqlen, w.nheads, w.headdim), generator=g,
                     dtype=torch.float32).to(io)
    dfinal = torch.randn((w.batch, w.nheads, w.headdim, w.dstate), generator=g,
                         dtype=torch.float32)
    return {"dy": dy, "dfinal": dfinal}
