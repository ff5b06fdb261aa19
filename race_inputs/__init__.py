"""Seeded synthetic inputs for the RACE attention workloads.

This module only draws random numbers and holds the workload table; it
contains none of the method's arithmetic.  Both the fp64 oracle side (tests,
CPU baseline) and the HIP side (tests, benchmark, smoke check) take their
inputs from here, so the two never feed each other.

Shapes follow the pages' workloads: the single-layer scaling runs (batch 1,
4 heads, head dim 128; "RACE Attention" slides, frame "The GPU operator
reaches 12M tokens at a small budget") and the language-model and
long-classification task shapes (slides backup frame "task models differ from
the scaling operator").  Each tensor has its own sub-seed
1000 * config + {Q: 1, K: 2, V: 3, dO: 4, W: 5, per-head W: 6}.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, replace

import torch


@dataclass(frozen=True)
class Workload:
    key: int
    name: str
    B: int
    H: int
    N: int
    d: int
    P: int
    L: int
    beta: float
    causal: bool
    dtype: str          # "f32" or "bf16"
    phases: tuple       # ("fwd",) or ("fwd", "bwd")
    dist: str           # value-distribution recipe, see make_inputs

    @property
    def R(self) -> int:
        return 1 << self.P

    def with_size(self, N=None, B=None, H=None) -> "Workload":
        return replace(self, N=self.N if N is None else N,
                       B=self.B if B is None else B, H=self.H if H is None else H)


WORKLOADS = {
    1: Workload(1, "noncausal_fwd_f32_n1k", 1, 1, 1024, 64, 3, 2, 1.0, False, "f32", ("fwd",), "iid"),
    2: Workload(2, "causal_fwd_lm_b8h8_n1k", 8, 8, 1024, 64, 4, 4, 2.0, True, "bf16", ("fwd",), "iid_over_sqrt_d"),
    3: Workload(3, "noncausal_fwdbwd_cls_b2h4_n64k", 2, 4, 65536, 64, 3, 3, 4.0, False, "bf16",
                ("fwd", "bwd"), "lognormal_norms"),
    4: Workload(4, "noncausal_fwdbwd_h4_n12m_d128", 1, 4, 12_000_000, 128, 4, 2, 4.0, False, "bf16",
                ("fwd", "bwd"), "iid"),
    5: Workload(5, "causal_fwdbwd_h4_n1m_d128_p6l4", 1, 4, 1_048_576, 128, 6, 4, 8.0, True, "bf16",
                ("fwd", "bwd"), "clustered_keys"),
}


def torch_dtype(name: str):
    return {"f32": torch.float32, "bf16": torch.bfloat16}[name]


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def _randn(shape, seed, device):
    return torch.randn(shape, generator=_gen(seed, device), device=device, dtype=torch.float32)


def _lognormal_rows(shape, seed, device):
    """Rows with an isotropic direction and a norm drawn log-uniform in [0.5, 2]."""
    g = _gen(seed, device)
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    x = x / x.norm(dim=-1, keepdim=True)
    u = torch.rand(shape[:-1] + (1,), generator=g, device=device, dtype=torch.float32)
    lo, hi = math.log(0.5), math.log(2.0)
    return x * torch.exp(lo + (hi - lo) * u)


def _clustered_rows(shape, seed, device, n_centroids=256, noise=0.3):
    """Rows = one of 256 random unit centroids per (b, h), chosen uniformly,
    plus per-coordinate N(0, noise^2) noise."""
    B, H, N, d = shape
    g = _gen(seed, device)
    cent = torch.randn((B, H, n_centroids, d), generator=g, device=device, dtype=torch.float32)
    cent = cent / cent.norm(dim=-1, keepdim=True)
    idx = torch.randint(0, n_centroids, (B, H, N), generator=g, device=device)
    out = torch.empty(shape, device=device, dtype=torch.float32)
    step = 1 << 20
    for b in range(B):
        for h in range(H):
            for t0 in range(0, N, step):
                t1 = min(N, t0 + step)
                n = torch.randn((t1 - t0, d), generator=g, device=device, dtype=torch.float32)
                out[b, h, t0:t1] = cent[b, h][idx[b, h, t0:t1]] + noise * n
    return out


def _draw(dist, shape, seed, device, role):
    if dist == "iid" or role in ("dO",):
        return _randn(shape, seed, device)
    if dist == "iid_over_sqrt_d":
        return _randn(shape, seed, device) / math.sqrt(shape[-1])
    if dist == "lognormal_norms":
        return _lognormal_rows(shape, seed, device)
    if dist == "clustered_keys":
        if role == "K":
            return _clustered_rows(shape, seed, device)
        return _randn(shape, seed, device)
    raise ValueError(dist)


def make_W(w: Workload, seed_base: int | None = None) -> torch.Tensor:
    """Gaussian projection W[L][P][d], iid N(0, 1), float32, on the CPU."""
    base = 1000 * w.key if seed_base is None else seed_base
    return _randn((w.L, w.P, w.d), base + 5, "cpu")


def make_W_per_head(w: Workload, seed_base: int | None = None) -> torch.Tensor:
    """One set of Gaussian tables per head, W[H][L][P][d], iid N(0, 1),
    float32, on the CPU."""
    base = 1000 * w.key if seed_base is None else seed_base
    return _randn((w.H, w.L, w.P, w.d), base + 6, "cpu")


def make_inputs(w: Workload, device="cpu", seed_base: int | None = None,
                with_grad_out: bool | None = None) -> dict:
    """Seeded Q, K, V (and dO for backward workloads) in the workload's I/O dtype,
    shape (B, H, N, d), on ``device``; W as float32 (L, P, d) on the CPU.

    Large tensors are drawn in float32 chunks per tensor and cast to the I/O
    dtype (round-to-nearest-even), so device memory stays at one tensor of
    float32 scratch per draw.
    """
    base = 1000 * w.key if seed_base is None else seed_base
    shape = (w.B, w.H, w.N, w.d)
    dt = torch_dtype(w.dtype)
    out = {}
    roles = ["Q", "K", "V"]
    if with_grad_out if with_grad_out is not None else ("bwd" in w.phases):
        roles.append("dO")
    sub = {"Q": 1, "K": 2, "V": 3, "dO": 4}
    for r in roles:
        x = _draw(w.dist, shape, base + sub[r], device, r)
        out[r] = x.to(dt)
        del x
    out["W"] = make_W(w, seed_base)
    out["beta"] = float(w.beta)
    return out
