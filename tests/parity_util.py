"""Shared helpers of the GPU parity tests (oracle side + comparison)."""
import sys

import numpy as np
import torch

from oracle import race_oracle as orc

TOL = {"f32": 1e-5, "bf16": 2e-2}


def to64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to(torch.float64).cpu().numpy()


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def max_rel(x: np.ndarray, ref: np.ndarray) -> float:
    den = np.abs(ref).max()
    return float(np.abs(x - ref).max() / (den if den > 0 else 1.0))


def check(name, got: torch.Tensor, ref: np.ndarray, tol: float, vmax: float | None = None):
    """max|got - ref| <= tol * max|ref| (and <= tol * vmax when given)."""
    g = to64(got)
    assert np.all(np.isfinite(g)), f"{name}: non-finite values"
    err = float(np.abs(g - ref).max())
    rel = err / max(np.abs(ref).max(), 1e-300)
    say(f"  {name}: max|err|={err:.3e} rel_to_max|ref|={rel:.3e} tol={tol:g}")
    assert rel <= tol, f"{name}: {rel:.3e} > {tol}"
    if vmax is not None:
        assert err <= tol * vmax, f"{name}: {err:.3e} > {tol} * max|V| = {tol * vmax:.3e}"


def oracle_fwd(inp, causal):
    Q, K, V = (to64(inp[k]) for k in ("Q", "K", "V"))
    return orc.forward(Q, K, V, inp["W"].double().numpy(), inp["beta"], causal)


def oracle_bwd(inp, causal):
    Q, K, V, dO = (to64(inp[k]) for k in ("Q", "K", "V", "dO"))
    return orc.backward(Q, K, V, inp["W"].double().numpy(), inp["beta"], dO, causal)
