"""GPU parity of dL/dbeta (the inverse temperature the pages train: corner
logits beta * u . v_r) against the fp64 oracle.

The bar is the one of every gradient: |dbeta - ref| <= tol * |ref| (tol 1e-5
for fp32 I/O, 2e-2 for bf16 I/O).  dbeta sums one term per token, side,
head and table; with an upstream gradient dO drawn independently of O those
terms have random signs and their sum is a small remainder of large parts
(|ref| / sum |terms| about 1e-2), so the test takes dO = O (the oracle's
output rounded to the I/O dtype: the gradient of sum |O|^2 / 2), whose terms
mostly share a sign (|ref| / sum |terms| between 0.47 and 1 in these cases).
The scale sum |terms| is printed beside the error.  Two runs must give the
same bits (the per-wave shares are summed in a fixed order).
"""
from dataclasses import replace

import numpy as np
import pytest
import torch

import race_inputs as ri
from oracle import race_oracle as orc
from parity_util import TOL, say, to64

pytestmark = pytest.mark.gpu

race = pytest.importorskip("linear_attention_soft_amd")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    race.lib()


def _ref(inp, w, dO):
    Q, K, V = (to64(inp[k]) for k in ("Q", "K", "V"))
    Wn = inp["W"].double().numpy()
    tot, scale = 0.0, 0.0
    for b in range(w.B):
        for h in range(w.H):
            tq, tk = orc.dbeta_head(Q[b, h], K[b, h], V[b, h], Wn, w.beta, dO[b, h], w.causal)
            tot += float(tq.sum() + tk.sum())
            scale += float(np.abs(tq).sum() + np.abs(tk).sum())
    return tot, scale


@pytest.mark.parametrize("key,N,B,H,dtype,causal,give_o", [
    (1, 700, 1, 1, "f32", False, False),
    (3, 3000, 2, 2, "bf16", False, False),
    (4, 4000, 1, 2, "bf16", False, False),
    (5, 2500, 1, 2, "bf16", False, False),
    (2, 600, 1, 2, "f32", True, False),
    (2, 600, 1, 2, "f32", True, True),
    (5, 1100, 1, 2, "bf16", True, True),
    (4, 1500, 1, 2, "bf16", True, False),
])
def test_dbeta_parity(key, N, B, H, dtype, causal, give_o):
    w = replace(ri.WORKLOADS[key].with_size(N=N, B=B, H=H), causal=causal, dtype=dtype)
    inp = ri.make_inputs(w, device="cpu", with_grad_out=False)
    # upstream gradient dO = O from the oracle, rounded to the I/O dtype
    Wn = inp["W"].double().numpy()
    O_ref = orc.forward(to64(inp["Q"]), to64(inp["K"]), to64(inp["V"]), Wn, w.beta, causal)
    inp["dO"] = torch.from_numpy(O_ref).to(inp["Q"].dtype)
    dev = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    say(f"dbeta key={key} N={N} B={B} H={H} {dtype} causal={causal} O given={give_o} P={w.P} L={w.L} beta={w.beta}")
    O, state = race.race_attn_fwd(dev["Q"], dev["K"], dev["V"], dev["W"], w.beta, w.P, w.L, causal)
    got = []
    for _ in range(2):
        *_, db = race.race_attn_bwd(dev["Q"], dev["K"], dev["V"], dev["W"], w.beta, w.P, w.L, causal, dev["dO"],
                                    state, O=O if give_o else None, dbeta=True)
        torch.cuda.synchronize()
        got.append(db.cpu())
    assert torch.equal(got[0], got[1]), "dbeta differs between two runs"
    ref, scale = _ref(inp, w, to64(inp["dO"]))
    err = abs(float(got[0][0]) - ref)
    say(f"  dbeta gpu {float(got[0][0]):.6e} ref {ref:.6e} |err| {err:.3e} |err|/|ref| {err / abs(ref):.3e} "
        f"(sum |terms| {scale:.3e}, |ref|/sum {abs(ref) / scale:.3f}) tol {TOL[dtype]:g}")
    assert abs(ref) >= 0.3 * scale, "case chosen so that dbeta is not a small remainder"
    assert err <= TOL[dtype] * abs(ref)


def test_dbeta_absent_leaves_gradients_unchanged():
    """Asking for dbeta does not change dQ, dK, dV (bitwise)."""
    w = replace(ri.WORKLOADS[5].with_size(N=1100, B=1, H=2), causal=True, dtype="bf16")
    inp = ri.make_inputs(w, device="cuda", with_grad_out=True)
    Wd = inp["W"].cuda()
    O, st = race.race_attn_fwd(inp["Q"], inp["K"], inp["V"], Wd, w.beta, w.P, w.L, True)
    a = race.race_attn_bwd(inp["Q"], inp["K"], inp["V"], Wd, w.beta, w.P, w.L, True, inp["dO"], st, O=O)
    b = race.race_attn_bwd(inp["Q"], inp["K"], inp["V"], Wd, w.beta, w.P, w.L, True, inp["dO"], st, O=O, dbeta=True)
    torch.cuda.synchronize()
    for x, y in zip(a, b[:3]):
        assert torch.equal(x, y)
