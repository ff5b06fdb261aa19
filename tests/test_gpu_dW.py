"""GPU parity of the table gradient dL/dW and of per-head tables against
the fp64 oracle.

The pre-activations of a row x are W^(l) x (slides, frame "Soft corner
assignments make hashing differentiable"), so dW^(l) sums dL/dPre^(l) x^T
over the query and key rows of every batch row and head that use the table.
dW is compared per tensor like the other gradients: max|dW - ref| <= tol *
max|ref| (tol 1e-5 for fp32 I/O, 2e-2 for bf16 I/O).  Per-head tables
([H][L][P][d]) are also checked on O, dQ, dK, dV and on the recurrent
decode.  Two runs give the same bits (fixed-order sums), and asking for dW
leaves dQ, dK, dV unchanged.
"""
from dataclasses import replace

import numpy as np
import pytest
import torch

import race_inputs as ri
from oracle import race_oracle as orc
from parity_util import TOL, check, say, to64

pytestmark = pytest.mark.gpu

race = pytest.importorskip("linear_attention_soft_amd")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    race.lib()


def _inputs(w, per_head):
    inp = ri.make_inputs(w, device="cpu", with_grad_out=True)
    if per_head:
        inp["W"] = ri.make_W_per_head(w)
    return inp


@pytest.mark.parametrize("key,N,B,H,dtype,causal,per_head", [
    (1, 700, 1, 1, "f32", False, False),
    (1, 900, 2, 3, "f32", False, True),
    (3, 3000, 2, 2, "bf16", False, True),
    (4, 1500, 1, 2, "bf16", False, False),
    (2, 600, 1, 2, "f32", True, False),
    (2, 650, 2, 2, "f32", True, True),
    (5, 1100, 1, 2, "bf16", True, True),
    (5, 1553, 1, 1, "bf16", True, False),
    (5, 1200, 1, 2, "bf16", False, True),
])
def test_dW_parity(key, N, B, H, dtype, causal, per_head):
    w = replace(ri.WORKLOADS[key].with_size(N=N, B=B, H=H), causal=causal, dtype=dtype)
    inp = _inputs(w, per_head)
    dev = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    say(f"dW key={key} N={N} B={B} H={H} {dtype} causal={causal} per_head={per_head} P={w.P} L={w.L} beta={w.beta}")
    O, state = race.race_attn_fwd(dev["Q"], dev["K"], dev["V"], dev["W"], w.beta, w.P, w.L, causal)
    runs = []
    for _ in range(2):
        g = race.race_attn_bwd(dev["Q"], dev["K"], dev["V"], dev["W"], w.beta, w.P, w.L, causal, dev["dO"], state,
                               O=O if causal else None, dW=True)
        torch.cuda.synchronize()
        runs.append([t.cpu() for t in g])
    assert torch.equal(runs[0][3], runs[1][3]), "dW differs between two runs"
    plain = race.race_attn_bwd(dev["Q"], dev["K"], dev["V"], dev["W"], w.beta, w.P, w.L, causal, dev["dO"], state,
                               O=O if causal else None)
    torch.cuda.synchronize()
    for x, y in zip(plain, runs[0][:3]):
        assert torch.equal(x.cpu(), y), "asking for dW changed dQ, dK or dV"
    Q, K, V, dO = (to64(inp[k]) for k in ("Q", "K", "V", "dO"))
    Wn = inp["W"].double().numpy()
    tol = TOL[dtype]
    check("dW", runs[0][3], orc.dW(Q, K, V, Wn, w.beta, dO, causal), tol)
    if per_head:
        check("O", O, orc.forward(Q, K, V, Wn, w.beta, causal), tol, float(np.abs(V).max()))
        for name, got, ref in zip(("dQ", "dK", "dV"), runs[0][:3], orc.backward(Q, K, V, Wn, w.beta, dO, causal)):
            check(name, got, ref, tol)


def test_per_head_tables_that_are_equal_match_shared_tables():
    """[H][L][P][d] tables that repeat one [L][P][d] set give the shared-table
    O, dQ, dK, dV bit for bit, and a dW whose sum over heads is the
    shared-table dW."""
    w = replace(ri.WORKLOADS[4].with_size(N=2100, B=2, H=2), causal=False, dtype="bf16")
    inp = ri.make_inputs(w, device="cuda", with_grad_out=True)
    W3 = inp["W"].cuda()
    W4 = W3.unsqueeze(0).repeat(w.H, 1, 1, 1).contiguous()
    for causal in (False, True):
        say(f"per-head equal tables causal={causal}")
        outs = []
        for Wd in (W3, W4):
            O, st = race.race_attn_fwd(inp["Q"], inp["K"], inp["V"], Wd, w.beta, w.P, w.L, causal)
            g = race.race_attn_bwd(inp["Q"], inp["K"], inp["V"], Wd, w.beta, w.P, w.L, causal, inp["dO"], st,
                                   O=O if causal else None, dW=True)
            torch.cuda.synchronize()
            outs.append((O,) + tuple(g))
        for a, b in zip(outs[0][:4], outs[1][:4]):
            assert torch.equal(a, b)
        s = outs[1][4].sum(dim=0).double()
        ref = outs[0][4].double()
        assert float((s - ref).abs().max()) <= 1e-5 * float(ref.abs().max())


def test_decode_with_per_head_tables():
    """Prefill and decode with per-head tables equal the oracle's causal
    forward of the whole sequence on the decoded rows."""
    w = replace(ri.WORKLOADS[2].with_size(N=700, B=1, H=3), causal=True, dtype="f32")
    inp = _inputs(w, True)
    n0 = 650
    dev = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    say(f"decode per-head tables N={w.N} prompt={n0}")
    st = race.race_attn_decode_prefill(dev["K"][:, :, :n0].contiguous(), dev["V"][:, :, :n0].contiguous(),
                                       dev["W"], w.beta, w.P, w.L)
    O = race.race_attn_decode(dev["Q"][:, :, n0:].contiguous(), dev["K"][:, :, n0:].contiguous(),
                              dev["V"][:, :, n0:].contiguous(), dev["W"], w.beta, w.P, w.L, st)
    torch.cuda.synchronize()
    Q, K, V = (to64(inp[k]) for k in ("Q", "K", "V"))
    ref = orc.forward(Q, K, V, inp["W"].double().numpy(), w.beta, True)[:, :, n0:]
    check("O decode", O, ref, TOL["f32"], float(np.abs(V).max()))


@pytest.mark.parametrize("causal", [False, True])
def test_dW_edge_cases(causal):
    """Two tokens, a ragged length of one tile plus a few rows, one token
    (the layer returns V whatever the assignments are, so dW = 0 up to the
    float32 rounding of terms that cancel) and beta = 0 (uniform assignments
    whatever W is: dW is exactly zero)."""
    for key, N, B, H, dtype, beta in [(1, 2, 1, 2, "f32", None), (2, 131, 2, 1, "f32", None),
                                       (5, 67, 1, 1, "bf16", None), (1, 1, 1, 2, "f32", None),
                                       (1, 300, 1, 1, "f32", 0.0)]:
        w = replace(ri.WORKLOADS[key].with_size(N=N, B=B, H=H), causal=causal, dtype=dtype)
        if beta is not None:
            w = replace(w, beta=beta)
        inp = _inputs(w, per_head=(B > 1))
        dev = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
        say(f"dW edge key={key} N={N} B={B} H={H} {dtype} causal={causal} beta={w.beta}")
        O, state = race.race_attn_fwd(dev["Q"], dev["K"], dev["V"], dev["W"], w.beta, w.P, w.L, causal)
        *_, dW = race.race_attn_bwd(dev["Q"], dev["K"], dev["V"], dev["W"], w.beta, w.P, w.L, causal, dev["dO"],
                                    state, O=O if causal else None, dW=True)
        torch.cuda.synchronize()
        if w.beta == 0.0:
            assert float(dW.abs().max()) == 0.0
            continue
        if N == 1:
            scale = w.beta * float(inp["dO"].abs().max() * inp["V"].abs().max()
                                   * torch.maximum(inp["Q"].abs().max(), inp["K"].abs().max()))
            say(f"  one token: max|dW| {float(dW.abs().max()):.3e}, cancelling-term scale {scale:.3e}")
            assert float(dW.abs().max()) <= 1e-5 * scale
            continue
        Q, K, V, dO = (to64(inp[k]) for k in ("Q", "K", "V", "dO"))
        check("dW", dW, orc.dW(Q, K, V, inp["W"].double().numpy(), w.beta, dO, causal), TOL[dtype])
