"""GPU parity at head dims between the compiled ones (a multiple of 8 up to
128), against the fp64 oracle.

Such a d runs on the kernels of the next compiled head dim D (64 or 128):
the library pads the token rows with zero columns in the workspace, reads W
with the caller's row pitch (columns past d read as zero) and copies the
outputs back, so the result is the layer at d (zero columns add nothing to a
projection and give zero output columns).  The decode kernel and the
soft-assignment export take the caller's row pitch directly.  Tolerances as
in the other parity tests: 1e-5 (fp32 I/O) or 2e-2 (bf16 I/O) of each
output's largest reference magnitude.
"""
from dataclasses import replace

import numpy as np
import pytest
import torch

import race_inputs as ri
from oracle import race_oracle as orc
from parity_util import TOL, check, oracle_bwd, oracle_fwd, say, to64

pytestmark = pytest.mark.gpu

race = pytest.importorskip("linear_attention_soft_amd")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    race.lib()


def _case(key, d, N, B, H, dtype, causal, P=None, L=None, seed=None):
    w = replace(ri.WORKLOADS[key].with_size(N=N, B=B, H=H), d=d, dtype=dtype, causal=causal)
    if P is not None:
        w = replace(w, P=P, L=L)
    inp = ri.make_inputs(w, device="cpu", seed_base=seed, with_grad_out=True)
    dev = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    return w, inp, dev


# (workload key for the value recipe, d, N, B, H, dtype, causal, P, L)
CASES = [
    (4, 96, 3000, 1, 2, "bf16", False, 4, 2),
    (4, 96, 2100, 1, 2, "bf16", True, 4, 2),
    (1, 40, 1500, 2, 1, "f32", False, 3, 2),
    (2, 40, 900, 1, 2, "f32", True, 4, 4),
    (5, 120, 2200, 1, 2, "bf16", True, 6, 4),
    (5, 120, 2600, 1, 2, "bf16", False, 6, 4),
    (3, 8, 1300, 1, 2, "bf16", False, 3, 3),
    (2, 72, 1000, 1, 2, "f32", False, 4, 2),
]


@pytest.mark.parametrize("key,d,N,B,H,dtype,causal,P,L", CASES)
def test_head_dim_parity(key, d, N, B, H, dtype, causal, P, L):
    w, inp, dev = _case(key, d, N, B, H, dtype, causal, P, L)
    say(f"d={d} key={key} N={N} B={B} H={H} {dtype} causal={causal} P={P} L={L} beta={w.beta}")
    O, state = race.race_attn_fwd(dev["Q"], dev["K"], dev["V"], dev["W"], w.beta, P, L, causal)
    dQ, dK, dV = race.race_attn_bwd(dev["Q"], dev["K"], dev["V"], dev["W"], w.beta, P, L, causal, dev["dO"],
                                    state, O=O if causal else None)
    torch.cuda.synchronize()
    assert O.shape == (B, H, N, d) and dQ.shape == (B, H, N, d)
    tol = TOL[dtype]
    check("O", O, oracle_fwd(inp, causal), tol, vmax=float(np.abs(to64(inp["V"])).max()))
    rdQ, rdK, rdV = oracle_bwd(inp, causal)
    check("dQ", dQ, rdQ, tol)
    check("dK", dK, rdK, tol)
    check("dV", dV, rdV, tol)


@pytest.mark.parametrize("key,d,N,dtype,causal,P,L", [(4, 96, 2100, "bf16", True, 4, 2),
                                                      (5, 120, 2600, "bf16", False, 6, 4),
                                                      (1, 40, 1500, "f32", False, 3, 2)])
def test_head_dim_dbeta(key, d, N, dtype, causal, P, L):
    """dbeta with the upstream gradient dO = O (the oracle's, rounded to the
    I/O dtype), so that dbeta is not a small remainder of cancelling
    per-token terms; bar tol * |ref|."""
    w, inp, _ = _case(key, d, N, 1, 2, dtype, causal, P, L)
    Q, K, V = (to64(inp[k]) for k in ("Q", "K", "V"))
    Wn = inp["W"].double().numpy()
    inp["dO"] = torch.from_numpy(orc.forward(Q, K, V, Wn, w.beta, causal)).to(inp["Q"].dtype)
    dev = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    O, state = race.race_attn_fwd(dev["Q"], dev["K"], dev["V"], dev["W"], w.beta, P, L, causal)
    *_, db = race.race_attn_bwd(dev["Q"], dev["K"], dev["V"], dev["W"], w.beta, P, L, causal, dev["dO"], state,
                                O=O if causal else None, dbeta=True)
    torch.cuda.synchronize()
    dO = to64(inp["dO"])
    ref, scale = 0.0, 0.0
    for h in range(2):
        tq, tk = orc.dbeta_head(Q[0, h], K[0, h], V[0, h], Wn, w.beta, dO[0, h], causal)
        ref += float(tq.sum() + tk.sum())
        scale += float(np.abs(tq).sum() + np.abs(tk).sum())
    err = abs(float(db[0]) - ref)
    say(f"d={d} dbeta gpu {float(db[0]):.6e} ref {ref:.6e} |err|/|ref| {err / abs(ref):.3e} "
        f"(|ref| / sum|terms| {abs(ref) / scale:.3f})")
    assert abs(ref) >= 0.3 * scale
    assert err <= TOL[dtype] * abs(ref)


@pytest.mark.parametrize("causal", [False, True])
def test_head_dim_dW_and_stateless(causal):
    """dW with per-head tables at d = 96 (the table pitch is the caller's d),
    and the backward without a state giving the same bits."""
    key = 2 if causal else 4
    w, inp, dev = _case(key, 96, 1400, 2, 2, "f32", causal, 4, 2)
    Wh = ri.make_W_per_head(w).cuda()
    O, st = race.race_attn_fwd(dev["Q"], dev["K"], dev["V"], Wh, w.beta, w.P, w.L, causal)
    g1 = race.race_attn_bwd(dev["Q"], dev["K"], dev["V"], Wh, w.beta, w.P, w.L, causal, dev["dO"], st,
                            O=O if causal else None, dW=True)
    g2 = race.race_attn_bwd(dev["Q"], dev["K"], dev["V"], Wh, w.beta, w.P, w.L, causal, dev["dO"], None,
                            O=O if causal else None, dW=True)
    torch.cuda.synchronize()
    for a, b in zip(g1[:3], g2[:3]):
        assert torch.equal(a, b)
    dW = g1[-1]
    assert dW.shape == Wh.shape
    Q, K, V, dO = (to64(inp[k]) for k in ("Q", "K", "V", "dO"))
    check("dW (per-head tables)", dW, orc.dW(Q, K, V, Wh.double().cpu().numpy(), w.beta, dO, causal), TOL["f32"])


def test_head_dim_decode_softbucket_banks_noalloc():
    """d = 96: decode after a prefill against the oracle's causal forward from
    the prompt's bank; the soft-assignment export; the bank export; the
    allocation-free forward equal to the forward."""
    w, inp, dev = _case(4, 96, 1200, 1, 2, "bf16", False, 4, 2)
    Wd = dev["W"]
    n0 = 1100
    st = race.race_attn_decode_prefill(dev["K"][:, :, :n0].contiguous(), dev["V"][:, :, :n0].contiguous(), Wd,
                                       w.beta, w.P, w.L)
    new = {k: dev[k][:, :, n0:].contiguous() for k in ("Q", "K", "V")}
    Od = race.race_attn_decode(new["Q"], new["K"], new["V"], Wd, w.beta, w.P, w.L, st)
    phi = race.race_softbucket_debug(dev["Q"], Wd, w.beta, w.P, w.L)
    O, state = race.race_attn_fwd(dev["Q"], dev["K"], dev["V"], Wd, w.beta, w.P, w.L, False)
    c, m, _, _ = race.race_bucket_stats_debug(dev["Q"], Wd, w.P, w.L, False, state=state)
    O2 = torch.empty_like(O)
    state2 = torch.empty_like(state)
    race.race_attn_fwd_noalloc(dev["Q"], dev["K"], dev["V"], Wd, w.beta, w.P, w.L, False, O2, state2)
    torch.cuda.synchronize()
    assert torch.equal(O, O2) and torch.equal(state, state2)
    Q, K, V = (to64(inp[k]) for k in ("Q", "K", "V"))
    Wn = inp["W"].double().numpy()
    ref = np.empty((1, 2, 100, 96))
    for h in range(2):
        c0, m0 = orc.state_head(K[0, h, :n0], V[0, h, :n0], Wn, w.beta)
        ref[0, h] = orc.causal_forward_head(Q[0, h, n0:], K[0, h, n0:], V[0, h, n0:], Wn, w.beta,
                                            content0=c0, mass0=m0)
        sref = orc.soft_assign(Q[0, h], Wn, w.beta).transpose(1, 0, 2)
        err = np.abs(to64(phi[0, h]) - sref).max()
        say(f"  softbucket head {h}: max|err| {err:.2e}")
        assert err < 1e-3
        cr, mr = orc.state_head(K[0, h], V[0, h], Wn, w.beta)
        check(f"content head {h}", c[0, h, 0], cr, TOL["bf16"])
        check(f"mass head {h}", m[0, h, 0], mr, TOL["bf16"])
    check("O (decode)", Od, ref, TOL["bf16"], vmax=float(np.abs(V).max()))
