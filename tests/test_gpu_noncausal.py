"""GPU parity of the non-causal HIP path against the fp64 oracle.

Element-by-element comparison on seeded inputs that span several 128-token
tiles, several workgroups and a ragged tail; tolerances: fp32 I/O 1e-5 and
bf16 I/O 2e-2, relative to the reference's max |value| per output (and for O
also to max |V|).
"""
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


def _inputs(key, N, B=None, H=None, seed=None, with_grad=True):
    w = ri.WORKLOADS[key].with_size(N=N, B=B, H=H)
    inp = ri.make_inputs(w, device="cpu", seed_base=seed, with_grad_out=with_grad)
    dev = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    return w, inp, dev


def _run_fwd(w, dev):
    O, state = race.race_attn_fwd(dev["Q"], dev["K"], dev["V"], dev["W"], w.beta, w.P, w.L, w.causal)
    torch.cuda.synchronize()
    return O, state


# ----------------------------------------------------------------- soft assignments
@pytest.mark.parametrize("key,N,dtype", [(1, 300, "f32"), (2, 200, "f32"), (4, 333, "f32"),
                                          (3, 300, "bf16"), (4, 257, "bf16"), (5, 290, "bf16")])
def test_softbucket_matches_oracle(key, N, dtype):
    w = ri.WORKLOADS[key].with_size(N=N, B=1, H=2)
    from dataclasses import replace
    w = replace(w, dtype=dtype)
    inp = ri.make_inputs(w, device="cpu", with_grad_out=False)
    say(f"softbucket key={key} N={N} dtype={dtype} P={w.P} L={w.L}")
    phi = race.race_softbucket_debug(inp["Q"].cuda(), inp["W"].cuda(), w.beta, w.P, w.L)
    torch.cuda.synchronize()
    X = to64(inp["Q"])
    W = inp["W"].double().numpy()
    for b in range(w.B):
        for h in range(w.H):
            ref = orc.soft_assign(X[b, h], W, w.beta).transpose(1, 0, 2)   # (N, L, R)
            got = to64(phi[b, h])
            err = np.abs(got - ref).max()
            # |dphi/dpre_t| <= beta/2 per hyperplane.  f32: fp32 accumulation of
            # the d-term projection (a plain fp32 emulation gives ~6e-6 here);
            # bf16: W is split into bf16 hi + lo, leaving a 2^-18 relative
            # residual per weight (observed 1.5e-4 at d = 128, beta = 4).
            assert err < (2e-5 if dtype == "f32" else 1e-3), err


# ----------------------------------------------------------------- forward
def test_forward_f32_n1k_full():
    """Non-causal forward, fp32, N=1024, d=64, P=3, L=2, beta=1 (the whole workload)."""
    w, inp, dev = _inputs(1, N=1024, with_grad=False)
    say(f"forward {w.name}")
    O, state = _run_fwd(w, dev)
    ref = oracle_fwd(inp, False)
    check("O", O, ref, TOL["f32"], vmax=float(to64(inp["V"]).__abs__().max()))


def test_forward_bank_matches_oracle():
    """The state buffer holds the bucket bank: content[BH][LRP][d], mass[BH][LRP]."""
    w, inp, dev = _inputs(1, N=1000, B=1, H=2, with_grad=False)
    O, state = _run_fwd(w, dev)
    st = state.view(torch.float32)
    BH, LRP, d = 2, 32, w.d
    content = to64(st[:BH * LRP * d]).reshape(BH, LRP, d)
    mass = to64(st[BH * LRP * d:BH * LRP * (d + 1)]).reshape(BH, LRP)
    K, V = to64(inp["K"]), to64(inp["V"])
    for bh in range(BH):
        c_ref, m_ref = orc.state_head(K[0, bh], V[0, bh], inp["W"].double().numpy(), w.beta)
        LR = w.L * w.R
        np.testing.assert_allclose(content[bh, :LR], c_ref.reshape(LR, d), rtol=0, atol=2e-5 * np.abs(c_ref).max())
        np.testing.assert_allclose(mass[bh, :LR], m_ref.reshape(LR), rtol=1e-5)
        assert np.all(content[bh, LR:] == 0) and np.all(mass[bh, LR:] == 0)


@pytest.mark.parametrize("key,N,B,H,dtype", [
    (1, 300, 1, 2, "f32"), (4, 777, 2, 1, "f32"), (2, 1000, 1, 1, "f32"),
    (3, 4161, 1, 2, "bf16"), (4, 8225, 1, 2, "bf16"), (2, 2000, 1, 2, "bf16"),
])
def test_forward_backward_parity(key, N, B, H, dtype):
    from dataclasses import replace
    w = replace(ri.WORKLOADS[key].with_size(N=N, B=B, H=H), causal=False, dtype=dtype)
    inp = ri.make_inputs(w, device="cpu", with_grad_out=True)
    dev = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    say(f"fwd+bwd key={key} N={N} B={B} H={H} dtype={dtype} d={w.d} P={w.P} L={w.L} beta={w.beta}")
    O, state = _run_fwd(w, dev)
    dQ, dK, dV = race.race_attn_bwd(dev["Q"], dev["K"], dev["V"], dev["W"], w.beta, w.P, w.L, False,
                                    dev["dO"], state)
    torch.cuda.synchronize()
    tol = TOL[dtype]
    vmax = float(np.abs(to64(inp["V"])).max())
    check("O", O, oracle_fwd(inp, False), tol, vmax=vmax)
    rdQ, rdK, rdV = oracle_bwd(inp, False)
    check("dQ", dQ, rdQ, tol)
    check("dK", dK, rdK, tol)
    check("dV", dV, rdV, tol)


def test_long_classification_workload_full():
    """B=2, H=4, N=65536, d=64, P=3, L=3, beta=4, bf16, log-uniform row norms: the whole workload."""
    w, inp, dev = _inputs(3, N=65536)
    say(f"fwd+bwd {w.name} (full size)")
    O, state = _run_fwd(w, dev)
    dQ, dK, dV = race.race_attn_bwd(dev["Q"], dev["K"], dev["V"], dev["W"], w.beta, w.P, w.L, False,
                                    dev["dO"], state)
    torch.cuda.synchronize()
    vmax = float(np.abs(to64(inp["V"])).max())
    check("O", O, oracle_fwd(inp, False), TOL["bf16"], vmax=vmax)
    rdQ, rdK, rdV = oracle_bwd(inp, False)
    check("dQ", dQ, rdQ, TOL["bf16"])
    check("dK", dK, rdK, TOL["bf16"])
    check("dV", dV, rdV, TOL["bf16"])


def test_strong_signal_values():
    """Values that follow the keys' directions, so each output depends strongly
    on its query's buckets (O is far from the mean of V)."""
    w, inp, dev = _inputs(4, N=16384, B=1, H=2)
    g = torch.Generator().manual_seed(77)
    V = (inp["K"].float() + 0.1 * torch.randn(inp["K"].shape, generator=g)).to(torch.bfloat16)
    inp["V"] = V
    dev["V"] = V.cuda()
    O, state = _run_fwd(w, dev)
    ref = oracle_fwd(inp, False)
    assert np.abs(ref).max() > 0.05 * np.abs(to64(V)).max()   # iid values give ~0.01
    check("O", O, ref, TOL["bf16"])
    dQ, dK, dV = race.race_attn_bwd(dev["Q"], dev["K"], dev["V"], dev["W"], w.beta, w.P, w.L, False,
                                    dev["dO"], state)
    torch.cuda.synchronize()
    rdQ, rdK, rdV = oracle_bwd(inp, False)
    check("dQ", dQ, rdQ, TOL["bf16"])
    check("dK", dK, rdK, TOL["bf16"])
    check("dV", dV, rdV, TOL["bf16"])


def test_degenerate_inputs():
    """One token (O = V), constant V (O = V), beta = 0 (O = mean V)."""
    w, inp, dev = _inputs(1, N=1, B=1, H=1, with_grad=False)
    O, _ = _run_fwd(w, dev)
    assert torch.allclose(O.cpu(), inp["V"], atol=1e-6)
    w, inp, dev = _inputs(1, N=500, B=1, H=1, with_grad=False)
    c = torch.linspace(-2, 2, w.d)
    dev["V"] = c.expand(1, 1, 500, w.d).contiguous().cuda()
    O, _ = _run_fwd(w, dev)
    assert (O.cpu() - c).abs().max() < 1e-5
    O, _ = race.race_attn_fwd(dev["Q"], dev["K"], inp["V"].cuda(), dev["W"], 0.0, w.P, w.L, False)
    torch.cuda.synchronize()
    assert (O.cpu() - inp["V"].mean(dim=2, keepdim=True)).abs().max() < 1e-5


def test_deterministic():
    w, inp, dev = _inputs(4, N=20000, B=1, H=2)
    O1, s1 = _run_fwd(w, dev)
    O2, s2 = _run_fwd(w, dev)
    assert torch.equal(O1, O2) and torch.equal(s1, s2)
    g1 = race.race_attn_bwd(dev["Q"], dev["K"], dev["V"], dev["W"], w.beta, w.P, w.L, False, dev["dO"], s1)
    g2 = race.race_attn_bwd(dev["Q"], dev["K"], dev["V"], dev["W"], w.beta, w.P, w.L, False, dev["dO"], s1)
    torch.cuda.synchronize()
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)
