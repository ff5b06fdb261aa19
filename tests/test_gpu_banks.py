"""GPU parity of the bucket banks themselves (the bank export), entry by
entry against the fp64 oracle.

Non-causal: content = sum_j phi(K_j) V_j^T and mass = sum_j phi(K_j) over
all keys (slides frame "Each bucket stores mass and a weighted value sum"),
and the gradient bank dcontent = sum_t phi(Q_t) g_t^T, dmass = sum_t phi(Q_t)
h_t with g = dO / Den, h = -(dO . O) / Den.  Causal: the bank of the keys
before every sequence segment and the gradient bank of the queries after it
(slides frame "Causality is a prefix update of the same statistics").
Tolerance: 1e-5 (fp32 I/O) or 2e-2 (bf16 I/O) of each bank's largest entry.
The largest error relative to each entry is printed beside it (the masses of
short segments sum a few dozen assignments, so single assignments' errors
show there).
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


def _banks(w, inp):
    dev = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    Q, K, V, dO, W = dev["Q"], dev["K"], dev["V"], dev["dO"], dev["W"]
    O, state = race.race_attn_fwd(Q, K, V, W, w.beta, w.P, w.L, w.causal)
    shape = race._shape_of(Q, W, w.L, w.P)
    ws = torch.empty(race.race_attn_workspace_bytes(shape, w.P, w.L, w.causal, race.RACE_WS_BWD), dtype=torch.uint8,
                     device="cuda")
    race.race_attn_bwd(Q, K, V, W, w.beta, w.P, w.L, w.causal, dO, state, O=O, workspace=ws)
    out = race.race_bucket_stats_debug(Q, W, w.P, w.L, w.causal, state=state, workspace=ws)
    torch.cuda.synchronize()
    return [to64(b) for b in out], race.race_bucket_stats_segments(shape, w.P, w.L, w.causal)


def _cmp(name, got, ref, tol, mass=False):
    err = float(np.abs(got - ref).max() / max(np.abs(ref).max(), 1e-300))
    extra = ""
    if mass:
        # masses are sums of positive assignments
        extra = f", per entry {float((np.abs(got - ref) / np.maximum(ref, 1e-300)).max()):.2e}"
    say(f"  {name}: rel {err:.2e}{extra} (bar {tol:.2e})")
    assert err <= tol


@pytest.mark.parametrize("key,N,B,H,dtype,P,L", [
    (1, 1000, 1, 2, "f32", 3, 2), (4, 3000, 2, 1, "bf16", 4, 2), (3, 2100, 1, 2, "bf16", 3, 3),
    (4, 2000, 1, 2, "bf16", 2, 2), (4, 1500, 1, 2, "f32", 4, 4), (5, 2113, 1, 2, "bf16", 6, 4),
])
def test_noncausal_banks(key, N, B, H, dtype, P, L):
    w = replace(ri.WORKLOADS[key].with_size(N=N, B=B, H=H), causal=False, dtype=dtype, P=P, L=L)
    inp = ri.make_inputs(w, device="cpu", with_grad_out=True)
    say(f"non-causal banks key={key} N={N} B={B} H={H} {dtype} P={P} L={L}")
    (c, m, dc, dm), (S, _) = _banks(w, inp)
    assert S == 1 and c.shape == (B, H, 1, L, 1 << P, w.d)
    Q, K, V, dO = (to64(inp[k]) for k in ("Q", "K", "V", "dO"))
    Wn = inp["W"].double().numpy()
    tol = TOL[dtype]
    for b in range(B):
        for h in range(H):
            cr, mr = orc.state_head(K[b, h], V[b, h], Wn, w.beta)
            Phi_Q, _, _, g, hh = orc.query_terms(Q[b, h], dO[b, h], Wn, w.beta, cr, mr)
            dcr, dmr = orc.grad_banks(None, Wn, w.beta, g, hh, Phi_Q=Phi_Q)
            _cmp("content", c[b, h, 0], cr, tol)
            _cmp("mass", m[b, h, 0], mr, tol, mass=True)
            _cmp("dcontent", dc[b, h, 0], dcr, tol)
            _cmp("dmass", dm[b, h, 0], dmr, tol)


@pytest.mark.parametrize("key,N,B,H,dtype,P,L", [
    (2, 1000, 1, 2, "f32", 4, 4), (5, 2113, 1, 2, "bf16", 6, 4), (4, 2500, 1, 1, "bf16", 2, 2),
    (3, 901, 2, 1, "bf16", 3, 3),
])
def test_causal_segment_banks(key, N, B, H, dtype, P, L):
    w = replace(ri.WORKLOADS[key].with_size(N=N, B=B, H=H), causal=True, dtype=dtype, P=P, L=L)
    inp = ri.make_inputs(w, device="cpu", with_grad_out=True)
    (c, m, dc, dm), (S, seg) = _banks(w, inp)
    say(f"causal banks key={key} N={N} B={B} H={H} {dtype} P={P} L={L}: {S} segments of {seg} tokens")
    assert S >= 2 and c.shape == (B, H, S, L, 1 << P, w.d)
    Q, K, V, dO = (to64(inp[k]) for k in ("Q", "K", "V", "dO"))
    Wn = inp["W"].double().numpy()
    tol = TOL[dtype]
    for b in range(B):
        for h in range(H):
            O, Den = orc.causal_forward_head(Q[b, h], K[b, h], V[b, h], Wn, w.beta, return_den=True)
            g = dO[b, h] / Den[:, None]
            hh = -np.sum(dO[b, h] * O, axis=1) / Den
            Phi_Q = orc.soft_assign(Q[b, h], Wn, w.beta)
            refs = {k: [] for k in ("c", "m", "dc", "dm")}
            for s in range(S):
                t0, t1 = s * seg, min(N, (s + 1) * seg)
                if t0:
                    cr, mr = orc.state_head(K[b, h, :t0], V[b, h, :t0], Wn, w.beta)
                else:
                    cr, mr = np.zeros((L, 1 << P, w.d)), np.zeros((L, 1 << P))
                dcr, dmr = orc.grad_banks(None, Wn, w.beta, g[t1:], hh[t1:], Phi_Q=Phi_Q[:, t1:])
                for k, v in (("c", cr), ("m", mr), ("dc", dcr), ("dm", dmr)):
                    refs[k].append(v)
            ref = {k: np.stack(v) for k, v in refs.items()}
            _cmp("content before each segment", c[b, h], ref["c"], tol)
            _cmp("mass before each segment", m[b, h, 1:], ref["m"][1:], tol, mass=True)
            assert np.all(m[b, h, 0] == 0)
            _cmp("dcontent after each segment", dc[b, h], ref["dc"], tol)
            _cmp("dmass after each segment", dm[b, h], ref["dm"], tol)
            assert np.all(dc[b, h, S - 1] == 0) and np.all(dm[b, h, S - 1] == 0)
