"""Parity at the full workload sizes, on the inputs and in the launch
configuration that bench.py times.

The fp64 oracle streams every token once or twice (bucket banks are sums over
the whole sequence), then checks: the whole bucket bank (every entry), and
sampled output / gradient rows that the oracle evaluates one by one from its
own banks.  Causal: sampled rows read the oracle's prefix bank at their
position; the final 2048-token block is checked element by element from the
bank of everything before it; sum_j dV_j = sum_t dO_t holds at any size.
"""
import numpy as np
import pytest
import torch

import race_inputs as ri
from oracle import race_oracle as orc
from parity_util import TOL, say

pytestmark = pytest.mark.gpu

race = pytest.importorskip("linear_attention_soft_amd")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    race.lib()


def f64(t):
    return t.to(torch.float64).cpu().numpy()


def rel(got, ref):
    return float(np.abs(got - ref).max() / max(np.abs(ref).max(), 1e-300))


def _run(w):
    say(f"full-size {w.name}: inputs on the GPU")
    inp = ri.make_inputs(w, device="cuda")
    Wd = inp["W"].cuda()
    O, state = race.race_attn_fwd(inp["Q"], inp["K"], inp["V"], Wd, w.beta, w.P, w.L, w.causal)
    dQ, dK, dV = race.race_attn_bwd(inp["Q"], inp["K"], inp["V"], Wd, w.beta, w.P, w.L, w.causal, inp["dO"], state,
                                    O=O)
    torch.cuda.synchronize()
    say("  GPU forward + backward done")
    return inp, O, state, dQ, dK, dV


@pytest.mark.timeout(1200)
def test_noncausal_12m_tokens_full_size():
    w = ri.WORKLOADS[4]
    inp, O, state, dQ, dK, dV = _run(w)
    Q, K, V, dO = inp["Q"], inp["K"], inp["V"], inp["dO"]
    Wn = inp["W"].double().numpy()
    N, d, L, R = w.N, w.d, w.L, w.R
    LRP = 32
    st = state.view(torch.float32)
    nb = w.B * w.H * LRP * d
    cont_gpu = f64(st[:nb]).reshape(w.H, LRP, d)
    mass_gpu = f64(st[nb:nb + w.B * w.H * LRP]).reshape(w.H, LRP)
    rng = np.random.default_rng(404)
    step = 1 << 20
    tol = TOL["bf16"]
    # heads 0 and H-1 sampled for the bank, O and dQ; head H-1 for the gradient bank, dK and dV
    for h in (0, w.H - 1):
        content = np.zeros((L, R, d))
        mass = np.zeros((L, R))
        for t0 in range(0, N, step):
            c, m = orc.state_head(f64(K[0, h, t0:t0 + step]), f64(V[0, h, t0:t0 + step]), Wn, w.beta)
            content += c
            mass += m
        e_c = rel(cont_gpu[h, :L * R].reshape(L, R, d), content)
        e_m = rel(mass_gpu[h, :L * R].reshape(L, R), mass)
        say(f"  head {h}: bank content rel {e_c:.2e}, mass rel {e_m:.2e}")
        # each assignment is rounded to bf16 once before it is summed, so the
        # masses can deviate by at most 2^-9 relative (round-to-nearest-even of
        # this distribution is biased: an fp64 emulation gives 8.7e-4 here)
        assert e_c <= tol and e_m <= 2.0 ** -9
        idx = np.sort(rng.choice(N, 2048, replace=False))
        it = torch.from_numpy(idx).cuda()
        Qs, dOs = f64(Q[0, h][it]), f64(dO[0, h][it])
        dq_ref, o_ref, _, _, _ = orc.query_grads(Qs, dOs, Wn, w.beta, content, mass)
        e_o = rel(f64(O[0, h][it]), o_ref)
        e_q = rel(f64(dQ[0, h][it]), dq_ref)
        vmax = float(f64(V[0, h, :step]).__abs__().max())
        say(f"  head {h}: sampled O rel {e_o:.2e} (abs/max|V| {np.abs(f64(O[0, h][it]) - o_ref).max() / vmax:.2e}),"
            f" dQ rel {e_q:.2e}")
        assert e_o <= tol and e_q <= tol
        if h != w.H - 1:
            continue
        dc = np.zeros((L, R, d))
        dm = np.zeros((L, R))
        for t0 in range(0, N, step):
            Phi_Q, _, _, g, hh = orc.query_terms(f64(Q[0, h, t0:t0 + step]), f64(dO[0, h, t0:t0 + step]), Wn, w.beta,
                                                 content, mass)
            a, b = orc.grad_banks(None, Wn, w.beta, g, hh, Phi_Q=Phi_Q)
            dc += a
            dm += b
        idx = np.sort(rng.choice(N, 2048, replace=False))
        it = torch.from_numpy(idx).cuda()
        dk_ref, dv_ref = orc.key_grads(f64(K[0, h][it]), f64(V[0, h][it]), Wn, w.beta, dc, dm)
        e_k, e_v = rel(f64(dK[0, h][it]), dk_ref), rel(f64(dV[0, h][it]), dv_ref)
        say(f"  head {h}: sampled dK rel {e_k:.2e}, dV rel {e_v:.2e}")
        assert e_k <= tol and e_v <= tol


@pytest.mark.timeout(1200)
def test_causal_1m_tokens_wide_buckets_full_size():
    w = ri.WORKLOADS[5]
    inp, O, state, dQ, dK, dV = _run(w)
    Q, K, V, dO = inp["Q"], inp["K"], inp["V"], inp["dO"]
    Wn = inp["W"].double().numpy()
    N, d, L, R = w.N, w.d, w.L, w.R
    TAIL = 2048
    rng = np.random.default_rng(505)
    tol = TOL["bf16"]
    step = 1 << 16
    for h in range(w.H):
        samples = np.sort(rng.choice(N - TAIL, 512, replace=False))
        content = np.zeros((L, R, d))
        mass = np.zeros((L, R))
        pos = 0
        got_o, ref_o, got_q, ref_q = [], [], [], []
        si = 0
        for t0 in range(0, N - TAIL, step):
            t1 = min(N - TAIL, t0 + step)
            Kc, Vc = f64(K[0, h, t0:t1]), f64(V[0, h, t0:t1])
            while si < len(samples) and samples[si] < t1:
                t = int(samples[si])
                c, m = orc.state_head(Kc[pos - t0:t + 1 - t0], Vc[pos - t0:t + 1 - t0], Wn, w.beta)
                content += c
                mass += m
                pos = t + 1
                dq, o, _, _, _ = orc.query_grads(f64(Q[0, h, t:t + 1]), f64(dO[0, h, t:t + 1]), Wn, w.beta,
                                                 content, mass)
                ref_o.append(o[0]); ref_q.append(dq[0])
                got_o.append(f64(O[0, h, t])); got_q.append(f64(dQ[0, h, t]))
                si += 1
            if pos < t1:
                c, m = orc.state_head(Kc[pos - t0:], Vc[pos - t0:], Wn, w.beta)
                content += c
                mass += m
                pos = t1
        e_o = rel(np.array(got_o), np.array(ref_o))
        e_q = rel(np.array(got_q), np.array(ref_q))
        say(f"  head {h}: sampled causal O rel {e_o:.2e}, dQ rel {e_q:.2e}")
        assert e_o <= tol and e_q <= tol
        sl = slice(N - TAIL, N)
        Qt, Kt, Vt, dOt = (f64(x[0, h, sl]) for x in (Q, K, V, dO))
        ot = orc.causal_forward_head(Qt, Kt, Vt, Wn, w.beta, content0=content, mass0=mass)
        tq, tk, tv = orc.backward_head(Qt, Kt, Vt, Wn, w.beta, dOt, True, content0=content, mass0=mass)
        errs = [rel(f64(O[0, h, sl]), ot), rel(f64(dQ[0, h, sl]), tq), rel(f64(dK[0, h, sl]), tk),
                rel(f64(dV[0, h, sl]), tv)]
        say(f"  head {h}: final {TAIL}-token block O/dQ/dK/dV rel " + " ".join(f"{e:.2e}" for e in errs))
        assert max(errs) <= tol
        sdv = dV[0, h].double().sum(0).cpu().numpy()
        sdo = dO[0, h].double().sum(0).cpu().numpy()
        e_s = float(np.abs(sdv - sdo).max() / np.abs(sdo).max())
        say(f"  head {h}: sum_j dV_j vs sum_t dO_t rel {e_s:.2e}")
        assert e_s <= 1e-2
