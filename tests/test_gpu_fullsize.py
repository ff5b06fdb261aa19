"""Parity at the full workload sizes, on the inputs and in the launch
configuration that bench.py times.

The fp64 oracle streams the sequences chunk by chunk (bucket banks are sums
over whole sequences) and checks every head:

* non-causal, 12M tokens: the whole bucket bank and the whole gradient bank
  (every entry, through the bank export), and sampled O / dQ / dK / dV rows
  that the oracle evaluates one by one from its own banks;
* causal, 1M tokens, 64 corners per table: O at every token (the oracle's
  block-wise evaluation of the prefix readout), the bank before every
  sequence segment and the gradient bank after it (every entry, through the
  bank export), sampled dQ / dK / dV rows spread over the whole sequence
  (each from the oracle's prefix or suffix bank at that row), the final
  2048-token block element by element, and sum_j dV_j = sum_t dO_t.

Each workload runs once on the GPU (a module-scoped fixture); the oracle's
checks run as one test per head, so that each test ends (and reports)
within about half a minute of CPU work.
"""
import time

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


# each soft assignment is rounded to bf16 once before it is summed, so bank
# masses can deviate by at most 2^-9 relative (round-to-nearest-even of these
# assignments is biased: an fp64 emulation gives 8.7e-4 at 12M tokens)
MASS_TOL = 2.0 ** -9


def _run(w):
    say(f"full-size {w.name}: inputs on the GPU")
    inp = ri.make_inputs(w, device="cuda")
    Wd = inp["W"].cuda()
    Q, K, V, dO = inp["Q"], inp["K"], inp["V"], inp["dO"]
    O, state = race.race_attn_fwd(Q, K, V, Wd, w.beta, w.P, w.L, w.causal)
    shape = race._shape_of(Q, Wd, w.L, w.P)
    ws = torch.empty(race.race_attn_workspace_bytes(shape, w.P, w.L, w.causal, race.RACE_WS_BWD), dtype=torch.uint8,
                     device="cuda")
    dQ, dK, dV = race.race_attn_bwd(Q, K, V, Wd, w.beta, w.P, w.L, w.causal, dO, state, O=O, workspace=ws)
    banks = race.race_bucket_stats_debug(Q, Wd, w.P, w.L, w.causal, state=state, workspace=ws)
    torch.cuda.synchronize()
    say("  GPU forward + backward done")
    return inp, O, dQ, dK, dV, [f64(b) for b in banks]


@pytest.fixture(scope="module")
def run_w4():
    return _run(ri.WORKLOADS[4])


@pytest.fixture(scope="module")
def run_w5():
    return _run(ri.WORKLOADS[5])


@pytest.mark.timeout(1500)
@pytest.mark.parametrize("h", range(ri.WORKLOADS[4].H))
def test_noncausal_12m_tokens_full_size(run_w4, h):
    w = ri.WORKLOADS[4]
    inp, O, dQ, dK, dV, (cont_g, mass_g, dcont_g, dmass_g) = run_w4
    Q, K, V, dO = inp["Q"], inp["K"], inp["V"], inp["dO"]
    Wn = inp["W"].double().numpy()
    N, L, R = w.N, w.L, w.R
    rng = np.random.default_rng(404 + h)
    step = 1 << 20
    tol = TOL["bf16"]
    t_start = time.time()
    content = np.zeros((L, R, w.d))
    mass = np.zeros((L, R))
    for t0 in range(0, N, step):
        c, m = orc.state_head(f64(K[0, h, t0:t0 + step]), f64(V[0, h, t0:t0 + step]), Wn, w.beta)
        content += c
        mass += m
    e_c, e_m = rel(cont_g[0, h, 0], content), rel(mass_g[0, h, 0], mass)
    say(f"  head {h}: bank content rel {e_c:.2e}, mass rel {e_m:.2e}")
    assert e_c <= tol and e_m <= MASS_TOL
    idx = np.sort(rng.choice(N, 2048, replace=False))
    it = torch.from_numpy(idx).cuda()
    dq_ref, o_ref, _, _, _ = orc.query_grads(f64(Q[0, h][it]), f64(dO[0, h][it]), Wn, w.beta, content, mass)
    e_o, e_q = rel(f64(O[0, h][it]), o_ref), rel(f64(dQ[0, h][it]), dq_ref)
    vmax = float(np.abs(f64(V[0, h, :step])).max())
    e_ov = float(np.abs(f64(O[0, h][it]) - o_ref).max() / vmax)
    say(f"  head {h}: sampled O rel {e_o:.2e} (abs / max|V| {e_ov:.2e}), dQ rel {e_q:.2e}")
    assert e_o <= tol and e_ov <= tol and e_q <= tol
    dc = np.zeros((L, R, w.d))
    dm = np.zeros((L, R))
    for t0 in range(0, N, step):
        Phi_Q, _, _, g, hh = orc.query_terms(f64(Q[0, h, t0:t0 + step]), f64(dO[0, h, t0:t0 + step]), Wn,
                                             w.beta, content, mass)
        a, b = orc.grad_banks(None, Wn, w.beta, g, hh, Phi_Q=Phi_Q)
        dc += a
        dm += b
    e_dc, e_dm = rel(dcont_g[0, h, 0], dc), rel(dmass_g[0, h, 0], dm)
    say(f"  head {h}: gradient bank dcontent rel {e_dc:.2e}, dmass rel {e_dm:.2e}")
    assert e_dc <= tol and e_dm <= tol
    idx = np.sort(rng.choice(N, 2048, replace=False))
    it = torch.from_numpy(idx).cuda()
    dk_ref, dv_ref = orc.key_grads(f64(K[0, h][it]), f64(V[0, h][it]), Wn, w.beta, dc, dm)
    e_k, e_v = rel(f64(dK[0, h][it]), dk_ref), rel(f64(dV[0, h][it]), dv_ref)
    say(f"  head {h}: sampled dK rel {e_k:.2e}, dV rel {e_v:.2e} ({time.time() - t_start:.0f} s)")
    assert e_k <= tol and e_v <= tol


@pytest.mark.timeout(1500)
@pytest.mark.parametrize("h", range(ri.WORKLOADS[5].H))
def test_causal_1m_tokens_wide_buckets_full_size(run_w5, h):
    w = ri.WORKLOADS[5]
    inp, O, dQ, dK, dV, (cont_g, mass_g, dcont_g, dmass_g) = run_w5
    Q, K, V, dO = inp["Q"], inp["K"], inp["V"], inp["dO"]
    Wn = inp["W"].double().numpy()
    N, d, L, R = w.N, w.d, w.L, w.R
    shape = race._shape_of(Q, inp["W"], w.L, w.P)
    nseg, seg = race.race_bucket_stats_segments(shape, w.P, w.L, True)
    assert cont_g.shape == (1, w.H, nseg, L, R, d)
    say(f"  {nseg} segments of {seg} tokens per head")
    TAIL = 2048
    rng = np.random.default_rng(505 + h)
    tol = TOL["bf16"]
    t_start = time.time()
    samples = np.sort(rng.choice(N, 512, replace=False))
    # forward sweep: O at every token, the bank before every segment,
    # and dQ at the sampled rows from the prefix bank at each of them
    c = np.zeros((L, R, d))
    m = np.zeros((L, R))
    Den = np.empty(N)
    dodo = np.empty(N)
    err_o, max_o, err_ov, vmax = 0.0, 0.0, 0.0, 0.0
    err_bc, max_bc, err_bm, max_bm = 0.0, 0.0, 0.0, 0.0
    got_q, ref_q = [], []
    for s in range(nseg):
        t0, t1 = s * seg, min(N, (s + 1) * seg)
        err_bc = max(err_bc, float(np.abs(cont_g[0, h, s] - c).max()))
        max_bc = max(max_bc, float(np.abs(c).max()))
        err_bm = max(err_bm, float((np.abs(mass_g[0, h, s] - m) / np.maximum(m, 1e-300)).max()) if s else 0.0)
        assert s or (np.all(cont_g[0, h, 0] == 0) and np.all(mass_g[0, h, 0] == 0))
        Qc, Kc, Vc, dOc = (f64(x[0, h, t0:t1]) for x in (Q, K, V, dO))
        o, den, c1, m1 = orc.causal_forward_head_kernel_blocks(Qc, Kc, Vc, Wn, w.beta, content0=c, mass0=m)
        og = f64(O[0, h, t0:t1])
        err_o = max(err_o, float(np.abs(og - o).max()))
        max_o = max(max_o, float(np.abs(o).max()))
        vmax = max(vmax, float(np.abs(Vc).max()))
        Den[t0:t1] = den
        dodo[t0:t1] = np.sum(dOc * o, axis=1)
        # prefix banks at the sampled rows of this segment (keys j <= t)
        cr, mr, pos = c.copy(), m.copy(), t0
        for t in samples[(samples >= t0) & (samples < t1)]:
            a, b = orc.state_head(Kc[pos - t0:t + 1 - t0], Vc[pos - t0:t + 1 - t0], Wn, w.beta)
            cr += a
            mr += b
            pos = t + 1
            dq, _, _, _, _ = orc.query_grads(Qc[t - t0:t + 1 - t0], dOc[t - t0:t + 1 - t0], Wn, w.beta, cr, mr)
            ref_q.append(dq[0])
            got_q.append(f64(dQ[0, h, int(t)]))
        c, m = c1, m1
    e_o, e_ov, e_q = err_o / max_o, err_o / vmax, rel(np.array(got_q), np.array(ref_q))
    e_bc = err_bc / max_bc
    say(f"  head {h}: O at all {N} tokens rel {e_o:.2e} (abs / max|V| {e_ov:.2e}); banks before each segment "
        f"content rel {e_bc:.2e}, mass rel {err_bm:.2e}; sampled dQ rel {e_q:.2e} ({time.time() - t_start:.0f} s)")
    assert e_o <= tol and e_ov <= tol and e_bc <= tol and err_bm <= MASS_TOL and e_q <= tol
    # backward sweep: the gradient bank after every segment, and dK, dV at
    # the sampled rows from the suffix bank at each of them (queries t >= j)
    dc = np.zeros((L, R, d))
    dm = np.zeros((L, R))
    err_gc, max_gc, err_gm, max_gm = 0.0, 0.0, 0.0, 0.0
    got_k, ref_k, got_v, ref_v = [], [], [], []
    for s in reversed(range(nseg)):
        t0, t1 = s * seg, min(N, (s + 1) * seg)
        err_gc = max(err_gc, float(np.abs(dcont_g[0, h, s] - dc).max()))
        max_gc = max(max_gc, float(np.abs(dc).max()))
        err_gm = max(err_gm, float(np.abs(dmass_g[0, h, s] - dm).max()))
        max_gm = max(max_gm, float(np.abs(dm).max()))
        Qc, Kc, Vc, dOc = (f64(x[0, h, t0:t1]) for x in (Q, K, V, dO))
        g = dOc / Den[t0:t1, None]
        hh = -dodo[t0:t1] / Den[t0:t1]
        Phi_Q = orc.soft_assign(Qc, Wn, w.beta)
        dcr, dmr, pos = dc.copy(), dm.copy(), t1
        for j in samples[(samples >= t0) & (samples < t1)][::-1]:
            a, b = orc.grad_banks(None, Wn, w.beta, g[j - t0:pos - t0], hh[j - t0:pos - t0],
                                  Phi_Q=Phi_Q[:, j - t0:pos - t0])
            dcr += a
            dmr += b
            pos = j
            dk, dv = orc.key_grads(Kc[j - t0:j + 1 - t0], Vc[j - t0:j + 1 - t0], Wn, w.beta, dcr, dmr)
            ref_k.append(dk[0]); ref_v.append(dv[0])
            got_k.append(f64(dK[0, h, int(j)])); got_v.append(f64(dV[0, h, int(j)]))
        a, b = orc.grad_banks(None, Wn, w.beta, g[:pos - t0], hh[:pos - t0], Phi_Q=Phi_Q[:, :pos - t0])
        dc, dm = dcr + a, dmr + b
    e_gc, e_gm = err_gc / max_gc, err_gm / max_gm
    e_k, e_v = rel(np.array(got_k), np.array(ref_k)), rel(np.array(got_v), np.array(ref_v))
    say(f"  head {h}: gradient banks after each segment dcontent rel {e_gc:.2e}, dmass rel {e_gm:.2e}; "
        f"sampled dK rel {e_k:.2e}, dV rel {e_v:.2e} ({time.time() - t_start:.0f} s)")
    assert e_gc <= tol and e_gm <= tol and e_k <= tol and e_v <= tol
    # the final block element by element, from the oracle's bank of everything before it
    c0, m0 = np.zeros((L, R, d)), np.zeros((L, R))
    for t0 in range(0, N - TAIL, 1 << 16):
        t1 = min(N - TAIL, t0 + (1 << 16))
        a, b = orc.state_head(f64(K[0, h, t0:t1]), f64(V[0, h, t0:t1]), Wn, w.beta)
        c0 += a
        m0 += b
    sl = slice(N - TAIL, N)
    Qt, Kt, Vt, dOt = (f64(x[0, h, sl]) for x in (Q, K, V, dO))
    tq, tk, tv = orc.backward_head(Qt, Kt, Vt, Wn, w.beta, dOt, True, content0=c0, mass0=m0)
    errs = [rel(f64(dQ[0, h, sl]), tq), rel(f64(dK[0, h, sl]), tk), rel(f64(dV[0, h, sl]), tv)]
    say(f"  head {h}: final {TAIL}-token block dQ/dK/dV rel " + " ".join(f"{e:.2e}" for e in errs))
    assert max(errs) <= tol
    sdv = dV[0, h].double().sum(0).cpu().numpy()
    sdo = dO[0, h].double().sum(0).cpu().numpy()
    e_s = float(np.abs(sdv - sdo).max() / np.abs(sdo).max())
    say(f"  head {h}: sum_j dV_j vs sum_t dO_t rel {e_s:.2e} ({time.time() - t_start:.0f} s)")
    assert e_s <= 1e-2
