"""GPU parity at the (P, L) settings of the pages' single-layer scaling runs,
and the boundary's state-less backward and caller streams.

The scaling runs ("RACE Attention" slides, frame "The GPU operator reaches
12M tokens at a small budget") use batch 1, 4 heads, head dim 128 at
(P, L) = (2, 2), (3, 3) and (4, 4).  Each setting is checked forward and
backward, non-causal and causal, bf16 and float32 I/O, at sizes that span
several tiles, workgroups and causal segments with a ragged tail, against
the fp64 oracle (tolerances 1e-5 fp32, 2e-2 bf16, relative to max |ref|).
P < 3 runs through the widening to three hyperplanes per table (zero rows
of W), so P = 1 and P = 2 are checked at d = 64 as well.
"""
from dataclasses import replace

import numpy as np
import pytest
import torch

import race_inputs as ri
from parity_util import TOL, check, oracle_bwd, oracle_fwd, say, to64

pytestmark = pytest.mark.gpu

race = pytest.importorskip("linear_attention_soft_amd")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    race.lib()


def _case(P, L, N, dtype, causal, d=128, H=4, key=4):
    """Workload 4's recipe (iid N(0,1) rows, beta 4) with the given (P, L, d);
    W drawn for that shape from the workload's W seed."""
    w = replace(ri.WORKLOADS[key].with_size(N=N, B=1, H=H), P=P, L=L, d=d, causal=causal, dtype=dtype)
    inp = ri.make_inputs(w, device="cpu", with_grad_out=True)
    dev = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    return w, inp, dev


def _parity(w, inp, dev):
    O, state = race.race_attn_fwd(dev["Q"], dev["K"], dev["V"], dev["W"], w.beta, w.P, w.L, w.causal)
    dQ, dK, dV = race.race_attn_bwd(dev["Q"], dev["K"], dev["V"], dev["W"], w.beta, w.P, w.L, w.causal,
                                    dev["dO"], state, O=O if w.causal else None)
    torch.cuda.synchronize()
    tol = TOL[w.dtype]
    vmax = float(np.abs(to64(inp["V"])).max())
    check("O", O, oracle_fwd(inp, w.causal), tol, vmax=vmax)
    rdQ, rdK, rdV = oracle_bwd(inp, w.causal)
    check("dQ", dQ, rdQ, tol)
    check("dK", dK, rdK, tol)
    check("dV", dV, rdV, tol)


SETTINGS = [(2, 2), (3, 3), (4, 4)]


@pytest.mark.parametrize("P,L", SETTINGS)
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_scaling_settings_noncausal(P, L, dtype):
    w, inp, dev = _case(P, L, 5000, dtype, False)
    say(f"non-causal d=128 P={P} L={L} {dtype} N={w.N} H={w.H}")
    _parity(w, inp, dev)


@pytest.mark.parametrize("P,L", SETTINGS)
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_scaling_settings_causal(P, L, dtype):
    w, inp, dev = _case(P, L, 2500, dtype, True)
    say(f"causal d=128 P={P} L={L} {dtype} N={w.N} H={w.H}")
    if dtype == "f32" and (P, L) == (4, 4):
        # float32 causal walks with a 64-row bank need more LDS than a CU has
        with pytest.raises(race.RaceError) as e:
            race.race_attn_fwd(dev["Q"], dev["K"], dev["V"], dev["W"], w.beta, w.P, w.L, True)
        assert e.value.name == "RACE_ERR_UNSUPPORTED"
        return
    _parity(w, inp, dev)


@pytest.mark.parametrize("P,L,causal", [(1, 3, False), (2, 4, False), (1, 2, True), (2, 3, True)])
def test_widened_small_P_d64(P, L, causal):
    w, inp, dev = _case(P, L, 3000, "bf16", causal, d=64, H=2)
    say(f"widened P={P} L={L} causal={causal} d=64 bf16 N={w.N}")
    _parity(w, inp, dev)


@pytest.mark.parametrize("causal,dtype", [(False, "bf16"), (True, "bf16"), (True, "f32"), (False, "f32")])
def test_backward_without_state(causal, dtype):
    """state = NULL: the backward rebuilds the bank (and, causal, the segment
    banks and Den) itself; the same kernels run, so the gradients equal
    those of the backward that takes the forward's state, bit for bit."""
    # the wide causal shape has bf16 kernels only; float32 causal takes the LM shape
    key = (5 if dtype == "bf16" else 2) if causal else 4
    w = replace(ri.WORKLOADS[key].with_size(N=3000, B=1, H=2), causal=causal, dtype=dtype)
    inp = ri.make_inputs(w, device="cuda", with_grad_out=True)
    W = inp["W"].cuda()
    say(f"backward without state causal={causal} {dtype} P={w.P} L={w.L}")
    Q, K, V, dO = inp["Q"], inp["K"], inp["V"], inp["dO"]
    O, st = race.race_attn_fwd(Q, K, V, W, w.beta, w.P, w.L, causal)
    a = race.race_attn_bwd(Q, K, V, W, w.beta, w.P, w.L, causal, dO, st, O=O, dbeta=True)
    b = race.race_attn_bwd(Q, K, V, W, w.beta, w.P, w.L, causal, dO, None, O=O, dbeta=True)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)
    if causal:
        # without O the causal backward rebuilds h from Den O in a walk
        c = race.race_attn_bwd(Q, K, V, W, w.beta, w.P, w.L, True, dO, st, O=None)
        e = race.race_attn_bwd(Q, K, V, W, w.beta, w.P, w.L, True, dO, None, O=None)
        torch.cuda.synchronize()
        for x, y in zip(c, e):
            assert torch.equal(x, y)


def test_caller_stream():
    """Calls on a side stream: the binding allocates its buffers on that
    stream, so a workspace freed on return is not handed to the default
    stream's next allocation while the kernels still run.  The side stream
    is held back by a sleep kernel while the default stream allocates and
    overwrites fresh memory; results must equal the default-stream ones."""
    w = replace(ri.WORKLOADS[4].with_size(N=50000, B=1, H=2), causal=False)
    inp = ri.make_inputs(w, device="cuda", with_grad_out=True)
    W = inp["W"].cuda()
    Q, K, V, dO = inp["Q"], inp["K"], inp["V"], inp["dO"]
    O0, st0 = race.race_attn_fwd(Q, K, V, W, w.beta, w.P, w.L, False)
    g0 = race.race_attn_bwd(Q, K, V, W, w.beta, w.P, w.L, False, dO, st0)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        torch.cuda._sleep(50_000_000)
    O1, st1 = race.race_attn_fwd(Q, K, V, W, w.beta, w.P, w.L, False, stream=s)
    junk = torch.empty(64 << 20, dtype=torch.uint8, device="cuda")
    junk.fill_(0xA5)
    with torch.cuda.stream(s):
        torch.cuda._sleep(50_000_000)
    g1 = race.race_attn_bwd(Q, K, V, W, w.beta, w.P, w.L, False, dO, st1, stream=s)
    junk2 = torch.empty(64 << 20, dtype=torch.uint8, device="cuda")
    junk2.fill_(0x5A)
    torch.cuda.synchronize()
    assert torch.equal(O0, O1)
    for x, y in zip(g0, g1):
        assert torch.equal(x, y)
