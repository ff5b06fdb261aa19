"""A whole training step of the layer (forward, then backward with dbeta and
dW) captured in a HIP graph.  Every entry point only enqueues kernels on the
caller's stream (no allocation, memset or synchronisation), so the step is
capturable; replays must equal the eager step bit for bit (every sum is in a
fixed order).  Each replay is followed by eager work and a synchronisation,
and every replay is checked."""
from dataclasses import replace

import pytest
import torch

import race_inputs as ri
from parity_util import say

pytestmark = pytest.mark.gpu

race = pytest.importorskip("linear_attention_soft_amd")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    race.lib()


@pytest.mark.parametrize("key,N,causal", [(3, 3000, False), (5, 1100, True)])
def test_training_step_replayed_from_a_graph(key, N, causal):
    w = replace(ri.WORKLOADS[key].with_size(N=N, B=1, H=2), causal=causal, dtype="bf16")
    inp = ri.make_inputs(w, device="cuda", with_grad_out=True)
    Q, K, V, dO = inp["Q"], inp["K"], inp["V"], inp["dO"]
    W = inp["W"].cuda()
    say(f"graph step key={key} N={N} causal={causal}")
    shape = race._shape_of(Q, W, w.L, w.P)
    dev = "cuda"

    def buffers():
        b = {"O": torch.empty_like(Q), "dQ": torch.empty_like(Q), "dK": torch.empty_like(K),
             "dV": torch.empty_like(V), "dbeta": torch.empty(1, dtype=torch.float32, device=dev),
             "dW": torch.empty_like(W)}
        b["st"] = torch.empty(race.race_attn_state_bytes(shape, w.P, w.L, causal), dtype=torch.uint8, device=dev)
        b["wf"] = torch.empty(race.race_attn_workspace_bytes(shape, w.P, w.L, causal, 0), dtype=torch.uint8,
                              device=dev)
        b["wb"] = torch.empty(race.race_attn_workspace_bytes(shape, w.P, w.L, causal, 2), dtype=torch.uint8,
                              device=dev)
        return b

    def step(b):
        race.race_attn_fwd(Q, K, V, W, w.beta, w.P, w.L, causal, O=b["O"], state=b["st"], workspace=b["wf"])
        race.race_attn_bwd(Q, K, V, W, w.beta, w.P, w.L, causal, dO, b["st"], O=b["O"] if causal else None,
                           dQ=b["dQ"], dK=b["dK"], dV=b["dV"], dbeta=b["dbeta"], dW=b["dW"], workspace=b["wb"])

    race.profile_enable(False)
    eager = buffers()
    step(eager)
    torch.cuda.synchronize()
    outs = ("O", "dQ", "dK", "dV", "dbeta", "dW")
    ref = {k: eager[k].clone() for k in outs}

    gb = buffers()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(gb)
    for rep in range(3):
        for k in outs:
            gb[k].fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k in outs:
            assert torch.equal(gb[k], ref[k]), f"replay {rep}: {k} differs from the eager step"
        step(eager)          # eager work between replays
        torch.cuda.synchronize()
