"""GPU parity of the recurrent decode path (prefill bank + token-by-token
update-then-read) against the fp64 oracle's causal forward from a prefix
bank (slides frame "Causality is a prefix update of the same statistics").

Shapes: prompts spanning several 128-token tiles and workgroups with a
ragged tail, then a few decode tokens per (batch, head).  Tolerances as for
the forward: fp32 I/O 1e-5, bf16 I/O 2e-2 relative to max |O_ref| (and to
max |V|).
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


def _case(key, N, B, H, dtype):
    w = replace(ri.WORKLOADS[key].with_size(N=N, B=B, H=H), causal=True, dtype=dtype)
    inp = ri.make_inputs(w, device="cpu")
    return w, inp


def _oracle_tail(inp, w, n0):
    """Causal O of tokens n0.. given the bank of tokens < n0 (float64)."""
    Q, K, V = (to64(inp[k]) for k in ("Q", "K", "V"))
    Wn = inp["W"].double().numpy()
    out = np.empty(Q[:, :, n0:].shape)
    for b in range(w.B):
        for h in range(w.H):
            c0, m0 = orc.state_head(K[b, h, :n0], V[b, h, :n0], Wn, w.beta) if n0 > 0 else (None, None)
            out[b, h] = orc.causal_forward_head(Q[b, h, n0:], K[b, h, n0:], V[b, h, n0:], Wn, w.beta,
                                                content0=c0, mass0=m0)
    return out


@pytest.mark.parametrize("key,N0,N1,B,H,dtype", [
    (1, 900, 5, 1, 1, "f32"), (2, 1000, 4, 2, 2, "bf16"), (5, 2500, 3, 1, 2, "bf16"), (2, 333, 7, 1, 2, "f32"),
])
def test_prefill_then_decode(key, N0, N1, B, H, dtype):
    w, inp = _case(key, N0 + N1, B, H, dtype)
    say(f"decode key={key} prompt={N0} new={N1} B={B} H={H} {dtype} d={w.d} P={w.P} L={w.L} beta={w.beta}")
    dev = {k: inp[k].cuda() for k in ("Q", "K", "V")}
    Wd = inp["W"].cuda()
    st = race.race_attn_decode_prefill(dev["K"][:, :, :N0].contiguous(), dev["V"][:, :, :N0].contiguous(), Wd,
                                       w.beta, w.P, w.L)
    st2 = st.clone()
    new = {k: v[:, :, N0:].contiguous() for k, v in dev.items()}
    O = race.race_attn_decode(new["Q"], new["K"], new["V"], Wd, w.beta, w.P, w.L, st)
    # one token per call gives the same bits and the same final state
    outs = []
    for t in range(N1):
        one = {k: v[:, :, t:t + 1].contiguous() for k, v in new.items()}
        outs.append(race.race_attn_decode(one["Q"], one["K"], one["V"], Wd, w.beta, w.P, w.L, st2))
    torch.cuda.synchronize()
    assert torch.equal(torch.cat(outs, dim=2), O)
    assert torch.equal(st, st2)
    ref = _oracle_tail(inp, w, N0)
    vmax = float(np.abs(to64(inp["V"])).max())
    check("O (decode)", O, ref, TOL[dtype], vmax=vmax)


def test_decode_from_empty_state_is_the_causal_forward():
    """A zeroed state is the empty prefix: decoding a sequence token by token
    gives its causal forward."""
    w, inp = _case(2, 48, 1, 2, "f32")
    Wd = inp["W"].cuda()
    nb = race.race_attn_decode_state_bytes(race._shape_of(inp["Q"].cuda()), w.P, w.L)
    st = torch.zeros(nb // 4, dtype=torch.float32, device="cuda")
    O = race.race_attn_decode(inp["Q"].cuda(), inp["K"].cuda(), inp["V"].cuda(), Wd, w.beta, w.P, w.L, st)
    torch.cuda.synchronize()
    check("O (decode from empty)", O, _oracle_tail(inp, w, 0), TOL["f32"])


def test_prefill_bank_matches_oracle():
    """The prefill state is the bank of the prompt: content and mass."""
    w, inp = _case(5, 3001, 1, 2, "bf16")
    Wd = inp["W"].cuda()
    st = race.race_attn_decode_prefill(inp["K"].cuda(), inp["V"].cuda(), Wd, w.beta, w.P, w.L)
    torch.cuda.synchronize()
    LRP = st.numel() // (w.B * w.H * (w.d + 1))
    content = st[: w.B * w.H * LRP * w.d].view(w.B * w.H, LRP, w.d)
    mass = st[w.B * w.H * LRP * w.d:].view(w.B * w.H, LRP)
    K, V = to64(inp["K"]), to64(inp["V"])
    for h in range(w.H):
        c, m = orc.state_head(K[0, h], V[0, h], inp["W"].double().numpy(), w.beta)
        LR = w.L * w.R
        check(f"content head {h}", content[h, :LR], c.reshape(LR, w.d), TOL["bf16"])
        check(f"mass head {h}", mass[h, :LR], m.reshape(LR), 2.0 ** -9)


def test_decode_steps_replayed_from_a_graph():
    """Decode steps captured in a HIP graph (the launch-bound loop of a
    serving step) replay to the eager results bit for bit: the state is reset
    from the same prefill before each replay, and other eager decode work and
    synchronisations run between the replays."""
    w, inp = _case(2, 512, 2, 2, "f32")
    n0, steps = 500, 6
    dev = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    say(f"decode graph replay key=2 prompt={n0} steps={steps}")
    s0 = race.race_attn_decode_prefill(dev["K"][:, :, :n0].contiguous(), dev["V"][:, :, :n0].contiguous(),
                                       dev["W"], w.beta, w.P, w.L)
    toks = [{k: dev[k][:, :, n0 + i:n0 + i + 1].contiguous() for k in ("Q", "K", "V")} for i in range(steps)]
    st_e = s0.clone()
    O_e = [race.race_attn_decode(t["Q"], t["K"], t["V"], dev["W"], w.beta, w.P, w.L, st_e) for t in toks]
    torch.cuda.synchronize()

    race.profile_enable(False)
    st_g = s0.clone()
    O_g = [torch.empty_like(t["Q"]) for t in toks]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for t, o in zip(toks, O_g):
            race.race_attn_decode(t["Q"], t["K"], t["V"], dev["W"], w.beta, w.P, w.L, st_g, O=o)
    other = s0.clone()
    for rep in range(3):
        st_g.copy_(s0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(O_e, O_g):
            assert torch.equal(a, b), f"replay {rep}: O differs from the eager steps"
        assert torch.equal(st_e, st_g), f"replay {rep}: state differs from the eager steps"
        # unrelated eager decode work between replays
        race.race_attn_decode(toks[rep]["Q"], toks[rep]["K"], toks[rep]["V"], dev["W"], w.beta, w.P, w.L, other)
        torch.cuda.synchronize()
