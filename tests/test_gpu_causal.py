"""GPU parity of the causal HIP path (prefix bucket sums, forward and
backward) against the fp64 oracle.

Shapes span several 32-token chunks, several sequence segments per head
(segment banks from the scan) and a ragged tail.  Tolerances: fp32 I/O 1e-5,
bf16 I/O 2e-2, relative to the reference's max |value| per output.
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


def _case(key, N, B, H, dtype, seed=None):
    w = replace(ri.WORKLOADS[key].with_size(N=N, B=B, H=H), causal=True, dtype=dtype)
    inp = ri.make_inputs(w, device="cpu", seed_base=seed, with_grad_out=True)
    dev = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    return w, inp, dev


def _fwd_bwd(w, dev, bwd=True):
    O, state = race.race_attn_fwd(dev["Q"], dev["K"], dev["V"], dev["W"], w.beta, w.P, w.L, True)
    grads = None
    if bwd:
        grads = race.race_attn_bwd(dev["Q"], dev["K"], dev["V"], dev["W"], w.beta, w.P, w.L, True, dev["dO"], state)
    torch.cuda.synchronize()
    return O, state, grads


@pytest.mark.parametrize("key,N,B,H,dtype", [
    (2, 300, 1, 2, "f32"), (4, 777, 2, 1, "f32"), (1, 500, 1, 1, "f32"),
    (2, 1000, 1, 2, "bf16"), (4, 2113, 1, 2, "bf16"), (5, 1553, 1, 1, "bf16"), (3, 901, 1, 2, "bf16"),
])
def test_causal_forward_backward_parity(key, N, B, H, dtype):
    w, inp, dev = _case(key, N, B, H, dtype)
    say(f"causal fwd+bwd key={key} N={N} B={B} H={H} dtype={dtype} d={w.d} P={w.P} L={w.L} beta={w.beta}")
    O, state, (dQ, dK, dV) = _fwd_bwd(w, dev)
    tol = TOL[dtype]
    vmax = float(np.abs(to64(inp["V"])).max())
    check("O", O, oracle_fwd(inp, True), tol, vmax=vmax)
    rdQ, rdK, rdV = oracle_bwd(inp, True)
    check("dQ", dQ, rdQ, tol)
    check("dK", dK, rdK, tol)
    check("dV", dV, rdV, tol)


def test_causal_lm_workload_full():
    """B=8, H=8, N=1024, d=64, P=4, L=4, beta=2, bf16 Q/K/V ~ N(0,1)/sqrt(d): the whole workload."""
    w, inp, dev = _case(2, 1024, 8, 8, "bf16")
    say(f"causal forward {w.name} (full size) + backward")
    O, state, (dQ, dK, dV) = _fwd_bwd(w, dev)
    vmax = float(np.abs(to64(inp["V"])).max())
    check("O", O, oracle_fwd(inp, True), TOL["bf16"], vmax=vmax)
    rdQ, rdK, rdV = oracle_bwd(inp, True)
    check("dQ", dQ, rdQ, TOL["bf16"])
    check("dK", dK, rdK, TOL["bf16"])
    check("dV", dV, rdV, TOL["bf16"])


def test_causal_wide_buckets_reduced():
    """P=6 (R=64), L=4, d=128, beta=8, clustered keys: the wide-bucket workload's
    recipe at N = 2113 (34 segments of 64 tokens, two chunks each; the last holds one token)."""
    w, inp, dev = _case(5, 2113, 1, 2, "bf16")
    say(f"causal fwd+bwd {w.name} at N=2113")
    O, state, (dQ, dK, dV) = _fwd_bwd(w, dev)
    vmax = float(np.abs(to64(inp["V"])).max())
    check("O", O, oracle_fwd(inp, True), TOL["bf16"], vmax=vmax)
    rdQ, rdK, rdV = oracle_bwd(inp, True)
    check("dQ", dQ, rdQ, TOL["bf16"])
    check("dK", dK, rdK, TOL["bf16"])
    check("dV", dV, rdV, TOL["bf16"])


@pytest.mark.parametrize("N", [31, 32, 33, 95])
def test_causal_wide_buckets_one_to_three_chunks(N):
    """The wide-bucket recipe (P=6, L=4, d=128, bf16) over one partial chunk,
    exactly one chunk, one chunk and a one-token tail, and a 31-token tail:
    the transposed walks' split tables, shared score tiles and staging at
    their smallest extents."""
    w, inp, dev = _case(5, N, 1, 2, "bf16")
    say(f"causal fwd+bwd {w.name} at N={N}")
    O, state, (dQ, dK, dV) = _fwd_bwd(w, dev)
    vmax = float(np.abs(to64(inp["V"])).max())
    check("O", O, oracle_fwd(inp, True), TOL["bf16"], vmax=vmax)
    rdQ, rdK, rdV = oracle_bwd(inp, True)
    check("dQ", dQ, rdQ, TOL["bf16"])
    check("dK", dK, rdK, TOL["bf16"])
    check("dV", dV, rdV, TOL["bf16"])


def test_causal_degenerate():
    """O_1 = V_1; constant V gives that constant; beta = 0 gives running means;
    one-token sequences."""
    w, inp, dev = _case(2, 333, 1, 1, "f32")
    O, _, _ = _fwd_bwd(w, dev, bwd=False)
    assert torch.allclose(O[0, 0, 0].cpu(), inp["V"][0, 0, 0], atol=1e-6)
    c = torch.linspace(-1, 3, w.d)
    Vc = c.expand(1, 1, 333, w.d).contiguous().cuda()
    O, _ = race.race_attn_fwd(dev["Q"], dev["K"], Vc, dev["W"], w.beta, w.P, w.L, True)
    torch.cuda.synchronize()
    assert (O.cpu() - c).abs().max() < 1e-5
    O, _ = race.race_attn_fwd(dev["Q"], dev["K"], dev["V"], dev["W"], 0.0, w.P, w.L, True)
    torch.cuda.synchronize()
    run = torch.cumsum(inp["V"][0, 0].double(), 0) / torch.arange(1, 334, dtype=torch.float64)[:, None]
    assert (O[0, 0].cpu().double() - run).abs().max() < 1e-5
    w1, inp1, dev1 = _case(4, 1, 1, 3, "bf16")
    O1, _, (dQ1, dK1, dV1) = _fwd_bwd(w1, dev1)
    assert torch.allclose(O1.cpu().float(), inp1["V"].float(), atol=1e-2)


def test_causal_deterministic():
    """Two runs give identical bits (fixed-order sums, no float atomics).  The
    state buffers start zeroed so their alignment padding compares equal."""
    w, inp, dev = _case(5, 3000, 1, 2, "bf16")
    shape = race._shape_of(dev["Q"])
    nbytes = race.race_attn_state_bytes(shape, w.P, w.L, True)
    outs = []
    for _ in range(2):
        st = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
        O, st = race.race_attn_fwd(dev["Q"], dev["K"], dev["V"], dev["W"], w.beta, w.P, w.L, True, state=st)
        g = race.race_attn_bwd(dev["Q"], dev["K"], dev["V"], dev["W"], w.beta, w.P, w.L, True, dev["dO"], st)
        torch.cuda.synchronize()
        outs.append((O, st) + tuple(g))
    for a, b in zip(*outs):
        assert torch.equal(a, b)


@pytest.mark.parametrize("key,N,B,H,dtype", [(2, 700, 1, 2, "f32"), (5, 1553, 1, 2, "bf16")])
def test_causal_backward_given_O(key, N, B, H, dtype):
    """With the forward output handed over, h = -(dO . O) / Den comes from O
    elementwise instead of a rebuilding walk: same oracle bar, and agreement
    with the path that rebuilds Den O (fp32 I/O: to rounding; bf16 I/O: O is
    rounded to bf16 before it is read, so to the bf16 bar)."""
    w, inp, dev = _case(key, N, B, H, dtype)
    say(f"causal bwd given O key={key} N={N} H={H} dtype={dtype}")
    O, state = race.race_attn_fwd(dev["Q"], dev["K"], dev["V"], dev["W"], w.beta, w.P, w.L, True)
    g_o = race.race_attn_bwd(dev["Q"], dev["K"], dev["V"], dev["W"], w.beta, w.P, w.L, True, dev["dO"], state, O=O)
    g_n = race.race_attn_bwd(dev["Q"], dev["K"], dev["V"], dev["W"], w.beta, w.P, w.L, True, dev["dO"], state)
    torch.cuda.synchronize()
    tol = TOL[dtype]
    for name, got, ref in zip(("dQ", "dK", "dV"), g_o, oracle_bwd(inp, True)):
        check(name, got, ref, tol)
    for name, a, b in zip(("dQ", "dK", "dV"), g_o, g_n):
        check(name + " (O given vs rebuilt)", a, to64(b), tol)
