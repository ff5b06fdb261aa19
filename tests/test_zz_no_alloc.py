"""The allocation-free forward (race_attn_fwd_noalloc) against race_attn_fwd.

Both run the same kernels with the same plan, so O and the state must match
bit for bit; two calls in a row, the second on a smaller input, check that
nothing of the first call's scratch contents leaks into the second.  A call
whose scratch need exceeds the library's array is refused before anything is
enqueued.
"""
import ctypes
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


def _pair(w):
    inp = ri.make_inputs(w, device="cuda")
    W = inp["W"].cuda()
    Q, K, V = inp["Q"], inp["K"], inp["V"]
    shape = race._shape_of(Q, W, w.L, w.P)
    # both states start from the same bytes (alignment gaps are never written)
    nb = race.race_attn_state_bytes(shape, w.P, w.L, w.causal)
    st_ref = torch.full((nb,), 0x7f, dtype=torch.uint8, device="cuda")
    st = torch.full((nb,), 0x7f, dtype=torch.uint8, device="cuda")
    O_ref, _ = race.race_attn_fwd(Q, K, V, W, w.beta, w.P, w.L, w.causal, state=st_ref)
    O = torch.full_like(Q, float("nan"))
    race.race_attn_fwd_noalloc(Q, K, V, W, w.beta, w.P, w.L, w.causal, O, st)
    torch.cuda.synchronize()
    return O_ref, st_ref, O, st


@pytest.mark.parametrize("key,causal,sizes", [
    (4, False, ((1, 2, 40000), (1, 1, 5000))),
    (5, True, ((1, 2, 20000), (1, 2, 3000))),
    (2, True, ((2, 4, 1024), (1, 2, 300))),
    (1, False, ((1, 1, 1024), (1, 1, 77))),
])
def test_noalloc_forward_matches_forward(key, causal, sizes):
    for B, H, N in sizes:
        w = replace(ri.WORKLOADS[key].with_size(N=N, B=B, H=H), causal=causal)
        say(f"noalloc fwd {w.name} B={B} H={H} N={N} causal={causal}")
        O_ref, st_ref, O, st = _pair(w)
        assert torch.equal(O, O_ref), "O differs from race_attn_fwd"
        assert torch.equal(st, st_ref), "state differs from race_attn_fwd"


def test_noalloc_forward_without_state():
    w = ri.WORKLOADS[4].with_size(N=9000, B=1, H=2)
    inp = ri.make_inputs(w, device="cuda")
    W = inp["W"].cuda()
    O_ref, _ = race.race_attn_fwd(inp["Q"], inp["K"], inp["V"], W, w.beta, w.P, w.L, False)
    O = torch.empty_like(O_ref)
    race.race_attn_fwd_noalloc(inp["Q"], inp["K"], inp["V"], W, w.beta, w.P, w.L, False, O, None)
    torch.cuda.synchronize()
    assert torch.equal(O, O_ref)


def test_noalloc_forward_refuses_beyond_its_scratch():
    """Causal P = 6, L = 4 over 1M tokens without a state needs the segment
    banks, their sums and Den (about 84 MB): more than the 64 MiB array."""
    cap = race.lib().race_attn_fwd_noalloc_scratch_bytes()
    assert cap == 64 << 20
    w = ri.WORKLOADS[5]
    Q = torch.empty((w.B, w.H, w.N, w.d), dtype=torch.bfloat16, device="cuda")
    K, V, O = torch.empty_like(Q), torch.empty_like(Q), torch.empty_like(Q)
    W = ri.make_W(w).cuda()
    with pytest.raises(race.RaceError, match="scratch"):
        race.race_attn_fwd_noalloc(Q, K, V, W, w.beta, w.P, w.L, True, O, None)
    assert race.lib().race_last_error().decode().startswith("this call needs")
    torch.cuda.synchronize()
