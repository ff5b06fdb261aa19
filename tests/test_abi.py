"""C-ABI checks that need no GPU: the library loads, exports every function
include/race_attn.h declares, answers size queries, and rejects invalid
arguments on the host (nothing is launched in these tests)."""
import ctypes
import math
import os
import re

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "race_attn.h")

race = pytest.importorskip("linear_attention_soft_amd")


def _lib():
    if not os.path.exists(race.library_path):
        pytest.fail("librace_attn.so is not built (python -m linear_attention_soft_amd.build)")
    return race.lib()


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(race_[a-z_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = _declared_functions()
    for n in ("race_attn_fwd", "race_attn_bwd", "race_attn_state_bytes", "race_attn_workspace_bytes",
              "race_status_string", "race_last_error", "race_softbucket_debug"):
        assert n in names


def test_library_exports_every_declared_symbol():
    L = _lib()
    for n in _declared_functions():
        assert hasattr(L, n), n
    assert set(race.EXPORTED_SYMBOLS) == set(_declared_functions())


def test_status_strings():
    L = _lib()
    assert L.race_status_string(0) == b"RACE_OK"
    assert L.race_status_string(2) == b"RACE_ERR_UNSUPPORTED"


def _shape(B=1, H=2, N=1000, d=64, dtype=1, w_per_head=0):
    return race.race_shape(B, H, N, d, dtype, w_per_head)


def test_size_queries():
    s = _shape(N=4096, d=128)
    sb = race.race_attn_state_bytes(s, 4, 2, False)
    assert sb == 2 * 32 * 129 * 4            # B*H x LRP x (d + 1) float32
    assert race.race_attn_workspace_bytes(s, 4, 2, False, False) > 0
    assert race.race_attn_workspace_bytes(s, 4, 2, False, True) > 0
    # backward with dW adds float32 dPre of both sides: 2 x B*H*N x NHP, NHP = (LRP / 2^P) * P = 8 here
    for causal in (False, True):
        extra = (race.race_attn_workspace_bytes(s, 4, 2, causal, 2)
                 - race.race_attn_workspace_bytes(s, 4, 2, causal, 1))
        assert extra >= 2 * 2 * 4096 * 8 * 4
    assert race.race_attn_workspace_bytes(s, 4, 2, False, 3) == 0
    assert race.race_attn_workspace_bytes(s, 4, 2, False, 4) == 0     # no-state flag without a backward phase
    for causal in (False, True):
        for ph in (1, 2):
            assert (race.race_attn_workspace_bytes(s, 4, 2, causal, ph | 4)
                    > race.race_attn_workspace_bytes(s, 4, 2, causal, ph))


@pytest.mark.parametrize("d,D", [(96, 128), (72, 128), (40, 64), (8, 64)])
def test_head_dims_below_a_compiled_one(d, D):
    """A head dim d (a multiple of 8) below a compiled one D runs on D's
    kernels: the same state, plus room for zero-padded token tensors (forward:
    Q, K, V, O; backward: Q, K, V, dO, O, dQ, dK, dV; prefill: K, V)."""
    N, P, L = 4096, (4 if D == 128 else 3), 2
    s, t = _shape(N=N, d=d), _shape(N=N, d=D)
    tb = -(-2 * N * D * 2 // 256) * 256                # B*H x N x D bf16, 256-byte aligned
    for causal in (False, True):
        assert race.race_attn_state_bytes(s, P, L, causal) == race.race_attn_state_bytes(t, P, L, causal)
        for ph, n in ((0, 4), (1, 8), (2, 8), (5, 8)):
            assert (race.race_attn_workspace_bytes(s, P, L, causal, ph)
                    == race.race_attn_workspace_bytes(t, P, L, causal, ph) + n * tb)
    Lb = _lib()
    assert Lb.race_attn_decode_state_bytes(ctypes.byref(s), P, L) == Lb.race_attn_decode_state_bytes(ctypes.byref(t), P, L)
    assert (Lb.race_attn_decode_prefill_workspace_bytes(ctypes.byref(s), P, L)
            == Lb.race_attn_decode_prefill_workspace_bytes(ctypes.byref(t), P, L) + 2 * tb)
    # invalid arguments give 0
    assert race.race_attn_state_bytes(s, 0, 2, False) == 0
    assert race.race_attn_state_bytes(s, 4, 0, False) == 0
    assert race.race_attn_state_bytes(_shape(N=0), 4, 2, False) == 0


FAKE = 0x100000  # aligned, never dereferenced: every call below fails a host check first


def _fwd(shape, P=3, L=2, causal=0, beta=1.0, q=FAKE, o=FAKE + 0x10000000, ws=FAKE + 0x20000000, wsb=1 << 30,
         state=None, stateb=0):
    Lb = _lib()
    k, v, w = FAKE + 0x1000000, FAKE + 0x2000000, FAKE + 0x3000000
    return Lb.race_attn_fwd(q, k, v, w, ctypes.c_float(beta), P, L, causal, o,
                            ctypes.byref(shape) if shape is not None else None, state, stateb, ws, wsb, None)


@pytest.mark.parametrize("kw,code", [
    (dict(shape=None), 1),
    (dict(P=0), 1), (dict(P=9), 1), (dict(L=0), 1), (dict(causal=2), 1),
    (dict(beta=math.nan), 1), (dict(beta=math.inf), 1),
    (dict(q=None), 1),
    (dict(q=FAKE + 4), 1),                      # misaligned
    (dict(o=FAKE), 1),                          # O overlaps Q
    (dict(wsb=16), 3),                          # workspace too small
    (dict(ws=None), 3),
    (dict(state=FAKE + 0x30000000, stateb=8), 3),
    (dict(L=64), 2),                            # L * 2^P above 256
])
def test_forward_rejects_bad_arguments(kw, code):
    shape = kw.pop("shape", _shape())
    st = _fwd(shape, **kw)
    assert st == code, (kw, st, _lib().race_last_error())
    assert _lib().race_last_error() != b""


@pytest.mark.parametrize("shape,code", [
    (_shape(d=100), 2), (_shape(d=136), 2), (_shape(d=0), 1), (_shape(N=0), 1), (_shape(B=0), 1),
    (_shape(dtype=7), 1),
    (_shape(w_per_head=2), 1),
])
def test_forward_rejects_bad_shapes(shape, code):
    assert _fwd(shape) == code


def test_backward_rejects_bad_arguments():
    Lb = _lib()
    s = _shape()
    base = [FAKE + i * 0x1000000 for i in range(12)]

    def call(state=base[9], stateb=1 << 30, ws=base[10], wsb=1 << 30, beta=1.0, dq=base[6], dbeta=None, dW=None):
        return Lb.race_attn_bwd(base[0], base[1], base[2], base[3], ctypes.c_float(beta), 3, 2, 0, None, base[5],
                                dq, base[7], base[8], dbeta, dW, ctypes.byref(s), state, stateb, ws, wsb, None)

    wb_st = race.race_attn_workspace_bytes(s, 3, 2, False, 1)
    wb_nost = race.race_attn_workspace_bytes(s, 3, 2, False, 1 | 4)
    assert wb_nost > wb_st
    assert call(state=None, wsb=wb_st) == 3     # backward without a state needs the larger workspace
    assert call(state=base[6]) == 1             # state is dQ
    assert call(state=base[10]) == 1            # state is the workspace
    assert call(beta=math.nan) == 1
    assert call(stateb=4) == 3
    assert call(wsb=4) == 3
    assert call(dq=base[0]) == 1                # dQ overlaps Q
    assert call(dbeta=base[1] + 2) == 1         # dbeta misaligned
    assert call(dbeta=base[1] + 64) == 1        # dbeta inside K
    assert call(dW=base[11] + 2) == 1           # dW misaligned
    assert call(dW=base[2] + 64) == 1           # dW inside V
    assert call(dW=base[3]) == 1                # dW is W
    assert call(dW=base[11], dbeta=base[11] + 8) == 1   # dW overlaps dbeta
    wb1 = race.race_attn_workspace_bytes(s, 3, 2, False, 1)
    assert call(dW=base[11], wsb=wb1) == 3      # workspace sized for the backward without dW


def test_softbucket_debug_rejects_small_P():
    Lb = _lib()
    s = _shape()
    assert Lb.race_softbucket_debug(FAKE, FAKE + 0x1000000, ctypes.c_float(1.0), 2, 2, ctypes.byref(s),
                                    FAKE + 0x2000000, None) == 2


def test_decode_rejects_bad_arguments():
    Lb = _lib()
    s = _shape()
    base = [FAKE + i * 0x1000000 for i in range(8)]
    nb = Lb.race_attn_decode_state_bytes(ctypes.byref(s), 3, 2)
    assert nb > 0
    assert Lb.race_attn_decode_state_bytes(ctypes.byref(_shape(d=100)), 3, 2) == 0

    def call(q=base[0], state=base[5], sb=nb, beta=1.0, shape=s):
        return Lb.race_attn_decode(q, base[1], base[2], base[3], ctypes.c_float(beta), 3, 2, base[4],
                                   ctypes.byref(shape), state, sb, None)

    assert call(q=None) == 1
    assert call(state=None) == 1
    assert call(beta=math.inf) == 1
    assert call(sb=16) == 3
    assert call(q=base[0] + 4) == 1             # misaligned
    assert call(shape=_shape(d=100)) == 2
    wb = Lb.race_attn_decode_prefill_workspace_bytes(ctypes.byref(s), 3, 2)
    assert wb > 0
    assert Lb.race_attn_decode_prefill(base[1], base[2], base[3], ctypes.c_float(1.0), 3, 2, ctypes.byref(s),
                                       base[5], nb, None, 0, None) == 3
    assert Lb.race_attn_decode_prefill(base[1], base[2], base[3], ctypes.c_float(1.0), 3, 2, ctypes.byref(s),
                                       base[5], 8, base[6], wb, None) == 3


def test_plain_c_client(tmp_path):
    """The header compiles as C99 and a C program linked against the library
    sees the documented host-side contract (no GPU calls are made)."""
    import shutil
    import subprocess
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    lib = race.library_path
    if not os.path.exists(lib):
        pytest.skip("library not built")
    exe = tmp_path / "c_abi_check"
    src = os.path.join(os.path.dirname(__file__), "c_abi_check.c")
    r = subprocess.run([cc, "-std=c99", "-Wall", "-Werror", "-I", os.path.dirname(HEADER), src, lib,
                        f"-Wl,-rpath,{os.path.dirname(lib)}", "-o", str(exe)], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and r.stdout.strip() == "ok", (r.stdout, r.stderr)


def test_binding_rejects_mismatched_token_tensors():
    """The library takes one shape record for every token tensor, so the
    binding refuses tensors that differ from Q in shape, dtype or device
    before anything is launched (a shorter K would otherwise be read past
    its end)."""
    Q = torch.zeros(1, 2, 64, 64, dtype=torch.bfloat16)
    W = torch.zeros(2, 3, 64)
    short = torch.zeros(1, 2, 32, 64, dtype=torch.bfloat16)
    wrong_dtype = torch.zeros(1, 2, 64, 64)
    with pytest.raises(ValueError, match="K must have Q's shape"):
        race.race_attn_fwd(Q, short, Q, W, 1.0, 3, 2)
    with pytest.raises(ValueError, match="V must have Q's shape"):
        race.race_attn_fwd(Q, Q, wrong_dtype, W, 1.0, 3, 2)
    with pytest.raises(ValueError, match="O must have Q's shape"):
        race.race_attn_fwd(Q, Q, Q, W, 1.0, 3, 2, O=short)
    with pytest.raises(ValueError, match="dO must have Q's shape"):
        race.race_attn_bwd(Q, Q, Q, W, 1.0, 3, 2, False, short, None)
    with pytest.raises(ValueError, match="dK must have Q's shape"):
        race.race_attn_bwd(Q, Q, Q, W, 1.0, 3, 2, False, Q, None, dK=short)
    with pytest.raises(ValueError, match="V must have K's shape"):
        race.race_attn_decode_prefill(Q, short, W, 1.0, 3, 2)
    with pytest.raises(ValueError, match="O must have Q's shape"):
        race.race_attn_decode(Q, Q, Q, W, 1.0, 3, 2, None, O=wrong_dtype)


def test_build_lists_exactly_the_instance_files(tmp_path, monkeypatch):
    """build.py compiles the instance files the registry names; a missing
    listed file, or an instance file the registry does not name, is an error
    (a library silently missing kernel sets would only fail at run time)."""
    from linear_attention_soft_amd import build as B
    srcs = B.sources()
    assert srcs[-1] == "race_api.cpp"
    assert [f"race_inst_{n}.hip" for n in B.instance_names()] == srcs[:-1]
    fake = tmp_path / "csrc"
    fake.mkdir()
    for name in os.listdir(B.CSRC):
        (fake / name).write_bytes(open(os.path.join(B.CSRC, name), "rb").read())
    monkeypatch.setattr(B, "CSRC", str(fake))
    os.remove(fake / srcs[0])
    with pytest.raises(RuntimeError, match="missing"):
        B.sources()
    (fake / srcs[0]).write_text("// restored\n")
    (fake / "race_inst_unlisted.hip").write_text("// not in the registry\n")
    with pytest.raises(RuntimeError, match="not named"):
        B.sources()
