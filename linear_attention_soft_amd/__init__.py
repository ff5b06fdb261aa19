"""Python binding of the gfx950 RACE attention library (librace_attn.so).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI declared in ``include/race_attn.h``.  PyTorch
provides device memory and the current stream.  There is no fallback: if the
library is missing or a call fails, an exception is raised.
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "RaceError", "lib", "library_path", "race_attn_fwd", "race_attn_bwd", "race_softbucket_debug",
    "race_attn_state_bytes", "race_attn_workspace_bytes", "race_attn_decode_prefill", "race_attn_decode",
    "race_attn_decode_state_bytes", "race_attn_fwd_noalloc", "race_bucket_stats_segments",
    "race_bucket_stats_debug", "EXPORTED_SYMBOLS",
]

_PKG = os.path.dirname(os.path.abspath(__file__))
# RACE_ATTN_LIBRARY selects another build of the same library (the host
# sanitizer build of the CPU tests); by default the in-place build is loaded.
library_path = os.environ.get("RACE_ATTN_LIBRARY") or os.path.join(_PKG, "librace_attn.so")

RACE_F32, RACE_BF16 = 0, 1
RACE_WS_FWD, RACE_WS_BWD, RACE_WS_BWD_DW, RACE_WS_NO_STATE = 0, 1, 2, 4
EXPORTED_SYMBOLS = ("race_attn_fwd", "race_attn_bwd", "race_attn_state_bytes", "race_attn_workspace_bytes",
                    "race_softbucket_debug", "race_status_string", "race_last_error", "race_profile_enable",
                    "race_profile_reset", "race_profile_report", "race_attn_decode_state_bytes",
                    "race_attn_decode_prefill_workspace_bytes", "race_attn_decode_prefill", "race_attn_decode",
                    "race_attn_fwd_noalloc", "race_attn_fwd_noalloc_scratch_bytes", "race_bucket_stats_segments",
                    "race_bucket_stats_debug")


class RaceError(RuntimeError):
    def __init__(self, status: int, name: str, msg: str):
        super().__init__(f"{name}: {msg}")
        self.status = status
        self.name = name


class race_shape(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int64), ("H", ctypes.c_int64), ("N", ctypes.c_int64), ("d", ctypes.c_int64),
                ("dtype", ctypes.c_int32), ("w_per_head", ctypes.c_int32)]


_LIB = None


def lib() -> ctypes.CDLL:
    """Load librace_attn.so (built in place by ``linear_attention_soft_amd.build``)."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(library_path):
            raise RuntimeError(f"{library_path} is missing; build it with "
                               f"`python -m linear_attention_soft_amd.build`")
        L = ctypes.CDLL(library_path)
        vp, sz, i32, f32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_float
        sp = ctypes.POINTER(race_shape)
        L.race_attn_state_bytes.argtypes = [sp, i32, i32, i32]
        L.race_attn_state_bytes.restype = sz
        L.race_attn_workspace_bytes.argtypes = [sp, i32, i32, i32, i32]
        L.race_attn_workspace_bytes.restype = sz
        L.race_attn_fwd.argtypes = [vp, vp, vp, vp, f32, i32, i32, i32, vp, sp, vp, sz, vp, sz, vp]
        L.race_attn_fwd.restype = i32
        L.race_attn_bwd.argtypes = [vp, vp, vp, vp, f32, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp, sp, vp, sz, vp, sz,
                                    vp]
        L.race_attn_bwd.restype = i32
        L.race_softbucket_debug.argtypes = [vp, vp, f32, i32, i32, sp, vp, vp]
        L.race_softbucket_debug.restype = i32
        L.race_status_string.argtypes = [i32]
        L.race_status_string.restype = ctypes.c_char_p
        L.race_last_error.argtypes = []
        L.race_last_error.restype = ctypes.c_char_p
        L.race_profile_enable.argtypes = [i32]
        L.race_profile_enable.restype = i32
        L.race_profile_reset.argtypes = []
        L.race_profile_reset.restype = None
        L.race_profile_report.argtypes = [ctypes.c_char_p, sz]
        L.race_profile_report.restype = sz
        L.race_attn_decode_state_bytes.argtypes = [sp, i32, i32]
        L.race_attn_decode_state_bytes.restype = sz
        L.race_attn_decode_prefill_workspace_bytes.argtypes = [sp, i32, i32]
        L.race_attn_decode_prefill_workspace_bytes.restype = sz
        L.race_attn_decode_prefill.argtypes = [vp, vp, vp, f32, i32, i32, sp, vp, sz, vp, sz, vp]
        L.race_attn_decode_prefill.restype = i32
        L.race_attn_decode.argtypes = [vp, vp, vp, vp, f32, i32, i32, vp, sp, vp, sz, vp]
        L.race_attn_decode.restype = i32
        L.race_bucket_stats_segments.argtypes = [sp, i32, i32, i32, ctypes.POINTER(ctypes.c_int64)]
        L.race_bucket_stats_segments.restype = i32
        L.race_bucket_stats_debug.argtypes = [sp, i32, i32, i32, vp, sz, vp, sz, vp, vp, vp, vp, vp]
        L.race_bucket_stats_debug.restype = i32
        L.race_attn_fwd_noalloc.argtypes = [vp, vp, vp, vp, f32, i32, i32, i32, vp, sp, vp, sz, vp]
        L.race_attn_fwd_noalloc.restype = i32
        L.race_attn_fwd_noalloc_scratch_bytes.argtypes = []
        L.race_attn_fwd_noalloc_scratch_bytes.restype = sz
        _LIB = L
    return _LIB


def _check(status: int):
    if status != 0:
        L = lib()
        raise RaceError(status, L.race_status_string(status).decode(), L.race_last_error().decode())


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return RACE_F32
    if t.dtype == torch.bfloat16:
        return RACE_BF16
    raise TypeError(f"unsupported dtype {t.dtype}; use float32 or bfloat16")


def make_shape(B, H, N, d, dtype, w_per_head=False) -> race_shape:
    code = dtype if isinstance(dtype, int) else (RACE_BF16 if dtype == torch.bfloat16 else RACE_F32)
    return race_shape(int(B), int(H), int(N), int(d), code, int(bool(w_per_head)))


def _shape_of(x: torch.Tensor, W: torch.Tensor = None, L: int = None, P: int = None) -> race_shape:
    """Shape record of the token tensor x; W of shape [L, P, d] is shared by
    every head, W of shape [H, L, P, d] holds one set of tables per head."""
    if x.dim() != 4:
        raise ValueError("tensors must be [B, H, N, d]")
    B, H, N, d = x.shape
    per_head = 0
    if W is not None:
        if W.dim() == 4:
            per_head = 1
            if W.shape[0] != H:
                raise ValueError(f"per-head tables must be [H, L, P, d] with H = {H}")
        elif W.dim() != 3:
            raise ValueError("W must be [L, P, d] or [H, L, P, d]")
        if W.dtype != torch.float32 or W.shape[-1] != d or (L is not None and W.shape[-3] != L) or \
                (P is not None and W.shape[-2] != P):
            raise ValueError(f"W must be float32 [.., L={L}, P={P}, d={d}]")
    return race_shape(B, H, N, d, _dtype_code(x), per_head)


def _like(ref: torch.Tensor, ref_name: str, **tensors):
    """Every given token tensor must match ref's shape, dtype and device: the
    library receives one shape record and would read or write past the end
    of a smaller tensor."""
    for name, t in tensors.items():
        if t is None:
            continue
        if tuple(t.shape) != tuple(ref.shape) or t.dtype != ref.dtype or t.device != ref.device:
            raise ValueError(f"{name} must have {ref_name}'s shape {tuple(ref.shape)}, dtype {ref.dtype} and "
                             f"device {ref.device}; got {tuple(t.shape)}, {t.dtype}, {t.device}")


def _same_device(ref: torch.Tensor, **tensors):
    for name, t in tensors.items():
        if t is not None and t.device != ref.device:
            raise ValueError(f"{name} must be on {ref.device}; got {t.device}")


def _dev(t: torch.Tensor, name: str) -> int:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _torch_stream(stream, device) -> torch.cuda.Stream:
    """The launch stream as a torch stream: None is the current stream of
    device; a raw hipStream_t (int) is wrapped without taking ownership."""
    if stream is None:
        return torch.cuda.current_stream(device)
    if isinstance(stream, torch.cuda.Stream):
        return stream
    if hasattr(stream, "cuda_stream"):
        return torch.cuda.ExternalStream(stream.cuda_stream, device=device)
    return torch.cuda.ExternalStream(int(stream), device=device)


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def race_attn_state_bytes(shape: race_shape, P: int, L: int, causal: bool) -> int:
    return int(lib().race_attn_state_bytes(ctypes.byref(shape), P, L, int(causal)))


def race_attn_workspace_bytes(shape: race_shape, P: int, L: int, causal: bool, is_bwd) -> int:
    """is_bwd: 0 / False forward, 1 / True backward, 2 backward with dW."""
    return int(lib().race_attn_workspace_bytes(ctypes.byref(shape), P, L, int(causal), int(is_bwd)))


def _bytes(t):
    return t.numel() * t.element_size() if t is not None else 0


def _buffer(nbytes: int, device, given=None):
    """Caller's buffer, or a new one.  New buffers are allocated while the
    launch stream is current (see _on), so the caching allocator hands their
    memory to no other stream's allocation before the kernels that use it
    have finished."""
    if given is not None:
        return given
    return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)


def _on(stream, device):
    """Context in which the binding allocates the buffers of one call: the
    launch stream is current, so workspaces freed on return are reused only
    by later work on that stream."""
    return torch.cuda.stream(_torch_stream(stream, device))


def race_attn_fwd(Q, K, V, W, beta, P, L, causal=False, O=None, state=None, workspace=None, stream=None):
    """O = RACE(Q, K, V; W, beta, P, L, causal).  Returns (O, state).  W is
    [L, P, d] (every head) or [H, L, P, d] (per head)."""
    shape = _shape_of(Q, W, L, P)
    _like(Q, "Q", K=K, V=V, O=O)
    _same_device(Q, W=W, state=state, workspace=workspace)
    sb = race_attn_state_bytes(shape, P, L, causal)
    wb = race_attn_workspace_bytes(shape, P, L, causal, RACE_WS_FWD)
    if sb == 0 or wb == 0:
        # surface the library's own diagnosis
        _check(lib().race_attn_fwd(None, None, None, None, float(beta), P, L, int(causal), None,
                                   ctypes.byref(shape), None, 0, None, 0, None))
    with _on(stream, Q.device):
        O = torch.empty_like(Q) if O is None else O
        state = _buffer(sb, Q.device, state)
        workspace = _buffer(wb, Q.device, workspace)
        _check(lib().race_attn_fwd(_dev(Q, "Q"), _dev(K, "K"), _dev(V, "V"), _dev(W, "W"), float(beta), int(P),
                                   int(L), int(causal), _dev(O, "O"), ctypes.byref(shape), _dev(state, "state"),
                                   _bytes(state), _dev(workspace, "workspace"), _bytes(workspace), _stream(stream)))
    return O, state


def race_attn_fwd_noalloc(Q, K, V, W, beta, P, L, causal, O, state, stream=None):
    """The allocation-free forward: O and state are the caller's tensors
    (state sized by race_attn_state_bytes, or None); the library's own
    device scratch replaces the workspace.  Nothing is allocated."""
    shape = _shape_of(Q, W, L, P)
    _like(Q, "Q", K=K, V=V, O=O)
    _same_device(Q, W=W, state=state)
    _check(lib().race_attn_fwd_noalloc(_dev(Q, "Q"), _dev(K, "K"), _dev(V, "V"), _dev(W, "W"), float(beta), int(P),
                                       int(L), int(causal), _dev(O, "O"), ctypes.byref(shape),
                                       _dev(state, "state") if state is not None else None, _bytes(state),
                                       _stream(stream)))
    return O, state


def race_attn_bwd(Q, K, V, W, beta, P, L, causal, dO, state, O=None, dQ=None, dK=None, dV=None,
                  dbeta=None, dW=None, workspace=None, stream=None):
    """Exact gradients of sum(O * dO).  Returns (dQ, dK, dV), followed by
    dbeta when dbeta is True (a new float32 tensor of one element) or a
    float32 device tensor to write dL/dbeta into, then by dW when dW is True
    (a new float32 tensor shaped like W) or a float32 device tensor of W's
    shape to write dL/dW into.  state is race_attn_fwd's state, or None: the
    library then rebuilds it inside the workspace."""
    shape = _shape_of(Q, W, L, P)
    _like(Q, "Q", K=K, V=V, dO=dO, O=O, dQ=dQ, dK=dK, dV=dV)
    _same_device(Q, W=W, state=state, workspace=workspace)
    want_dbeta = dbeta is not None and dbeta is not False
    if want_dbeta and dbeta is not True and (dbeta.dtype != torch.float32 or not dbeta.is_cuda or
                                             dbeta.numel() < 1):
        raise ValueError("dbeta must be a float32 device tensor with at least one element")
    want_dW = dW is not None and dW is not False
    if want_dW and dW is not True and (dW.dtype != torch.float32 or not dW.is_cuda or dW.shape != W.shape):
        raise ValueError("dW must be a float32 device tensor shaped like W")
    phase = (RACE_WS_BWD_DW if want_dW else RACE_WS_BWD) | (RACE_WS_NO_STATE if state is None else 0)
    wb = race_attn_workspace_bytes(shape, P, L, causal, phase)
    if wb == 0:
        _check(lib().race_attn_bwd(None, None, None, None, float(beta), P, L, int(causal), None, None, None, None,
                                   None, None, None, ctypes.byref(shape), None, 0, None, 0, None))
    with _on(stream, Q.device):
        dQ = torch.empty_like(Q) if dQ is None else dQ
        dK = torch.empty_like(K) if dK is None else dK
        dV = torch.empty_like(V) if dV is None else dV
        if dbeta is True:
            dbeta = torch.zeros(1, dtype=torch.float32, device=Q.device)
        if dW is True:
            dW = torch.empty_like(W)
        workspace = _buffer(wb, Q.device, workspace)
        _check(lib().race_attn_bwd(_dev(Q, "Q"), _dev(K, "K"), _dev(V, "V"), _dev(W, "W"), float(beta), int(P),
                                   int(L), int(causal), _dev(O, "O") if O is not None else None, _dev(dO, "dO"),
                                   _dev(dQ, "dQ"), _dev(dK, "dK"), _dev(dV, "dV"),
                                   dbeta.data_ptr() if want_dbeta else None,
                                   _dev(dW, "dW") if want_dW else None, ctypes.byref(shape),
                                   _dev(state, "state") if state is not None else None,
                                   _bytes(state), _dev(workspace, "workspace"),
                                   _bytes(workspace), _stream(stream)))
    return (dQ, dK, dV) + ((dbeta,) if want_dbeta else ()) + ((dW,) if want_dW else ())


def profile_enable(on: bool = True):
    """Bracket every kernel launch with HIP events on its stream (see race_profile_report)."""
    lib().race_profile_enable(int(on))


def profile_reset():
    lib().race_profile_reset()


def profile_report() -> dict:
    """{kernel name: (launches, total ms)} of the launches recorded since the last reset."""
    L = lib()
    n = L.race_profile_report(None, 0)
    buf = ctypes.create_string_buffer(n + 16)
    L.race_profile_report(buf, len(buf))
    out = {}
    for line in buf.value.decode().splitlines():
        name, cnt, ms = line.split("\t")
        out[name] = (int(cnt), float(ms))
    return out


def race_softbucket_debug(X, W, beta, P, L, stream=None):
    """Soft assignments phi^(l)(X) as float32 [B, H, N, L, 2^P] (test export)."""
    shape = _shape_of(X, W, L, P)
    _same_device(X, W=W)
    B, H, N, d = X.shape
    with _on(stream, X.device):
        out = torch.empty((B, H, N, L, 1 << P), dtype=torch.float32, device=X.device)
        _check(lib().race_softbucket_debug(_dev(X, "X"), _dev(W, "W"), float(beta), int(P), int(L),
                                           ctypes.byref(shape), _dev(out, "phi"), _stream(stream)))
    return out


def race_bucket_stats_segments(shape: race_shape, P: int, L: int, causal: bool):
    """(banks per (batch, head), tokens per segment) of the bank export."""
    seg = ctypes.c_int64(0)
    n = lib().race_bucket_stats_segments(ctypes.byref(shape), int(P), int(L), int(causal), ctypes.byref(seg))
    if n == 0:
        raise ValueError("invalid or unsupported arguments")
    return int(n), int(seg.value)


def race_bucket_stats_debug(Q, W, P, L, causal, state=None, workspace=None, stream=None):
    """Banks left by race_attn_fwd in state and by race_attn_bwd in its
    workspace (test export), as float32 tensors
    (content [B, H, S, L, 2^P, d], mass [B, H, S, L, 2^P],
     dcontent, dmass likewise; None where the source is None).  Q gives the
    shape and dtype of the calls that filled them."""
    shape = _shape_of(Q, W, L, P)
    S, _ = race_bucket_stats_segments(shape, P, L, causal)
    B, H, N, d = Q.shape
    R = 1 << P
    mk = lambda *sh: torch.empty(sh, dtype=torch.float32, device=Q.device)
    with _on(stream, Q.device):
        c = mk(B, H, S, L, R, d) if state is not None else None
        m = mk(B, H, S, L, R) if state is not None else None
        dc = mk(B, H, S, L, R, d) if workspace is not None else None
        dm = mk(B, H, S, L, R) if workspace is not None else None
        p = lambda t: t.data_ptr() if t is not None else None
        _check(lib().race_bucket_stats_debug(ctypes.byref(shape), int(P), int(L), int(causal), p(state), _bytes(state),
                                             p(workspace), _bytes(workspace), p(c), p(m), p(dc), p(dm),
                                             _stream(stream)))
    return c, m, dc, dm


def race_attn_decode_state_bytes(shape: race_shape, P: int, L: int) -> int:
    return lib().race_attn_decode_state_bytes(ctypes.byref(shape), int(P), int(L))


def race_attn_decode_prefill(K, V, W, beta, P, L, state=None, workspace=None, stream=None):
    """Decode state (float32 bank: content [B*H][LRP][d] then mass [B*H][LRP])
    after the prompt K, V [B, H, N, d].  Returns the state tensor."""
    shape = _shape_of(K, W, L, P)
    _like(K, "K", V=V)
    _same_device(K, W=W, state=state, workspace=workspace)
    nb = race_attn_decode_state_bytes(shape, P, L)
    if nb == 0:
        _check(lib().race_attn_decode_prefill(None, None, None, float(beta), int(P), int(L), ctypes.byref(shape),
                                              None, 0, None, 0, None))
    wb = lib().race_attn_decode_prefill_workspace_bytes(ctypes.byref(shape), int(P), int(L))
    with _on(stream, K.device):
        if state is None:
            state = torch.empty(nb // 4, dtype=torch.float32, device=K.device)
        workspace = _buffer(wb, K.device, workspace)
        _check(lib().race_attn_decode_prefill(_dev(K, "K"), _dev(V, "V"), _dev(W, "W"), float(beta), int(P),
                                              int(L), ctypes.byref(shape), _dev(state, "state"), _bytes(state),
                                              _dev(workspace, "workspace"), _bytes(workspace), _stream(stream)))
    return state


def race_attn_decode(Q, K, V, W, beta, P, L, state, O=None, stream=None):
    """Decode the new tokens Q, K, V [B, H, n, d] in order from state (updated
    in place; a zeroed state is the empty prefix).  Returns O."""
    shape = _shape_of(Q, W, L, P)
    _like(Q, "Q", K=K, V=V, O=O)
    _same_device(Q, W=W, state=state)
    with _on(stream, Q.device):
        O = torch.empty_like(Q) if O is None else O
        _check(lib().race_attn_decode(_dev(Q, "Q"), _dev(K, "K"), _dev(V, "V"), _dev(W, "W"), float(beta), int(P),
                                      int(L), _dev(O, "O"), ctypes.byref(shape), _dev(state, "state"),
                                      _bytes(state), _stream(stream)))
    return O
