"""Causal linear attention with a fixed-size running state on MI355X (gfx950).

Thin Python layer over the C ABI of liblinattn.so (include/linattn.h): it
checks tensors, allocates outputs/workspace with PyTorch and passes raw device
pointers and torch's current HIP stream.  Every step of the computation runs
in the library's HIP kernels; there is no Python or CPU fallback.

    out, S, z = prefill(q, k, v)                   # q, k, v: [B, H, T, d] on cuda
    o = decode_step(q1, k1, v1, S, z)              # one token, updates S, z in place

mLSTM gates (identity features, forget and exponential input gates, the
max(|den|, 1) read-out and a stabiliser m carried with the state):

    out, S, z, m = prefill(q, k, v, phi="identity", igate=ig, fgate=fg, normalize="max1")
    o = decode_step(q1, k1, v1, S, z, phi="identity", igate=ig1, fgate=fg1, stab=m,
                    normalize="max1")
"""
from __future__ import annotations

import ctypes
from typing import Optional, Tuple

from . import _lib
from ._lib import LinAttnError  # noqa: F401

__all__ = ["prefill", "prefill_stage", "prefill_backward", "decode_step", "state_init",
           "feature_dim", "prefill_plan", "prefill_workspace_size", "make_desc", "LinAttnError"]


def _torch():
    import torch
    return torch


def _dtype_code(dt):
    torch = _torch()
    codes = {torch.float32: _lib.LA_F32, torch.bfloat16: _lib.LA_BF16, torch.float16: _lib.LA_F16}
    if dt not in codes:
        raise TypeError(f"unsupported element type {dt}; use float32, bfloat16 or float16")
    return codes[dt]


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _need(t, name, device=None, dtype=None, shape=None):
    if t is None:
        raise ValueError(f"{name} is required")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a CUDA (HIP) tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _check_W(W, phi, H, d_h, device):
    """The random-feature matrix of every head: [H, rff_D, d_h] fp32,
    contiguous, on q's device.  The kernels index it by head and input
    feature, so any other shape would be read out of bounds."""
    torch = _torch()
    if phi != "rff":
        if W is not None:
            raise ValueError(f"W is only used by the random-feature map, not {phi!r}")
        return
    if W is None:
        raise ValueError("phi='rff' needs W [H, rff_D, d_h]")
    if W.dim() != 3 or W.shape[0] != H or W.shape[2] != d_h or W.shape[1] < 1:
        raise ValueError(f"W has shape {tuple(W.shape)}, expected ({H}, rff_D, {d_h})")
    _need(W, "W", device=device, dtype=torch.float32)


_NORMS = {True: _lib.LA_NORM_SUM, "sum": _lib.LA_NORM_SUM, False: _lib.LA_NORM_NONE,
          "none": _lib.LA_NORM_NONE, "max1": _lib.LA_NORM_MAX1}


def _norm_code(normalize):
    for key, code in _NORMS.items():
        if normalize is key or (isinstance(key, str) and normalize == key):
            return code
    raise ValueError(f"unknown read-out {normalize!r}; use True, False or 'max1'")


def make_desc(B, H, T, d_h, d_v, dtype_code, phi="elu1", W=None, rff_D=None, decay=None,
              gate=None, eps=1e-6, chunk=0, segments=0, out_dtype_code=None,
              normalize=True, causal=True, igate=None, fgate=None, fgate_exp=False,
              stab=None) -> _lib.LaDesc:
    """Build an `la_desc`.  `decay` (SSD a_t), `gate` (RFA g_t) and the mLSTM
    gates (`fgate` forget and `igate` input pre-activations, with the
    stabiliser tensor `stab`) are exclusive; `out_dtype_code` defaults to the
    input type; `normalize` is True (phi(q).S / (phi(q).z + eps)), False (the
    numerator alone) or "max1" (divided by max(|phi(q).z|, 1)); `causal=False`
    the non-causal prefill."""
    d = _lib.LaDesc()
    d.B, d.H, d.T, d.d_h, d.d_v = int(B), int(H), int(T), int(d_h), int(d_v)
    d.dtype = int(dtype_code)
    d.out_dtype = int(dtype_code if out_dtype_code is None else out_dtype_code)
    if phi == "elu1":
        d.phi, d.rff_D, d.rff_W = _lib.LA_PHI_ELU1, 0, None
    elif phi == "rff":
        d.phi = _lib.LA_PHI_RFF
        d.rff_D = int(rff_D if rff_D is not None else (W.shape[-2] if W is not None else 0))
        d.rff_W = None if W is None else W.data_ptr()
    elif phi == "identity":
        d.phi, d.rff_D, d.rff_W = _lib.LA_PHI_IDENTITY, 0, None
    else:
        raise ValueError(f"unknown feature map {phi!r}")
    mlstm = igate is not None or fgate is not None
    if sum(x is not None for x in (decay, gate)) + (1 if mlstm else 0) > 1:
        raise ValueError("decay, gate and the mLSTM gates are exclusive")
    d.igate, d.fgate_exp, d.stab = None, 0, None
    if decay is not None:
        d.decay_kind, d.decay = _lib.LA_DECAY_SSD, decay.data_ptr()
    elif gate is not None:
        d.decay_kind, d.decay = _lib.LA_GATE_RFA, gate.data_ptr()
    elif mlstm:
        if igate is None or fgate is None:
            raise ValueError("the mLSTM gates need both igate and fgate")
        d.decay_kind, d.decay = _lib.LA_GATE_MLSTM, fgate.data_ptr()
        d.igate, d.fgate_exp = igate.data_ptr(), int(bool(fgate_exp))
        d.stab = None if stab is None else stab.data_ptr()
    else:
        d.decay_kind, d.decay = _lib.LA_DECAY_NONE, None
    d.eps = float(eps)
    d.chunk, d.segments = int(chunk), int(segments)
    d.norm = _norm_code(normalize)
    d.noncausal = 0 if causal else 1
    return d


def feature_dim(d_h: int, phi: str = "elu1", rff_D: int = 0) -> int:
    return 2 * rff_D if phi == "rff" else d_h


def _stream(device):
    return ctypes.c_void_p(_torch().cuda.current_stream(device).cuda_stream)


def state_init(B: int, H: int, d_prime: int, d_v: int, device="cuda", stab: bool = False):
    """Allocate a state (S [B,H,d',d_v], z [B,H,d'], fp32) and zero it with
    la_state_init; with stab=True also the mLSTM stabiliser m [B,H] (zero),
    returned as a third tensor."""
    torch = _torch()
    device = torch.device(device)
    S = torch.empty(B, H, d_prime, d_v, dtype=torch.float32, device=device)
    z = torch.empty(B, H, d_prime, dtype=torch.float32, device=device)
    if stab:
        m = torch.empty(B, H, dtype=torch.float32, device=device)
        g = torch.empty(1, dtype=torch.float32, device=device)   # stands in for the gates
        desc = make_desc(B, H, 0, d_prime, d_v, _lib.LA_F32, phi="identity", igate=g, fgate=g,
                         stab=m)
    else:
        desc = make_desc(B, H, 0, d_prime, d_v, _lib.LA_F32)
    _lib.check(_lib.lib().la_state_init(ctypes.byref(desc), _ptr(S), _ptr(z), _stream(device)))
    return (S, z, m) if stab else (S, z)


def _prefill_desc(q, k, v, phi, W, decay, gate, eps, chunk, segments, out_dtype=None,
                  normalize=True, causal=True, igate=None, fgate=None, fgate_exp=False,
                  stab=None):
    torch = _torch()
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, n, device=q.device, dtype=q.dtype)
    if q.dim() != 4:
        raise ValueError("q, k, v must be [B, H, T, d]")
    B, H, T, d_h = q.shape
    _need(k, "k", shape=(B, H, T, d_h))
    d_v = v.shape[-1]
    _need(v, "v", shape=(B, H, T, d_v))
    _check_W(W, phi, H, d_h, q.device)
    for a, n in ((decay, "decay"), (gate, "gate"), (igate, "igate"), (fgate, "fgate")):
        if a is not None:
            _need(a, n, device=q.device, dtype=torch.float32, shape=(B, H, T))
    if stab is not None:
        _need(stab, "stab", device=q.device, dtype=torch.float32, shape=(B, H))
    desc = make_desc(B, H, T, d_h, d_v, _dtype_code(q.dtype), phi, W, None, decay, gate, eps,
                     chunk, segments, _dtype_code(out_dtype or q.dtype), normalize, causal,
                     igate, fgate, fgate_exp, stab)
    return desc, (B, H, T, d_h, d_v)


def prefill_workspace_size(desc: _lib.LaDesc) -> int:
    n = ctypes.c_size_t(0)
    _lib.check(_lib.lib().la_prefill_workspace_size(ctypes.byref(desc), ctypes.byref(n)))
    return int(n.value)


def prefill_plan(desc: _lib.LaDesc):
    """(chunk, segments, path) la_prefill will use (path 1 = chunked MFMA)."""
    c, s, p = ctypes.c_int(0), ctypes.c_int(0), ctypes.c_int(0)
    _lib.check(_lib.lib().la_prefill_plan(ctypes.byref(desc), ctypes.byref(c), ctypes.byref(s),
                                          ctypes.byref(p)))
    return c.value, s.value, p.value


def prefill(q, k, v, *, phi: str = "elu1", W=None, decay=None, gate=None, eps: float = 1e-6,
            state: Optional[tuple] = None, chunk: int = 0, segments: int = 0, out=None,
            workspace=None, out_dtype=None, normalize=True, causal: bool = True,
            igate=None, fgate=None, fgate_exp: bool = False):
    """Causal linear attention over [B, H, T, d] inputs on the GPU.

    Returns (out, S, z).  If `state=(S, z)` is given the recurrence continues
    from it and the final state is written back into those tensors (in place);
    otherwise a zero state is allocated.  `out_dtype` is q's dtype (default)
    or torch.float32.  `normalize=False` returns the numerator phi(q)^T S
    alone (LA_NORM_NONE); z is still carried; "max1" divides by
    max(|phi(q)^T z|, 1).  `causal=False` is the non-causal form: the state
    takes in the whole sequence, then every token reads it out.

    mLSTM gates: `fgate` and `igate` ([B, H, T] fp32 pre-activations; forget
    gate sigmoid(fgate), or exp(fgate) with fgate_exp=True; input gate
    exp(igate)).  The state then carries the stabiliser m [B, H]: `state` is
    (S, z, m) and the result (out, S, z, m), with S, z held scaled by e^{-m}.
    """
    torch = _torch()
    out_dtype = out_dtype or q.dtype
    mlstm = igate is not None or fgate is not None
    if q.dim() != 4:
        raise ValueError("q, k, v must be [B, H, T, d]")
    B, H = q.shape[0], q.shape[1]
    _check_W(W, phi, H, q.shape[-1], q.device)
    if state is None:
        dp = feature_dim(q.shape[-1], phi, W.shape[-2] if W is not None else 0)
        st = state_init(B, H, dp, v.shape[-1], q.device, stab=mlstm)
    else:
        st = tuple(state)
        if len(st) != (3 if mlstm else 2):
            raise ValueError("state is (S, z, m) with the mLSTM gates, (S, z) otherwise")
    m = st[2] if mlstm else None
    desc, (B, H, T, d_h, d_v) = _prefill_desc(q, k, v, phi, W, decay, gate, eps, chunk, segments,
                                              out_dtype, normalize, causal, igate, fgate,
                                              fgate_exp, m)
    dp = feature_dim(d_h, phi, desc.rff_D)
    S, z = st[0], st[1]
    _need(S, "S", device=q.device, dtype=torch.float32, shape=(B, H, dp, d_v))
    _need(z, "z", device=q.device, dtype=torch.float32, shape=(B, H, dp))
    if out is None:
        out = torch.empty(B, H, T, d_v, dtype=out_dtype, device=q.device)
    else:
        _need(out, "out", device=q.device, dtype=out_dtype, shape=(B, H, T, d_v))
    nws = prefill_workspace_size(desc)
    if nws and (workspace is None or workspace.numel() * workspace.element_size() < nws):
        workspace = torch.empty(nws, dtype=torch.uint8, device=q.device)
    _lib.check(_lib.lib().la_prefill(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(S), _ptr(z),
                                     _ptr(out), _ptr(workspace) if nws else None, nws,
                                     _stream(q.device)))
    return (out, S, z, m) if mlstm else (out, S, z)


def prefill_stage(stage: int, q, k, v, S, z, out, workspace, *, phi="elu1", W=None, decay=None,
                  gate=None, eps=1e-6, chunk=0, segments=0, normalize=True, causal=True,
                  igate=None, fgate=None, fgate_exp=False, stab=None):
    """Run one of la_prefill's three stages (1 segment states, 2 scan, 3 outputs);
    out's dtype selects the output type."""
    desc, _ = _prefill_desc(q, k, v, phi, W, decay, gate, eps, chunk, segments, out.dtype,
                            normalize, causal, igate, fgate, fgate_exp, stab)
    nws = prefill_workspace_size(desc)
    _lib.check(_lib.lib().la_prefill_stage(ctypes.byref(desc), int(stage), _ptr(q), _ptr(k), _ptr(v),
                                           _ptr(S), _ptr(z), _ptr(out),
                                           _ptr(workspace) if nws else None, nws,
                                           _stream(q.device)))


def prefill_backward(q, k, v, dout, *, phi: str = "elu1", decay=None, gate=None,
                     eps: float = 1e-6, state: Optional[tuple] = None, normalize=True,
                     state_grad: bool = False, segments: int = 0, workspace=None,
                     igate=None, fgate=None, fgate_exp: bool = False):
    """Gradients of L = sum <dout, out> for la.prefill(q, k, v, ...) from the
    initial state `state=(S0, z0)` (zero if None).  dout has out's layout and
    dtype (q's, or float32).  Returns a dict of fp32 tensors: dq, dk, dv, and
    ddecay (with `decay`) or dgate (with `gate`), and dS0, dz0 when
    state_grad=True.  `segments` (0 = the default plan) sets how many runs of
    32-token chunks each sequence is cut into on the chunked path.

    mLSTM gates (`igate`, `fgate`, `fgate_exp` as for prefill, identity
    features): `state` is the scaled (S0, z0, m0); the result has dfgate and
    digate, and dS0, dz0 are the gradients of the scaled state."""
    torch = _torch()
    mlstm = igate is not None or fgate is not None
    stab = None
    if mlstm:
        B_, H_ = q.shape[0], q.shape[1]
        if state is not None:
            if len(state) != 3:
                raise ValueError("with the mLSTM gates state is (S0, z0, m0)")
            stab = state[2]
            _need(stab, "m0", device=q.device, dtype=torch.float32, shape=(B_, H_))
            state = state[:2]
        else:
            stab = torch.zeros(B_, H_, dtype=torch.float32, device=q.device)
    desc, (B, H, T, d_h, d_v) = _prefill_desc(q, k, v, phi, None, decay, gate, eps, 0, segments,
                                              dout.dtype, normalize, True, igate, fgate,
                                              fgate_exp, stab)
    _need(dout, "dout", device=q.device, shape=(B, H, T, d_v))
    dp = feature_dim(d_h, phi)
    S0 = z0 = None
    if state is not None:
        S0, z0 = state
        _need(S0, "S0", device=q.device, dtype=torch.float32, shape=(B, H, dp, d_v))
        _need(z0, "z0", device=q.device, dtype=torch.float32, shape=(B, H, dp))
    f32 = dict(dtype=torch.float32, device=q.device)
    g = {"dq": torch.empty(B, H, T, d_h, **f32), "dk": torch.empty(B, H, T, d_h, **f32),
         "dv": torch.empty(B, H, T, d_v, **f32)}
    dd = None
    if decay is not None or gate is not None:
        dd = torch.empty(B, H, T, **f32)
    elif mlstm:
        dd = torch.empty(2, B, H, T, **f32)   # dL/dfgate, then dL/digate
    dS0 = torch.empty(B, H, dp, d_v, **f32) if state_grad else None
    dz0 = torch.empty(B, H, dp, **f32) if state_grad else None
    n = ctypes.c_size_t(0)
    L = _lib.lib()
    _lib.check(L.la_prefill_backward_workspace_size(ctypes.byref(desc), ctypes.byref(n)))
    nws = int(n.value)
    if nws and (workspace is None or workspace.numel() * workspace.element_size() < nws):
        workspace = torch.empty(nws, dtype=torch.uint8, device=q.device)
    _lib.check(L.la_prefill_backward(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(S0),
                                     _ptr(z0), _ptr(dout), _ptr(g["dq"]), _ptr(g["dk"]),
                                     _ptr(g["dv"]), _ptr(dd), _ptr(dS0), _ptr(dz0),
                                     _ptr(workspace) if nws else None, nws, _stream(q.device)))
    if decay is not None:
        g["ddecay"] = dd
    if gate is not None:
        g["dgate"] = dd
    if mlstm:
        g["dfgate"], g["digate"] = dd[0], dd[1]
    if state_grad:
        g["dS0"], g["dz0"] = dS0, dz0
    return g


def decode_step(q, k, v, S, z, *, phi: str = "elu1", W=None, decay=None, gate=None,
                eps: float = 1e-6, out=None, out_dtype=None, normalize=True, igate=None,
                fgate=None, fgate_exp: bool = False, stab=None):
    """One token for B sequences x H heads: q, k [B, H, d_h], v [B, H, d_v].

    Updates (S, z) in place and returns out [B, H, d_v] (dtype of q);
    `normalize=False` returns the numerator alone, "max1" divides by
    max(|phi(q).z|, 1).  mLSTM gates: `igate`, `fgate` [B, H] and the
    stabiliser `stab` [B, H], updated in place with the state.
    """
    torch = _torch()
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, n, device=q.device, dtype=q.dtype)
    if q.dim() != 3:
        raise ValueError("decode inputs must be [B, H, d]")
    B, H, d_h = q.shape
    d_v = v.shape[-1]
    _need(k, "k", shape=(B, H, d_h))
    _need(v, "v", shape=(B, H, d_v))
    _check_W(W, phi, H, d_h, q.device)
    for a, n in ((decay, "decay"), (gate, "gate"), (igate, "igate"), (fgate, "fgate"),
                 (stab, "stab")):
        if a is not None:
            _need(a, n, device=q.device, dtype=torch.float32, shape=(B, H))
    out_dtype = out_dtype or q.dtype
    desc = make_desc(B, H, 1, d_h, d_v, _dtype_code(q.dtype), phi, W, None, decay, gate, eps,
                     out_dtype_code=_dtype_code(out_dtype), normalize=normalize, igate=igate,
                     fgate=fgate, fgate_exp=fgate_exp, stab=stab)
    dp = feature_dim(d_h, phi, desc.rff_D)
    _need(S, "S", device=q.device, dtype=torch.float32, shape=(B, H, dp, d_v))
    _need(z, "z", device=q.device, dtype=torch.float32, shape=(B, H, dp))
    if out is None:
        out = torch.empty(B, H, d_v, dtype=out_dtype, device=q.device)
    else:
        _need(out, "out", device=q.device, dtype=out_dtype, shape=(B, H, d_v))
    _lib.check(_lib.lib().la_decode_step(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(S),
                                         _ptr(z), _ptr(out), _stream(q.device)))
    return out
