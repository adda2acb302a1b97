"""ctypes binding of liblinattn.so: the C ABI declared in include/linattn.h.

Loading is lazy (first use) and fails loudly if the library was not built;
there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os
import re

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liblinattn.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "linattn.h")

LA_OK, LA_EINVAL, LA_EUNSUPPORTED, LA_EHIP = 0, 1, 2, 3
LA_F32, LA_BF16, LA_F16 = 0, 1, 2
LA_PHI_ELU1, LA_PHI_RFF, LA_PHI_IDENTITY = 0, 1, 2
LA_DECAY_NONE, LA_DECAY_SSD, LA_GATE_RFA, LA_GATE_MLSTM = 0, 1, 2, 3
LA_NORM_SUM, LA_NORM_NONE, LA_NORM_MAX1 = 0, 1, 2
NOALLOC_SCRATCH_BYTES = 64 << 20      # LA_NOALLOC_SCRATCH_BYTES


class LaDesc(ctypes.Structure):
    """Mirror of `la_desc` (field order and types as in include/linattn.h)."""
    _fields_ = [
        ("B", ctypes.c_int), ("H", ctypes.c_int), ("T", ctypes.c_int),
        ("d_h", ctypes.c_int), ("d_v", ctypes.c_int),
        ("dtype", ctypes.c_int), ("out_dtype", ctypes.c_int), ("phi", ctypes.c_int),
        ("rff_D", ctypes.c_int), ("rff_W", ctypes.c_void_p),
        ("decay_kind", ctypes.c_int), ("decay", ctypes.c_void_p),
        ("eps", ctypes.c_float), ("chunk", ctypes.c_int), ("segments", ctypes.c_int),
        ("norm", ctypes.c_int), ("noncausal", ctypes.c_int),
        ("igate", ctypes.c_void_p), ("fgate_exp", ctypes.c_int), ("stab", ctypes.c_void_p),
    ]


class LinAttnError(RuntimeError):
    def __init__(self, status, message):
        self.status = status
        super().__init__(f"{message} [{status}]")


_LIB = None

_P = ctypes.c_void_p
_D = ctypes.POINTER(LaDesc)
_SIGNATURES = {
    "la_feature_dim": (ctypes.c_int, [_D]),
    "la_state_init": (ctypes.c_int, [_D, _P, _P, _P]),
    "la_prefill_workspace_size": (ctypes.c_int, [_D, ctypes.POINTER(ctypes.c_size_t)]),
    "la_prefill_plan": (ctypes.c_int, [_D, ctypes.POINTER(ctypes.c_int),
                                       ctypes.POINTER(ctypes.c_int), ctypes.POINTER(ctypes.c_int)]),
    "la_prefill": (ctypes.c_int, [_D, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]),
    "la_prefill_noalloc": (ctypes.c_int, [_D, _P, _P, _P, _P, _P, _P, _P]),
    "la_prefill_stage": (ctypes.c_int, [_D, ctypes.c_int, _P, _P, _P, _P, _P, _P, _P,
                                        ctypes.c_size_t, _P]),
    "la_decode_step": (ctypes.c_int, [_D, _P, _P, _P, _P, _P, _P, _P]),
    "la_prefill_backward_workspace_size": (ctypes.c_int, [_D, ctypes.POINTER(ctypes.c_size_t)]),
    "la_prefill_backward": (ctypes.c_int, [_D, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                           _P, ctypes.c_size_t, _P]),
    "la_status_str": (ctypes.c_char_p, [ctypes.c_int]),
    "la_last_error": (ctypes.c_char_p, []),
}


def _hip_runtimes():
    """Distinct HIP runtime files mapped into this process."""
    try:
        maps = open("/proc/self/maps").read().splitlines()
    except OSError:
        return set()
    return {os.path.realpath(l.split()[-1]) for l in maps if "libamdhip64" in l.split()[-1]}


def lib():
    """The loaded library (raises if liblinattn.so is missing).

    PyTorch supplies device memory and streams, so the library must share
    torch's HIP runtime.  torch ships its own libamdhip64 with the same soname
    as ROCm's; importing torch first makes the dynamic loader resolve our
    dependency to that already-loaded copy instead of mapping a second runtime.
    """
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is not built; run __graft_entry__.build() (hipcc, gfx950)")
        import torch  # noqa: F401  (loads torch's HIP runtime before ours)
        handle = ctypes.CDLL(LIB_PATH)
        runtimes = _hip_runtimes()
        if len(runtimes) > 1:
            raise RuntimeError(f"two HIP runtimes are loaded in this process: {sorted(runtimes)}")
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _LIB = handle
    return _LIB


def check(status: int):
    if status != LA_OK:
        L = lib()
        raise LinAttnError(L.la_status_str(status).decode(), L.la_last_error().decode())


def header_functions():
    """Names of the functions include/linattn.h declares."""
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\*?(la_\w+)\s*\(", text, re.M)))
