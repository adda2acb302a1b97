"""la_prefill_noalloc, the prefill entry point that allocates nothing (for
callers under HIP graph capture or that may not call hipMalloc), against
la_prefill through the C ABI: the same kernels on the same inputs, so every
output, state and stabiliser must match bit for bit.  Two calls in a row on
one GPU share the static scratch array; the second, smaller one must not
see the first one's contents.  A prefill whose workspace exceeds the static
array is rejected before anything is enqueued.
"""
import ctypes

import pytest
import torch

import fixed_state_sequence_amd as la
from fixed_state_sequence_amd import _lib
from fixed_state_sequence_amd import inputs as I
from conftest import gpu_device


def _desc_for(x, dtype_code, out_dtype_code, **kw):
    B, H, T, d = x.q.shape
    return la.make_desc(B, H, T, d, x.v.shape[-1], dtype_code, decay=kw.get("decay"),
                        gate=kw.get("gate"), out_dtype_code=out_dtype_code,
                        igate=kw.get("igate"), fgate=kw.get("fgate"), stab=kw.get("stab"),
                        phi=kw.get("phi", "elu1"), normalize=kw.get("normalize", True))


def _both(x, dev, out_dtype, **gates):
    """(out, S, z, m) from la_prefill with a torch workspace and from
    la_prefill_noalloc, on the same inputs and initial state."""
    L = _lib.lib()
    g = {n: t.to(dev) for n, t in gates.items() if t is not None}
    q, k, v = x.q.to(dev), x.k.to(dev), x.v.to(dev)
    B, H, T, d = q.shape
    mlstm = "igate" in g
    results = []
    for entry in ("la_prefill", "la_prefill_noalloc"):
        S = torch.full((B, H, d, d), 0.25, device=dev)
        z = torch.full((B, H, d), 0.5, device=dev)
        m = torch.full((B, H), 0.125, device=dev) if mlstm else None
        out = torch.full((B, H, T, d), float("nan"), dtype=out_dtype, device=dev)
        desc = _desc_for(x, la._dtype_code(q.dtype), la._dtype_code(out_dtype),
                         phi="identity" if mlstm else "elu1",
                         normalize="max1" if mlstm else True, stab=m, **g)
        if entry == "la_prefill":
            nws = la.prefill_workspace_size(desc)
            ws = torch.empty(max(nws, 1), dtype=torch.uint8, device=dev)
            rc = L.la_prefill(ctypes.byref(desc), la._ptr(q), la._ptr(k), la._ptr(v), la._ptr(S),
                              la._ptr(z), la._ptr(out), la._ptr(ws), nws, la._stream(dev))
        else:
            assert la.prefill_workspace_size(desc) <= _lib.NOALLOC_SCRATCH_BYTES
            rc = L.la_prefill_noalloc(ctypes.byref(desc), la._ptr(q), la._ptr(k), la._ptr(v),
                                      la._ptr(S), la._ptr(z), la._ptr(out), la._stream(dev))
        _lib.check(rc)
        torch.cuda.synchronize()
        results.append((out, S, z, m))
    return results


def _assert_identical(a, b, what):
    for name, x, y in zip(("out", "S", "z", "m"), a, b):
        if x is None:
            continue
        assert torch.equal(x, y), f"{what}: {name} differs"
        assert torch.isfinite(x).all(), f"{what}: {name} not finite"


@pytest.mark.gpu
def test_noalloc_prefill_matches_la_prefill_twice_in_a_row():
    dev = gpu_device()
    # 1: the long-context workload (B=1, H=8, T=102400, d=128, bf16), the
    #    largest workspace of the measured prefills (33.8 MB of scratch)
    x1 = I.workload_inputs("long_prefill_b1_h8_t102400_d128", seed=5)
    print("noalloc call 1: long context", flush=True)
    a, b = _both(x1, dev, torch.float32)
    _assert_identical(a, b, "long context")
    # 2: a smaller prefill with the SSD decay (B=2, H=4, T=3000, d=64, a
    #    ragged tail) on the same scratch, which still holds call 1's slots
    x2 = I.prefill_inputs(2, 4, 3000, 64, dtype="bf16", seed=6, decay="ssd")
    print("noalloc call 2: SSD decay, smaller", flush=True)
    a, b = _both(x2, dev, torch.bfloat16, decay=x2.decay)
    _assert_identical(a, b, "SSD, second call")


@pytest.mark.gpu
def test_noalloc_prefill_mlstm_gates_and_empty_sequence():
    dev = gpu_device()
    x = I.prefill_inputs(1, 4, 20000, 128, dtype="bf16", seed=7, decay="mlstm",
                         scale=2.0 ** -0.5)
    print("noalloc: mLSTM gates", flush=True)
    a, b = _both(x, dev, torch.float32, igate=x.igate, fgate=x.fgate)
    _assert_identical(a, b, "mLSTM")
    # T = 0 is a no-op: the state stays as given
    L = _lib.lib()
    S = torch.ones(1, 2, 64, 64, device=dev)
    z = torch.ones(1, 2, 64, device=dev)
    desc = la.make_desc(1, 2, 0, 64, 64, _lib.LA_BF16)
    _lib.check(L.la_prefill_noalloc(ctypes.byref(desc), None, None, None, la._ptr(S), la._ptr(z),
                                    None, la._stream(dev)))
    torch.cuda.synchronize()
    assert bool((S == 1).all()) and bool((z == 1).all())
