"""The C ABI without a GPU: the library loads, exports every declared entry
point, and rejects bad arguments on the host before any HIP call."""
import ctypes

import pytest

from fixed_state_sequence_amd import _lib
import fixed_state_sequence_amd as la

L = _lib.lib()
FAKE = 0x10000  # aligned, never dereferenced: every call below fails validation


def desc(**kw):
    base = dict(B=1, H=8, T=102400, d_h=128, d_v=128, dtype_code=_lib.LA_BF16)
    base.update(kw)
    return la.make_desc(**base)


def status(rc):
    return L.la_status_str(rc).decode()


def test_every_declared_function_is_exported():
    names = _lib.header_functions()
    assert set(names) >= {"la_prefill", "la_decode_step", "la_state_init",
                          "la_prefill_workspace_size", "la_prefill_plan", "la_prefill_stage",
                          "la_feature_dim", "la_status_str", "la_last_error"}
    for n in names:
        assert hasattr(L, n), n


def test_status_strings():
    assert [status(i) for i in range(4)] == ["LA_OK", "LA_EINVAL", "LA_EUNSUPPORTED", "LA_EHIP"]


def test_feature_dim():
    assert L.la_feature_dim(ctypes.byref(desc())) == 128
    d = la.make_desc(256, 16, 1, 64, 64, _lib.LA_F32, phi="rff", rff_D=64)
    d.rff_W = FAKE
    assert L.la_feature_dim(ctypes.byref(d)) == 128
    assert L.la_feature_dim(ctypes.byref(desc(B=0))) == -1
    assert L.la_feature_dim(None) == -1


def test_plan_for_the_measured_prefills():
    # long context: chunked MFMA path, segments spread 8 heads over the chip
    c, s, p = la.prefill_plan(desc())
    assert (c, s, p) == (32, 32, 1)    # one workgroup per compute unit: 8 heads x 32 segments
    # stage 1 cuts every segment in two: 2 * 32 state slots per head; then
    # log Gamma and the mLSTM stabiliser per slot, and the mLSTM start
    # stabiliser per segment plus the final one, each rounded to 256 bytes
    slots = 2 * s
    r256 = lambda n: (n + 255) // 256 * 256
    assert la.prefill_workspace_size(desc()) == (8 * slots * (128 * 128 + 128) * 4
                                                 + 2 * r256(8 * slots * 4) + r256(8 * (s + 1) * 4))
    # fp32 inputs take the per-token kernel; no workspace
    d = desc(T=8, d_h=4, d_v=4, dtype_code=_lib.LA_F32)
    assert la.prefill_plan(d)[2] == 0 and la.prefill_workspace_size(d) == 0
    # explicit segments are honoured up to the chunk count, never leaving one empty
    d = desc(T=640, segments=4, chunk=64)
    assert la.prefill_plan(d) == (64, 4, 1)
    d = desc(T=9 * 64, segments=4, chunk=64)   # 9 chunks, 3 per segment -> 3 segments
    assert la.prefill_plan(d)[1] == 3
    d = desc(T=100, segments=50, chunk=64)
    assert la.prefill_plan(d)[1] == 2
    d = desc(T=100, segments=50)                # 4 chunks of 32 -> 4 segments
    assert la.prefill_plan(d) == (32, 4, 1)


@pytest.mark.parametrize("field,value", [("B", 0), ("H", -1), ("T", -5), ("d_h", 0), ("d_v", 0),
                                         ("dtype", 7), ("phi", 9), ("decay_kind", 5),
                                         ("chunk", 48), ("segments", -1), ("norm", 3),
                                         ("noncausal", 3), ("fgate_exp", 1)])
def test_bad_descriptor_fields_are_rejected(field, value):
    d = desc()
    setattr(d, field, value)
    rc = L.la_prefill(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 40, None)
    assert status(rc) == "LA_EINVAL"
    assert L.la_last_error().decode() != ""


def test_null_and_misaligned_pointers():
    d = desc()
    args = [FAKE] * 7
    for i in range(6):
        a = list(args)
        a[i] = None
        rc = L.la_prefill(ctypes.byref(d), *a, 1 << 40, None)
        assert status(rc) == "LA_EINVAL"
    a = list(args)
    a[0] = FAKE + 2
    assert status(L.la_prefill(ctypes.byref(d), *a, 1 << 40, None)) == "LA_EINVAL"
    assert "aligned" in L.la_last_error().decode()


def test_workspace_too_small():
    d = desc()
    need = la.prefill_workspace_size(d)
    rc = L.la_prefill(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, need - 1, None)
    assert status(rc) == "LA_EINVAL" and "workspace" in L.la_last_error().decode()
    rc = L.la_prefill(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, need, None)
    assert status(rc) == "LA_EINVAL"


def test_decay_pointer_consistency():
    d = desc()
    d.decay = FAKE   # decay array with LA_DECAY_NONE
    assert status(L.la_prefill(ctypes.byref(d), *([FAKE] * 7), 1 << 40, None)) == "LA_EINVAL"
    d = desc()
    d.decay_kind = _lib.LA_DECAY_SSD   # SSD with no array
    assert status(L.la_prefill(ctypes.byref(d), *([FAKE] * 7), 1 << 40, None)) == "LA_EINVAL"


def test_rff_descriptor_checks():
    d = desc(T=16, d_h=64, d_v=64, dtype_code=_lib.LA_F32)
    d.phi = _lib.LA_PHI_RFF
    d.rff_D = 64   # W missing
    assert status(L.la_prefill(ctypes.byref(d), *([FAKE] * 7), 0, None)) == "LA_EINVAL"
    d = desc(T=16)
    d.rff_D = 3    # elu+1 with rff_D set
    assert status(L.la_prefill(ctypes.byref(d), *([FAKE] * 7), 0, None)) == "LA_EINVAL"


def test_unsupported_widths():
    d = desc(d_h=512, d_v=512, dtype_code=_lib.LA_F32)
    assert status(L.la_prefill(ctypes.byref(d), *([FAKE] * 7), 0, None)) == "LA_EUNSUPPORTED"
    d = desc(d_h=64, d_v=12, dtype_code=_lib.LA_F32)     # d_v / 4 not a power of two
    assert status(L.la_decode_step(ctypes.byref(d), *([FAKE] * 6), None)) == "LA_EUNSUPPORTED"


def test_stage_index_checked():
    d = desc()
    assert status(L.la_prefill_stage(ctypes.byref(d), 4, *([FAKE] * 7), 1 << 40, None)) == "LA_EINVAL"


def test_decode_null_state():
    d = la.make_desc(256, 16, 1, 64, 64, _lib.LA_F32)
    assert status(L.la_decode_step(ctypes.byref(d), FAKE, FAKE, FAKE, None, FAKE, FAKE, None)) == "LA_EINVAL"
    assert status(L.la_state_init(ctypes.byref(d), FAKE, None, None)) == "LA_EINVAL"


def test_shares_torchs_hip_runtime():
    # one HIP runtime per process: the library resolves to torch's copy
    assert len(_lib._hip_runtimes()) == 1


def test_chunk_128_needs_narrow_state():
    d = desc(chunk=128)
    assert status(L.la_prefill(ctypes.byref(d), *([FAKE] * 7), 1 << 40, None)) == "LA_EUNSUPPORTED"
    assert la.prefill_plan(desc(chunk=128, d_h=64, d_v=64))[0] == 128


def test_noncausal_checks():
    d = desc(causal=False)
    d.decay_kind, d.decay = _lib.LA_DECAY_SSD, FAKE   # the non-causal form takes no decay
    assert status(L.la_prefill(ctypes.byref(d), *([FAKE] * 7), 1 << 40, None)) == "LA_EINVAL"
    d = la.make_desc(256, 16, 1, 64, 64, _lib.LA_F32, causal=False)   # decode is causal
    assert status(L.la_decode_step(ctypes.byref(d), *([FAKE] * 6), None)) == "LA_EINVAL"
    # a single segment still needs the workspace: the state comes first
    one = desc(T=640, segments=1, causal=False)
    assert la.prefill_plan(one)[1] == 1 and la.prefill_workspace_size(one) > 0
    assert la.prefill_workspace_size(desc(T=640, segments=1)) == 0



def test_mlstm_descriptor_checks():
    base = dict(T=640, d_h=128, d_v=128, dtype_code=_lib.LA_BF16)
    ok = desc(phi="identity", **base)
    ok.decay_kind, ok.decay, ok.igate, ok.stab = _lib.LA_GATE_MLSTM, FAKE, FAKE, FAKE
    assert la.prefill_plan(ok)[2] == 1                      # the chunked MFMA path
    for field in ("igate", "stab", "decay"):                # each array is required
        d = desc(phi="identity", **base)
        d.decay_kind, d.decay, d.igate, d.stab = _lib.LA_GATE_MLSTM, FAKE, FAKE, FAKE
        setattr(d, field, None)
        assert status(L.la_prefill(ctypes.byref(d), *([FAKE] * 7), 1 << 40, None)) == "LA_EINVAL"
    d = desc(phi="identity", **base)
    d.decay_kind, d.decay, d.igate, d.stab, d.fgate_exp = _lib.LA_GATE_MLSTM, FAKE, FAKE, FAKE, 2
    assert status(L.la_prefill(ctypes.byref(d), *([FAKE] * 7), 1 << 40, None)) == "LA_EINVAL"
    d = desc(**base)                                        # igate without the mLSTM gates
    d.igate = FAKE
    assert status(L.la_prefill(ctypes.byref(d), *([FAKE] * 7), 1 << 40, None)) == "LA_EINVAL"
    d = desc(phi="identity", causal=False, **base)          # no gates in the non-causal form
    d.decay_kind, d.decay, d.igate, d.stab = _lib.LA_GATE_MLSTM, FAKE, FAKE, FAKE
    assert status(L.la_prefill(ctypes.byref(d), *([FAKE] * 7), 1 << 40, None)) == "LA_EINVAL"
    # elu+1 with the mLSTM gates, and identity features without them, take the
    # per-token kernel
    d = desc(**base)
    d.decay_kind, d.decay, d.igate, d.stab = _lib.LA_GATE_MLSTM, FAKE, FAKE, FAKE
    assert la.prefill_plan(d)[2] == 0
    assert la.prefill_plan(desc(phi="identity", **base))[2] == 0
    assert L.la_feature_dim(ctypes.byref(desc(phi="identity", **base))) == 128


def test_backward_checks():
    bw = lambda d, ddecay=None, S0=None, z0=None, dS0=None, dz0=None, nws=1 << 40: status(
        L.la_prefill_backward(ctypes.byref(d), FAKE, FAKE, FAKE, S0, z0, FAKE, FAKE, FAKE, FAKE,
                              ddecay, dS0, dz0, FAKE, nws, None))
    base = dict(T=300, d_h=64, d_v=64, dtype_code=_lib.LA_BF16)
    n = ctypes.c_size_t(0)
    assert status(L.la_prefill_backward_workspace_size(ctypes.byref(desc(**base)), ctypes.byref(n))) == "LA_OK"
    # bf16, elu+1, no decay, d = 64: the chunked path.  Its workspace is the
    # prefill's (32-token chunks, the default plan: 5 segments of 2 chunks,
    # 10 stage-1 slots per head), a copy of the initial state, one gradient
    # state per segment and two floats per token, each rounded up to 256 bytes
    r = lambda b: (b + 255) // 256 * 256
    BH, E = 8, 64 * 64 + 64
    fwd = BH * 10 * E * 4 + 2 * r(BH * 10 * 4) + r(BH * 6 * 4)
    assert n.value == r(fwd) + r(BH * 64 * 64 * 4) + r(BH * 64 * 4) + r(BH * 5 * E * 4) + r(BH * 300 * 8)
    # fp32 inputs: the per-token kernel, B H T (d_v + 2) floats
    d32 = desc(T=300, d_h=64, d_v=64, dtype_code=_lib.LA_F32)
    assert status(L.la_prefill_backward_workspace_size(ctypes.byref(d32), ctypes.byref(n))) == "LA_OK"
    assert n.value == 8 * 300 * (64 + 2) * 4
    assert status(L.la_prefill_backward_workspace_size(ctypes.byref(desc(**base)), ctypes.byref(n))) == "LA_OK"
    # not covered: RFF, the non-causal form
    d = desc(T=16, d_h=64, d_v=64, dtype_code=_lib.LA_F32)
    d.phi, d.rff_D, d.rff_W = _lib.LA_PHI_RFF, 32, FAKE
    assert bw(d) == "LA_EUNSUPPORTED"
    assert bw(desc(causal=False, **base)) == "LA_EUNSUPPORTED"
    # the mLSTM gates, bf16: the chunked path, as above plus a zero start
    # stabiliser per head, each segment's log-decay, four floats per token
    # (the decay gradient's terms, log alpha' and beta') and the tile totals;
    # ddecay (both gates' gradients) required
    d = desc(phi="identity", **base)
    d.decay_kind, d.decay, d.igate, d.stab = _lib.LA_GATE_MLSTM, FAKE, FAKE, FAKE
    assert status(L.la_prefill_backward_workspace_size(ctypes.byref(d), ctypes.byref(n))) == "LA_OK"
    assert n.value == (r(fwd) + r(BH * 64 * 64 * 4) + r(BH * 64 * 4) + r(BH * 4) + r(BH * 5 * E * 4)
                       + r(BH * 300 * 8) + r(BH * 5 * 4) + 2 * r(BH * 300 * 4) + r(BH * 1 * 4)
                       + r(BH * 300 * 8))
    assert bw(d) == "LA_EINVAL"
    # fp32 inputs: the per-token path, B H T (d_v + 4) floats (alpha', beta'
    # per token beside the read-out's terms)
    d = desc(phi="identity", T=300, d_h=64, d_v=64, dtype_code=_lib.LA_F32)
    d.decay_kind, d.decay, d.igate, d.stab = _lib.LA_GATE_MLSTM, FAKE, FAKE, FAKE
    assert status(L.la_prefill_backward_workspace_size(ctypes.byref(d), ctypes.byref(n))) == "LA_OK"
    assert n.value == 8 * 300 * (64 + 4) * 4
    assert bw(d) == "LA_EINVAL"
    assert status(L.la_prefill_backward_workspace_size(ctypes.byref(desc(**base)), ctypes.byref(n))) == "LA_OK"
    # ddecay exactly with a decay; S0/z0 and dS0/dz0 in pairs; workspace size
    d = desc(**base)
    d.decay_kind, d.decay = _lib.LA_DECAY_SSD, FAKE
    assert bw(d) == "LA_EINVAL"
    assert bw(desc(**base), ddecay=FAKE) == "LA_EINVAL"
    assert bw(desc(**base), S0=FAKE) == "LA_EINVAL"
    assert bw(desc(**base), dS0=FAKE) == "LA_EINVAL"
    assert bw(desc(**base), nws=n.value - 1) == "LA_EINVAL"
    assert "workspace" in L.la_last_error().decode()


def test_backward_empty_sequence_needs_no_workspace():
    """T = 0 (an empty sum): no workspace, on either path."""
    n = ctypes.c_size_t(1)
    for dtype in (_lib.LA_BF16, _lib.LA_F32):
        d = desc(T=0, d_h=64, d_v=64, dtype_code=dtype)
        assert status(L.la_prefill_backward_workspace_size(ctypes.byref(d), ctypes.byref(n))) == "LA_OK"
        assert n.value == 0


def test_mis_shaped_rff_projection_is_rejected_before_any_launch():
    # The decode and per-token kernels index W by head and input feature:
    # [H, rff_D, d_h].  Any other shape must be refused in the binding (the C
    # ABI sees only a pointer), before a tensor is read.
    import torch
    H, d_h = 16, 64
    for bad in (torch.zeros(H - 1, 64, d_h), torch.zeros(H, 64, d_h - 1), torch.zeros(64, d_h),
                torch.zeros(H, 0, d_h), torch.zeros(1, H, 64, d_h)):
        with pytest.raises(ValueError, match="W has shape"):
            la._check_W(bad, "rff", H, d_h, None)
    with pytest.raises(ValueError, match="needs W"):
        la._check_W(None, "rff", H, d_h, None)
    with pytest.raises(ValueError, match="only used by the random-feature map"):
        la._check_W(torch.zeros(H, 64, d_h), "elu1", H, d_h, None)
    la._check_W(None, "elu1", H, d_h, None)
    # a well-shaped W passes the shape test and is then held to the device
    with pytest.raises(ValueError, match="CUDA"):
        la._check_W(torch.zeros(H, 64, d_h), "rff", H, d_h, None)


def test_noalloc_prefill_rejects_a_workspace_beyond_the_static_scratch():
    # 16 x 16 sequences of d = 128 cut into 4 segments hold 8 state slots
    # each (135 MB) against the 64 MiB static array: refused on the host,
    # before any HIP call (this runs without a GPU)
    d = desc(B=16, H=16, T=8192, segments=4)
    assert la.prefill_workspace_size(d) > _lib.NOALLOC_SCRATCH_BYTES
    rc = L.la_prefill_noalloc(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None)
    assert status(rc) == "LA_EINVAL"
    msg = L.la_last_error().decode()
    assert "static scratch" in msg and str(_lib.NOALLOC_SCRATCH_BYTES) in msg
    # bad pointers are refused before the size is even looked at
    rc = L.la_prefill_noalloc(ctypes.byref(desc()), FAKE, FAKE, FAKE, None, FAKE, FAKE, None)
    assert status(rc) == "LA_EINVAL" and "S is NULL" in L.la_last_error().decode()
