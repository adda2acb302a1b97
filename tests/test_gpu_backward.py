"""Prefill gradients on the GPU (la_prefill_backward) against the fp64
oracle's gradients of the definition (pinned by finite differences), element
by element: dq, dk, dv, the decay or gate gradient and the initial-state
gradients.  Bars: 1e-4 (fp32 inputs), 2e-2 (bf16 inputs), max |gpu - oracle|
/ rms(oracle) per gradient.
"""
import ctypes

import numpy as np
import pytest
import torch

import fixed_state_sequence_amd as la
from fixed_state_sequence_amd import inputs as I
from oracle import linattn_oracle as O
from conftest import rel_err, TOL, gpu_device

pytestmark = pytest.mark.gpu


def run(x, do, dev, phi, normalize, state=None, state_grad=True, segments=0):
    g = lambda t: None if t is None else t.to(dev)
    st = None if state is None else tuple(g(torch.as_tensor(s, dtype=torch.float32)) for s in state)
    out = la.prefill_backward(g(x.q), g(x.k), g(x.v), g(do), phi=phi, decay=g(x.decay),
                              gate=g(x.gate), state=st, normalize=normalize,
                              state_grad=state_grad, segments=segments)
    torch.cuda.synchronize()
    return {k: v.cpu().double().numpy() for k, v in out.items()}


def compare(got, ref, tol, label):
    errs = {k: rel_err(got[k], ref[k]) for k in got}
    print(label, errs)
    assert max(errs.values()) < tol, (label, errs)


@pytest.mark.parametrize("phi", ["elu1", "identity"])
@pytest.mark.parametrize("decay", [None, "ssd", "rfa"])
@pytest.mark.parametrize("normalize", [True, False, "max1"])
def test_backward_fp32_vs_oracle(phi, decay, normalize):
    dev = gpu_device()
    B, H, T, d, dv = 2, 2, 67, 16, 8
    x = I.prefill_inputs(B, H, T, d, dv, dtype="f32", seed=5, decay=decay, scale=0.7)
    if phi == "identity" and (normalize is True or decay is None):
        # signed identity features cancel in q.S and q.z; with no floor on the
        # divisor, or with a state that never forgets, the gradients of such
        # inputs lose relative accuracy in any fp32 arithmetic: positive
        # features keep them well conditioned
        x.q, x.k = x.q.abs(), x.k.abs()
    do = torch.randn(B, H, T, dv, generator=torch.Generator().manual_seed(8))
    rng = np.random.default_rng(4)
    S0 = rng.standard_normal((B, H, d, dv)) * 0.3
    z0 = np.abs(rng.standard_normal((B, H, d))) * 0.3
    got = run(x, do, dev, phi, normalize, state=(S0, z0))
    ref = O.prefill_gradients(x.q, x.k, x.v, do, phi=phi, decay=x.decay, gate=x.gate,
                              S0=S0, z0=z0, normalize=normalize)
    compare(got, ref, TOL["f32"], (phi, decay, normalize))


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("decay", [None, "ssd"])
def test_backward_bf16_widths(d, decay):
    dev = gpu_device()
    B, H, T = 1, 2, 300
    x = I.prefill_inputs(B, H, T, d, dtype="bf16", seed=d, decay=decay, scale=2.0 ** -0.5)
    do = torch.randn(B, H, T, d, generator=torch.Generator().manual_seed(3)).to(torch.bfloat16)
    got = run(x, do, dev, "elu1", True, state_grad=False)
    ref = O.prefill_gradients(x.q, x.k, x.v, do, decay=x.decay)
    ref = {k: ref[k] for k in got}
    compare(got, ref, TOL["bf16"], (d, decay))


def test_backward_zero_state_equals_explicit_zero_state():
    dev = gpu_device()
    x = I.prefill_inputs(1, 3, 40, 8, 4, dtype="f32", seed=2, decay="rfa")
    do = torch.randn(1, 3, 40, 4, generator=torch.Generator().manual_seed(1))
    a = run(x, do, dev, "elu1", True)
    b = run(x, do, dev, "elu1", True, state=(np.zeros((1, 3, 8, 4)), np.zeros((1, 3, 8))))
    for k in a:
        np.testing.assert_array_equal(a[k], b[k])


# The chunked MFMA gradients (bf16, elu+1, no decay, d in {64, 128}): one,
# the default and three segments of 32-token chunks; tails that leave a
# chunk ragged; a sequence shorter than one chunk; every read-out form; dout
# in bf16 and fp32; a carried-in state and its gradient.
CHUNKED = [
    # d, T, segments, normalize, dout fp32, with state
    (64, 300, 0, True, False, False),
    (128, 300, 0, True, False, True),
    (128, 300, 1, True, True, True),
    (128, 333, 3, True, False, False),
    (64, 95, 3, False, False, True),
    (128, 211, 0, "max1", False, True),
    (64, 211, 1, "max1", True, False),
    (128, 20, 0, True, False, True),
    (64, 1, 0, True, True, True),
    (128, 64, 2, False, True, False),
]


@pytest.mark.parametrize("d,T,segments,normalize,dout32,with_state", CHUNKED)
def test_backward_chunked_vs_oracle(d, T, segments, normalize, dout32, with_state):
    dev = gpu_device()
    B, H = 1, 2
    x = I.prefill_inputs(B, H, T, d, dtype="bf16", seed=T + d, scale=2.0 ** -0.5)
    do = torch.randn(B, H, T, d, generator=torch.Generator().manual_seed(T))
    if not dout32:
        do = do.to(torch.bfloat16)
    state = None
    if with_state:
        rng = np.random.default_rng(d)
        state = (rng.standard_normal((B, H, d, d)) * 0.3, np.abs(rng.standard_normal((B, H, d))) * 3)
    print(f"chunked backward: d={d} T={T} segments={segments} norm={normalize} "
          f"dout32={dout32} state={with_state}", flush=True)
    got = run(x, do, dev, "elu1", normalize, state=state, state_grad=True, segments=segments)
    ref = O.prefill_gradients(x.q, x.k, x.v, do, S0=None if state is None else state[0],
                              z0=None if state is None else state[1], normalize=normalize)
    compare(got, ref, TOL["bf16"], (d, T, segments, normalize, dout32, with_state))


# The chunked path with a decay: the SSD decay (a = sigmoid(N(3, 1)), and a
# strongly decaying draw, sigmoid(N(-1, 1)), where e^{l} spans many orders
# within a chunk) and the RFA gate, with their gradients dL/da and dL/dg.
CHUNKED_DECAY = [
    # d, T, segments, normalize, dout fp32, with state, decay, decay mean
    (128, 300, 0, True, False, True, "ssd", 3.0),
    (64, 333, 3, True, True, False, "rfa", 3.0),
    (128, 95, 1, "max1", False, True, "rfa", 3.0),
    (64, 211, 0, False, False, True, "ssd", 3.0),
    (128, 20, 0, True, False, False, "ssd", 3.0),
    (128, 257, 0, True, False, True, "ssd", -1.0),
    (64, 64, 2, True, False, True, "rfa", 3.0),
]


@pytest.mark.parametrize("d,T,segments,normalize,dout32,with_state,decay,mean", CHUNKED_DECAY)
def test_backward_chunked_decay_vs_oracle(d, T, segments, normalize, dout32, with_state, decay,
                                          mean):
    dev = gpu_device()
    B, H = 1, 2
    x = I.prefill_inputs(B, H, T, d, dtype="bf16", seed=T + 7 * d, scale=2.0 ** -0.5,
                         decay=decay, decay_mean=mean)
    do = torch.randn(B, H, T, d, generator=torch.Generator().manual_seed(T + 1))
    if not dout32:
        do = do.to(torch.bfloat16)
    state = None
    if with_state:
        rng = np.random.default_rng(d + 1)
        state = (rng.standard_normal((B, H, d, d)) * 0.3, np.abs(rng.standard_normal((B, H, d))) * 3)
    print(f"chunked backward: d={d} T={T} segments={segments} norm={normalize} "
          f"dout32={dout32} state={with_state} decay={decay} mean={mean}", flush=True)
    got = run(x, do, dev, "elu1", normalize, state=state, state_grad=True, segments=segments)
    ref = O.prefill_gradients(x.q, x.k, x.v, do, decay=x.decay, gate=x.gate,
                              S0=None if state is None else state[0],
                              z0=None if state is None else state[1], normalize=normalize)
    compare(got, ref, TOL["bf16"], (d, T, segments, normalize, dout32, with_state, decay, mean))


# The two workloads bench.py times the gradients on, at full size, in its
# launch configuration (default plan, bf16 dout), against the oracle's
# recurrent gradients (pinned to the quadratic form and to finite
# differences): the elu+1 prefill shape, every sequence; the long-context
# shape, two heads end to end (the gradients of the first tokens are the
# largest there, about 1/sqrt(t), so the bar is met only with the early
# chunks exact), and every head's initial-state gradient.

def _workload_grads(name, seed=1):
    dev = gpu_device()
    x = I.workload_inputs(name, seed=0)
    do = torch.randn(x.q.shape, generator=torch.Generator().manual_seed(seed)).to(torch.bfloat16)
    got = run(x, do, dev, "elu1", True, state_grad=True)
    return x, do, got


def test_backward_elu_prefill_b4_h8_t2048_d64_full():
    x, do, got = _workload_grads("elu_prefill_b4_h8_t2048_d64")
    ref = O.prefill_gradients_recurrent(x.q, x.k, x.v, do)
    compare(got, ref, TOL["bf16"], "elu prefill backward 4x8x2048x64")


def test_backward_long_prefill_b1_h8_t102400_d128_two_heads():
    x, do, got = _workload_grads("long_prefill_b1_h8_t102400_d128")
    hs = [0, 5]
    ref = O.prefill_gradients_recurrent(x.q[0, hs], x.k[0, hs], x.v[0, hs], do[0, hs])
    compare({k: v[0, hs] for k, v in got.items()}, ref, TOL["bf16"],
            "long prefill backward 1x8x102400x128, heads 0 and 5")
    for k in got:
        assert np.isfinite(got[k]).all(), k


def test_backward_ssd_prefill_b2_h16_t8192_d128_eight_sequences():
    """The SSD-decay prefill workload's gradients at full size in the default
    plan (bf16 dout), eight (b, h) sequences end to end against the oracle's
    recurrent gradients, dL/da included."""
    dev = gpu_device()
    x = I.workload_inputs("ssd_prefill_b2_h16_t8192_d128", seed=0)
    do = torch.randn(x.q.shape, generator=torch.Generator().manual_seed(1)).to(torch.bfloat16)
    got = run(x, do, dev, "elu1", True, state_grad=True)
    pairs = [(0, 0), (0, 5), (0, 11), (0, 15), (1, 2), (1, 7), (1, 9), (1, 14)]
    bs, hs = [p[0] for p in pairs], [p[1] for p in pairs]
    ref = O.prefill_gradients_recurrent(x.q[bs, hs], x.k[bs, hs], x.v[bs, hs], do[bs, hs],
                                        decay=x.decay[bs, hs])
    compare({k: v[bs, hs] for k, v in got.items()}, ref, TOL["bf16"],
            "ssd prefill backward 2x16x8192x128, eight sequences")
    for k in got:
        assert np.isfinite(got[k]).all(), k


def test_backward_chunked_many_short_sequences():
    """128 sequences of 40 tokens (one segment each, a ragged second chunk)
    with the SSD decay on the chunked path."""
    dev = gpu_device()
    B, H, T, d = 8, 16, 40, 64
    x = I.prefill_inputs(B, H, T, d, dtype="bf16", seed=21, decay="ssd", scale=2.0 ** -0.5)
    do = torch.randn(B, H, T, d, generator=torch.Generator().manual_seed(22)).to(torch.bfloat16)
    got = run(x, do, dev, "elu1", True, state_grad=True)
    ref = O.prefill_gradients(x.q, x.k, x.v, do, decay=x.decay)
    compare(got, ref, TOL["bf16"], "many short sequences")


@pytest.mark.parametrize("dtype,phi", [("f16", "elu1"), ("bf16", "identity")])
def test_backward_per_token_path_16_bit(dtype, phi):
    """16-bit inputs the chunked path does not take (fp16, identity features)
    go through the per-token kernel, against the oracle on the same values."""
    dev = gpu_device()
    B, H, T, d = 1, 2, 70, 32
    x = I.prefill_inputs(B, H, T, d, dtype=dtype, seed=23, decay="rfa", scale=0.5)
    if phi == "identity":
        x.q, x.k = x.q.abs(), x.k.abs()   # positive features keep q.z away from 0
    dt = torch.float16 if dtype == "f16" else torch.bfloat16
    do = torch.randn(B, H, T, d, generator=torch.Generator().manual_seed(24)).to(dt)
    got = run(x, do, dev, phi, True, state_grad=True)
    ref = O.prefill_gradients(x.q, x.k, x.v, do, phi=phi, gate=x.gate)
    compare(got, ref, TOL["bf16"], (dtype, phi))


def test_backward_chunked_decay_zero_and_one():
    """Decay values of exactly 0 (a full reset: the state before the token is
    forgotten) keep every gradient finite and equal to the oracle's, dL/da
    included: L is smooth in a_r at 0 and its gradient there is <G_r,
    S_{r-1}> + <gz_r, z_{r-1}>.  Decay 1 gives the gradients of the form with
    no decay."""
    dev = gpu_device()
    B, H, T, d = 1, 2, 150, 64
    x = I.prefill_inputs(B, H, T, d, dtype="bf16", seed=31, decay="ssd", scale=2.0 ** -0.5)
    x.decay[:, :, [0, 37, 64, 99, 149]] = 0.0
    do = torch.randn(B, H, T, d, generator=torch.Generator().manual_seed(32)).to(torch.bfloat16)
    rng = np.random.default_rng(33)
    state = (rng.standard_normal((B, H, d, d)) * 0.3, np.abs(rng.standard_normal((B, H, d))) * 3)
    got = run(x, do, dev, "elu1", True, state=state, state_grad=True, segments=3)
    ref = O.prefill_gradients(x.q, x.k, x.v, do, decay=x.decay, S0=state[0], z0=state[1])
    assert set(got) == set(ref) and np.isfinite(got["ddecay"]).all()
    compare(got, ref, TOL["bf16"], "decay with zeros")
    keep = ("dq", "dk", "dv", "dS0", "dz0")
    # decay 1 against the chunked path with no decay
    x.decay[:] = 1.0
    a = run(x, do, dev, "elu1", True, state=state, state_grad=True, segments=3)
    x1 = I.prefill_inputs(B, H, T, d, dtype="bf16", seed=31, scale=2.0 ** -0.5)
    b = run(x1, do, dev, "elu1", True, state=state, state_grad=True, segments=3)
    compare({k: a[k] for k in keep}, b, 1e-4, "decay 1 against no decay")
    assert np.isfinite(a["ddecay"]).all()


@pytest.mark.parametrize("decay", [None, "ssd"])
def test_backward_empty_sequence(decay):
    """T = 0: L is an empty sum, so dL/dS0 and dL/dz0 are zero and there is
    nothing else to write.  Called through the C ABI with dS0 and dz0 filled
    with NaN beforehand, so an output left unwritten fails; the workspace size
    is 0."""
    dev = gpu_device()
    B, H, d = 2, 3, 64
    L = la._lib.lib()
    one = torch.ones(1, device=dev)   # a valid pointer for the (empty) decay arrays
    desc = la.make_desc(B, H, 0, d, d, la._lib.LA_BF16, decay=one if decay else None)
    S0 = torch.randn(B, H, d, d, device=dev)
    z0 = torch.rand(B, H, d, device=dev)
    dS0 = torch.full((B, H, d, d), float("nan"), device=dev)
    dz0 = torch.full((B, H, d), float("nan"), device=dev)
    dd = torch.full((1,), float("nan"), device=dev) if decay else None
    n = ctypes.c_size_t(1)
    la._lib.check(L.la_prefill_backward_workspace_size(ctypes.byref(desc), ctypes.byref(n)))
    assert n.value == 0
    p = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())
    la._lib.check(L.la_prefill_backward(ctypes.byref(desc), None, None, None, p(S0), p(z0), None,
                                        None, None, None, p(dd), p(dS0), p(dz0), None, 0,
                                        ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)))
    torch.cuda.synchronize()
    assert torch.count_nonzero(dS0).item() == 0 and torch.count_nonzero(dz0).item() == 0
    assert not torch.isnan(dS0).any() and not torch.isnan(dz0).any()


@pytest.mark.parametrize("kind", ["ssd", "rfa"])
@pytest.mark.parametrize("segments", [1, 3])
def test_backward_chunked_near_zero_decays(kind, segments):
    """Decay or gate values at and near 0 on the chunked path (d = 128, bf16):
    exact resets, values below and just above the threshold where the
    gradient is taken as <G_r, S_{r-1}> + <gz_r, z_{r-1}> instead of a suffix
    sum over a_r, resets next to each other and at segment edges; the decay
    gradient is compared element by element with the oracle's (which never
    divides by a)."""
    dev = gpu_device()
    B, H, T, d = 1, 2, 333, 128
    x = I.prefill_inputs(B, H, T, d, dtype="bf16", seed=41, decay=kind, scale=2.0 ** -0.5)
    a = x.decay if kind == "ssd" else x.gate
    special = {0: 0.0, 5: 1e-7, 6: 0.0, 7: 0.0, 40: 1e-3, 63: 0.0, 64: 0.003, 111: 0.0,
               150: 0.0039, 151: 0.004, 224: 0.0, 300: 2e-5, 332: 0.0}
    for t, val in special.items():
        a[:, :, t] = val
    do = torch.randn(B, H, T, d, generator=torch.Generator().manual_seed(42)).to(torch.bfloat16)
    rng = np.random.default_rng(43)
    state = (rng.standard_normal((B, H, d, d)) * 0.3, np.abs(rng.standard_normal((B, H, d))) * 3)
    got = run(x, do, dev, "elu1", True, state=state, state_grad=True, segments=segments)
    ref = O.prefill_gradients_recurrent(x.q, x.k, x.v, do, decay=x.decay, gate=x.gate,
                                        S0=state[0], z0=state[1])
    name = "ddecay" if kind == "ssd" else "dgate"
    assert np.isfinite(got[name]).all()
    compare(got, ref, TOL["bf16"], ("near-zero", kind, segments))
    # the special tokens themselves, against the rms of the decay gradient
    r = float(np.sqrt(np.mean(ref[name] ** 2)))
    ts = sorted(special)
    worst = float(np.abs(got[name][..., ts] - ref[name][..., ts]).max() / r)
    print("special tokens", worst)
    assert worst < TOL["bf16"]


@pytest.mark.parametrize("kind", ["ssd", "rfa"])
@pytest.mark.parametrize("phi", ["elu1", "identity"])
def test_backward_per_token_near_zero_decays(kind, phi):
    """The same on the per-token kernel (fp32 inputs): resets and near-zero
    decays, the exact gradient over the whole sequence from the initial
    state, at the fp32 bar."""
    dev = gpu_device()
    B, H, T, d, dv = 2, 2, 90, 16, 8
    x = I.prefill_inputs(B, H, T, d, dv, dtype="f32", seed=44, decay=kind, scale=0.7)
    if phi == "identity":
        x.q, x.k = x.q.abs(), x.k.abs()
    a = x.decay if kind == "ssd" else x.gate
    for t, val in {0: 0.0, 3: 1e-6, 4: 0.0, 30: 0.002, 31: 0.0, 89: 0.0}.items():
        a[:, :, t] = val
    do = torch.randn(B, H, T, dv, generator=torch.Generator().manual_seed(45))
    rng = np.random.default_rng(46)
    S0 = rng.standard_normal((B, H, d, dv)) * 0.3
    z0 = np.abs(rng.standard_normal((B, H, d))) * 0.3
    got = run(x, do, dev, phi, True, state=(S0, z0))
    ref = O.prefill_gradients(x.q, x.k, x.v, do, phi=phi, decay=x.decay, gate=x.gate,
                              S0=S0, z0=z0)
    compare(got, ref, TOL["f32"], ("per-token near-zero", kind, phi))


# ------------------------------------------------------------------ mLSTM gates
# The per-token backward with the forward's stabilised state, against the
# oracle's mLSTM gradients (pinned by finite differences of the stabilised
# forward oracle): dq, dk, dv, dL/dfgate, dL/digate and the scaled start
# state's dS0', dz0'.

def _mlstm_case(B, H, T, d, dv, dtype, seed, ishift=0.0, fexp=False, positive=False):
    x = I.prefill_inputs(B, H, T, d, dv, dtype=dtype, seed=seed, decay="mlstm", scale=0.7)
    x.igate = x.igate + ishift
    if fexp:
        x.fgate = -torch.nn.functional.softplus(-x.fgate)   # log sigmoid: the exp form's input
    if positive:
        x.q, x.k = x.q.abs(), x.k.abs()
    return x


def _mlstm_run(x, do, dev, normalize, fexp, state, segments=0):
    g = lambda t: None if t is None else t.to(dev)
    st = None if state is None else tuple(torch.as_tensor(s, dtype=torch.float32, device=dev)
                                          for s in state)
    out = la.prefill_backward(g(x.q), g(x.k), g(x.v), g(do), phi="identity", igate=g(x.igate),
                              fgate=g(x.fgate), fgate_exp=fexp, state=st, normalize=normalize,
                              state_grad=True, segments=segments)
    torch.cuda.synchronize()
    return {k: v.cpu().double().numpy() for k, v in out.items()}


@pytest.mark.parametrize("normalize", ["max1", True, False])
@pytest.mark.parametrize("fexp", [False, True])
@pytest.mark.parametrize("with_state", [False, True])
def test_backward_mlstm_fp32_vs_oracle(normalize, fexp, with_state):
    dev = gpu_device()
    B, H, T, d, dv = 2, 2, 67, 16, 8
    x = _mlstm_case(B, H, T, d, dv, "f32", seed=7 + int(fexp), fexp=fexp,
                    positive=normalize is True)
    do = torch.randn(B, H, T, dv, generator=torch.Generator().manual_seed(9))
    state = None
    if with_state:
        rng = np.random.default_rng(5)
        state = (rng.standard_normal((B, H, d, dv)) * 0.3,
                 np.abs(rng.standard_normal((B, H, d))) * 0.3, rng.standard_normal((B, H)))
    got = _mlstm_run(x, do, dev, normalize, fexp, state)
    S0, z0, m0 = (None, None, None) if state is None else state
    ref = O.mlstm_gradients(x.q, x.k, x.v, do, x.igate, x.fgate, fexp, 1e-6, S0, z0, m0, normalize)
    compare(got, {k: ref[k] for k in got}, TOL["f32"], ("mlstm", normalize, fexp, with_state))


def test_backward_mlstm_input_gates_beyond_fp32():
    """Input pre-activations near 100 (e^100 overflows fp32) and a start state
    at the same scale (m0 near 100): the stabilised state carries the
    gradients without overflow.  Every weight then carries e^100, so |q.z| >>
    1 and the max1 read-out is q.S / |q.z|, which needs positive features to
    stay well conditioned (as in the forward's test of this case)."""
    dev = gpu_device()
    B, H, T, d, dv = 1, 2, 50, 16, 16
    x = _mlstm_case(B, H, T, d, dv, "f32", seed=13, ishift=100.0, positive=True)
    do = torch.randn(B, H, T, dv, generator=torch.Generator().manual_seed(2))
    rng = np.random.default_rng(3)
    state = (np.abs(rng.standard_normal((B, H, d, dv))) * 0.3,
             np.abs(rng.standard_normal((B, H, d))) * 0.3, 100.0 + rng.standard_normal((B, H)))
    got = _mlstm_run(x, do, dev, "max1", False, state)
    for key, val in got.items():
        assert np.isfinite(val).all(), key
    ref = O.mlstm_gradients(x.q, x.k, x.v, do, x.igate, x.fgate, False, 1e-6, *state,
                            normalize="max1")
    compare(got, {k: ref[k] for k in got}, TOL["f32"], "mlstm, input gates + 100")


@pytest.mark.parametrize("d", [64, 128])
def test_backward_mlstm_bf16_vs_oracle(d):
    dev = gpu_device()
    B, H, T = 1, 2, 200
    x = _mlstm_case(B, H, T, d, d, "bf16", seed=d)
    do = torch.randn(B, H, T, d, generator=torch.Generator().manual_seed(4)).to(torch.bfloat16)
    got = _mlstm_run(x, do, dev, "max1", False, None)
    ref = O.mlstm_gradients(x.q, x.k, x.v, do, x.igate, x.fgate, False, 1e-6, normalize="max1")
    compare(got, {k: ref[k] for k in got}, TOL["bf16"], ("mlstm bf16", d))


# The chunked path with the mLSTM gates (bf16, identity features, d 64/128):
# (d, T, segments, read-out, exponential forget gate, carried-in state,
# input-gate shift).  The sum read-out takes positive features and z0, so
# that q.z stays away from 0; so do input gates shifted up: the max1 floor
# e^{-m} then sits far below |q.z|, every output is q.S / |q.z|, and signed
# features put q.z near 0 for some tokens, whose gradients (about 100 times
# the rms at +4) no fp32 arithmetic resolves (the per-token kernel misses
# the oracle there by as much as the chunked passes).
MLSTM_CHUNKED = [
    (64, 333, 0, "max1", False, False, 0.0, False),
    (64, 333, 3, "max1", True, True, 0.0, False),
    (128, 257, 1, "max1", False, True, 0.0, False),
    (128, 640, 0, "max1", False, False, 4.0, False),
    (64, 200, 2, True, False, True, 0.0, False),
    (128, 161, 0, False, True, False, 0.0, False),
    (64, 95, 5, "max1", False, True, 25.0, False),
    (128, 31, 0, "max1", True, True, 0.0, False),
    (128, 300, 3, "max1", False, True, 0.0, True),
    (64, 129, 0, True, True, False, 0.0, True),
]


@pytest.mark.parametrize("d,T,segments,normalize,fexp,with_state,ishift,dout32", MLSTM_CHUNKED)
def test_backward_mlstm_chunked_vs_oracle(d, T, segments, normalize, fexp, with_state, ishift,
                                          dout32):
    """bf16 inputs with the mLSTM gates take the chunked passes: the
    stabiliser rebuilt per chunk from each segment's start (the prefill's
    scan), alpha' and beta' as decay and key weight, the gates' gradients
    from the suffix sums.  Every gradient against the oracle's."""
    dev = gpu_device()
    B, H = 2, 2
    positive = normalize is True or ishift > 0
    x = _mlstm_case(B, H, T, d, d, "bf16", seed=T + d, ishift=ishift, fexp=fexp,
                    positive=positive)
    do = torch.randn(B, H, T, d, generator=torch.Generator().manual_seed(T))
    if not dout32:
        do = do.to(torch.bfloat16)
    state = None
    if with_state:
        rng = np.random.default_rng(d + T)
        z0 = rng.standard_normal((B, H, d)) * 0.3
        S0 = rng.standard_normal((B, H, d, d)) * 0.3
        state = (np.abs(S0) if positive else S0, np.abs(z0) if positive else z0,
                 ishift + rng.standard_normal((B, H)))
    got = _mlstm_run(x, do, dev, normalize, fexp, state, segments)
    S0, z0, m0 = (None, None, None) if state is None else state
    ref = O.mlstm_gradients(x.q, x.k, x.v, do, x.igate, x.fgate, fexp, 1e-6, S0, z0, m0, normalize)
    compare(got, {k: ref[k] for k in got}, TOL["bf16"],
            ("mlstm chunked", d, T, segments, normalize, fexp, with_state, ishift, dout32))


def test_backward_mlstm_chunked_equals_per_token_on_the_same_values():
    """The chunked passes (bf16 inputs) and the per-token kernel (the same
    values as fp32 inputs) compute the same gradients: 8 segments of a
    4096-token sequence at d = 128, with a carried-in state."""
    dev = gpu_device()
    B, H, T, d = 1, 2, 4096, 128
    x = _mlstm_case(B, H, T, d, d, "bf16", seed=41)
    do = torch.randn(B, H, T, d, generator=torch.Generator().manual_seed(42)).to(torch.bfloat16)
    rng = np.random.default_rng(43)
    state = (rng.standard_normal((B, H, d, d)) * 0.3, rng.standard_normal((B, H, d)) * 0.3,
             rng.standard_normal((B, H)))
    got = _mlstm_run(x, do, dev, "max1", False, state, segments=8)
    x32 = _mlstm_case(B, H, T, d, d, "bf16", seed=41)
    for n in ("q", "k", "v"):
        setattr(x32, n, getattr(x32, n).float())
    ref = _mlstm_run(x32, do.float(), dev, "max1", False, state)
    compare(got, ref, TOL["bf16"], "mlstm chunked vs per-token")
