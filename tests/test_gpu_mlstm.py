"""mLSTM gates on the GPU against the fp64 oracle (wikillm "Linear attention",
Variants / "Matrix memory with exponential gates (mLSTM)"): identity
features, forget gate sigmoid(f~) or exp(f~), input gate exp(i~), the read-out
divided by max(|q.z|, 1) (and the other two read-outs), and the stabiliser m
carried with the state.

The library and the oracle keep the same scaled state (S', z', m) with
S = e^m S' (the oracle's stabilised recurrence); outputs are compared
element by element, the states as S', z' and m.  Bars: 1e-4 (fp32 inputs),
2e-2 (bf16/fp16 inputs), max |gpu - oracle| / rms(oracle).
"""
import numpy as np
import pytest
import torch

import fixed_state_sequence_amd as la
from fixed_state_sequence_amd import inputs as I
from oracle import linattn_oracle as O
from conftest import rel_err, TOL, gpu_device

pytestmark = pytest.mark.gpu


def run(x, dev, state=None, **kw):
    g = lambda t: None if t is None else t.to(dev)
    kw.setdefault("out_dtype", torch.float32)
    st = None if state is None else tuple(g(torch.as_tensor(s, dtype=torch.float32)) for s in state)
    out, S, z, m = la.prefill(g(x.q), g(x.k), g(x.v), phi="identity", igate=g(x.igate),
                              fgate=g(x.fgate), state=st, **kw)
    torch.cuda.synchronize()
    return out, S, z, m


def oracle(x, state=None, fgate_exp=False, normalize="max1", eps=1e-6):
    S0, z0, m0 = (None, None, None) if state is None else state
    return O.mlstm_recurrence(x.q, x.k, x.v, x.igate, x.fgate, fgate_exp, eps, S0, z0, m0,
                              normalize)


def errors(got, ref):
    out, S, z, m = got
    o_ref, S_ref, z_ref, m_ref = ref
    return (rel_err(out, o_ref), rel_err(S, S_ref), rel_err(z, z_ref),
            float(np.abs(m.cpu().double().numpy() - m_ref).max()))


def random_state(B, H, d, dv, seed, positive=False):
    g = np.random.default_rng(seed)
    z0 = g.standard_normal((B, H, d)) * 0.3
    return (g.standard_normal((B, H, d, dv)) * 0.3, np.abs(z0) if positive else z0,
            g.standard_normal((B, H)))


def condition(x, normalize):
    """With identity features q.z is signed, so the read-out q.S / (q.z + eps)
    has no floor and loses all relative accuracy where q.z passes near 0 (the
    max1 read-out floors it at 1).  Its tests take positive q and k, which
    keep the denominator away from 0."""
    if normalize is True:
        x.q, x.k = x.q.abs(), x.k.abs()
    return x


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("chunk", [32, 64])
@pytest.mark.parametrize("fgate_exp", [False, True])
def test_mfma_mlstm_vs_oracle(d, chunk, fgate_exp):
    dev = gpu_device()
    B, H, T = 2, 3, 333
    x = I.prefill_inputs(B, H, T, d, dtype="bf16", seed=d + chunk + fgate_exp, decay="mlstm",
                         scale=2.0 ** -0.5)
    if fgate_exp:
        x.fgate = -torch.nn.functional.softplus(-x.fgate)   # log sigmoid: same gates, exp form
    for segments in (1, 0, 3):
        desc = la.make_desc(B, H, T, d, d, 1, phi="identity", igate=x.igate, fgate=x.fgate,
                            chunk=chunk, segments=segments, normalize="max1",
                            stab=torch.empty(1))
        assert la.prefill_plan(desc)[2] == 1
        got = run(x, dev, chunk=chunk, segments=segments, normalize="max1", fgate_exp=fgate_exp)
        e = errors(got, oracle(x, fgate_exp=fgate_exp))
        print(d, chunk, fgate_exp, segments, e)
        assert max(e[:3]) < TOL["bf16"] and e[3] < 1e-3, e


@pytest.mark.parametrize("normalize", ["max1", True, False])
@pytest.mark.parametrize("segments", [1, 0])
def test_mfma_mlstm_readouts_and_carried_state(normalize, segments):
    dev = gpu_device()
    B, H, T, d = 1, 4, 500, 128
    x = condition(I.prefill_inputs(B, H, T, d, dtype="bf16", seed=31, decay="mlstm",
                                   scale=2.0 ** -0.5), normalize)
    state = random_state(B, H, d, d, 5, positive=normalize is True)
    got = run(x, dev, state=state, segments=segments, normalize=normalize)
    e = errors(got, oracle(x, state=state, normalize=normalize))
    print(normalize, segments, e)
    assert max(e[:3]) < TOL["bf16"] and e[3] < 1e-3, e


def test_mfma_mlstm_input_gates_beyond_fp32_range():
    # i = e^{100 + x} overflows fp32; the stabilised state does not.  A common
    # factor e^{100} on every weight makes |q.z| >> 1 everywhere, so the max1
    # read-out becomes q.S / |q.z| and needs the positive features of the
    # sum read-out's tests to stay well conditioned.
    dev = gpu_device()
    B, H, T, d = 1, 2, 300, 64
    x = condition(I.prefill_inputs(B, H, T, d, dtype="bf16", seed=8, decay="mlstm",
                                   scale=2.0 ** -0.5), True)
    x.igate = x.igate + 100.0
    for segments in (1, 0):
        got = run(x, dev, segments=segments, normalize="max1")
        assert all(torch.isfinite(t).all() for t in got)
        e = errors(got, oracle(x))
        print(segments, e)
        assert max(e[:3]) < TOL["bf16"] and e[3] < 1e-3, e


@pytest.mark.parametrize("d,tail", [(128, 17), (128, 26), (64, 20)])
def test_mfma_mlstm_ragged_tail_in_multi_segment_state(d, tail):
    # the stage-1 lane reads of the last valid rows (see the same test for
    # the SSD decay), with the mLSTM weights
    dev = gpu_device()
    T = 12 * 32 + tail
    x = I.prefill_inputs(1, 2, T, d, dtype="bf16", seed=21, decay="mlstm", scale=2.0 ** -0.5)
    for segments in (2, 0):
        got = run(x, dev, segments=segments, normalize="max1")
        e = errors(got, oracle(x))
        print(d, tail, segments, e)
        assert max(e[:3]) < TOL["bf16"] and e[3] < 1e-3, e


def test_mlstm_fp16_inputs_take_the_per_token_kernel():
    # fp16 q, k would enter the MFMAs rounded to bf16; identity features
    # cancel in q.k, so the chunked kernel takes bf16 inputs only and fp16
    # runs on the per-token kernel in fp32
    dev = gpu_device()
    x = I.prefill_inputs(2, 2, 260, 64, dtype="f16", seed=12, decay="mlstm", scale=2.0 ** -0.5)
    desc = la.make_desc(2, 2, 260, 64, 64, la._lib.LA_F16, phi="identity", igate=x.igate,
                        fgate=x.fgate, stab=torch.empty(1))
    assert la.prefill_plan(desc)[2] == 0
    got = run(x, dev, out_dtype=torch.float16, normalize="max1")
    o_ref = oracle(x)
    ex = (np.abs(got[0].double().cpu().numpy() - o_ref[0]) - 2.0 ** -11 * np.abs(o_ref[0])).max()
    rms = float(np.sqrt(np.mean(o_ref[0] ** 2)))
    print("fp16", max(ex, 0) / rms, errors(got, o_ref)[1:])
    assert max(ex, 0) / rms < TOL["f16"]
    assert max(errors(got, o_ref)[1:3]) < TOL["f16"]


def test_mfma_mlstm_continuation():
    # prefill(T1) then prefill(T2) from its state equals prefill(T1 + T2)
    dev = gpu_device()
    B, H, T, T1, d = 1, 2, 700, 290, 128
    x = I.prefill_inputs(B, H, T, d, dtype="bf16", seed=21, decay="mlstm", scale=2.0 ** -0.5)
    cut = lambda a, b: I.PrefillInputs(x.q[:, :, a:b].contiguous(), x.k[:, :, a:b].contiguous(),
                                       x.v[:, :, a:b].contiguous(),
                                       igate=x.igate[:, :, a:b].contiguous(),
                                       fgate=x.fgate[:, :, a:b].contiguous())
    o1, S1, z1, m1 = run(cut(0, T1), dev, normalize="max1")
    o2, S2, z2, m2 = run(cut(T1, T), dev, state=(S1.cpu(), z1.cpu(), m1.cpu()), normalize="max1")
    ref = oracle(x)
    got = (torch.cat([o1, o2], dim=2), S2, z2, m2)
    e = errors(got, ref)
    print(e)
    assert max(e[:3]) < TOL["bf16"] and e[3] < 1e-3, e


@pytest.mark.parametrize("fgate_exp", [False, True])
@pytest.mark.parametrize("normalize", ["max1", True, False])
def test_per_token_mlstm_fp32(fgate_exp, normalize):
    dev = gpu_device()
    B, H, T, d, dv = 2, 3, 57, 16, 8
    x = condition(I.prefill_inputs(B, H, T, d, dv, dtype="f32", seed=3, decay="mlstm"),
                  normalize)
    if fgate_exp:
        x.fgate = -torch.nn.functional.softplus(-x.fgate)
    state = random_state(B, H, d, dv, 9, positive=normalize is True)
    got = run(x, dev, state=state, normalize=normalize, fgate_exp=fgate_exp)
    e = errors(got, oracle(x, state=state, fgate_exp=fgate_exp, normalize=normalize))
    print(fgate_exp, normalize, e)
    assert max(e[:3]) < TOL["f32"] and e[3] < 1e-5, e


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("d,dv", [(64, 64), (128, 64), (128, 128)])
@pytest.mark.parametrize("normalize", ["max1", True])
def test_decode_mlstm_steps(dtype, d, dv, normalize):
    dev = gpu_device()
    N, H, steps = 40, 4, 6
    x = condition(I.prefill_inputs(N, H, steps, d, dv, dtype=dtype, seed=d + dv, decay="mlstm",
                                   scale=2.0 ** -0.5), normalize)
    S, z, m = la.state_init(N, H, d, dv, dev, stab=True)
    outs = []
    for t in range(steps):
        g = lambda a: a[:, :, t].contiguous().to(dev)
        outs.append(la.decode_step(g(x.q), g(x.k), g(x.v), S, z, phi="identity", igate=g(x.igate),
                                   fgate=g(x.fgate), stab=m, normalize=normalize,
                                   out_dtype=torch.float32))
    torch.cuda.synchronize()
    o = torch.stack(outs, dim=2)
    ref = oracle(x, normalize=normalize)
    e = errors((o, S, z, m), ref)
    print(dtype, d, dv, normalize, e)
    assert max(e[:3]) < TOL[dtype] and e[3] < 1e-5, e


def test_prefill_then_decode_mlstm():
    dev = gpu_device()
    B, H, T, d, extra = 2, 4, 320, 128, 3
    x = I.prefill_inputs(B, H, T + extra, d, dtype="bf16", seed=44, decay="mlstm",
                         scale=2.0 ** -0.5)
    head = I.PrefillInputs(x.q[:, :, :T].contiguous(), x.k[:, :, :T].contiguous(),
                           x.v[:, :, :T].contiguous(), igate=x.igate[:, :, :T].contiguous(),
                           fgate=x.fgate[:, :, :T].contiguous())
    _, S, z, m = run(head, dev, normalize="max1")
    outs = []
    for t in range(T, T + extra):
        g = lambda a: a[:, :, t].contiguous().to(dev)
        outs.append(la.decode_step(g(x.q), g(x.k), g(x.v), S, z, phi="identity", igate=g(x.igate),
                                   fgate=g(x.fgate), stab=m, normalize="max1",
                                   out_dtype=torch.float32))
    torch.cuda.synchronize()
    ref = oracle(x)
    e = errors((torch.stack(outs, dim=2), S, z, m),
               (ref[0][:, :, T:], ref[1], ref[2], ref[3]))
    print(e)
    assert max(e[:3]) < TOL["bf16"] and e[3] < 1e-3, e
