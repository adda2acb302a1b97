"""GPU path vs the fp64 oracle, element by element, on seeded inputs.

Tolerance (max |gpu - oracle| / rms(oracle)): 1e-4 for fp32 inputs and 2e-2
for bf16/fp16 inputs.  Small cases span several chunks, a ragged tail and
several segments; every decay kind, chunk size and width is covered.
"""
import numpy as np
import pytest
import torch

import fixed_state_sequence_amd as la
from fixed_state_sequence_amd import inputs as I
from oracle import linattn_oracle as O
from conftest import rel_err, TOL, gpu_device

pytestmark = pytest.mark.gpu


def run_prefill(x, dev, **kw):
    g = lambda t: None if t is None else t.to(dev)
    kw.setdefault("out_dtype", torch.float32)
    out, S, z = la.prefill(g(x.q), g(x.k), g(x.v), decay=g(x.decay), gate=g(x.gate), **kw)
    torch.cuda.synchronize()
    return out, S, z


def oracle_prefill(x, **kw):
    return O.causal_linear_attention(x.q, x.k, x.v, decay=x.decay, gate=x.gate, **kw)


def test_tiny_worked_example_fp32():
    dev = gpu_device()
    x = I.workload_inputs("tiny_causal_t8_d4")
    out, S, z = run_prefill(x, dev)
    o_ref, S_ref, z_ref = oracle_prefill(x)
    print("tiny", rel_err(out, o_ref), rel_err(S, S_ref))
    assert rel_err(out, o_ref) < TOL["f32"]
    assert rel_err(S, S_ref) < TOL["f32"] and rel_err(z, z_ref) < TOL["f32"]
    # and the masked-quadratic form the page checks against
    q = O.phi_elu1(x.q); k = O.phi_elu1(x.k)
    assert rel_err(out, O.masked_quadratic(q, k, x.v)) < TOL["f32"]


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("decay", [None, "ssd", "rfa"])
@pytest.mark.parametrize("chunk", [32, 64, 128])
def test_prefill_mfma_vs_oracle(d, decay, chunk):
    dev = gpu_device()
    if d == 128 and chunk == 128:
        pytest.skip("chunk 128 with d = 128 does not fit in LDS (rejected, see test_abi)")
    x = I.prefill_inputs(2, 3, 333, d, dtype="bf16", seed=d + chunk, decay=decay)
    for segments in (1, 0, 3):
        desc = la.make_desc(2, 3, 333, d, d, 1, decay=x.decay, gate=x.gate, chunk=chunk,
                            segments=segments)
        assert la.prefill_plan(desc)[2] == 1
        out, S, z = run_prefill(x, dev, chunk=chunk, segments=segments)
        o_ref, S_ref, z_ref = oracle_prefill(x)
        e = (rel_err(out, o_ref), rel_err(S, S_ref), rel_err(z, z_ref))
        print(d, decay, chunk, segments, e)
        assert max(e) < TOL["bf16"], e


@pytest.mark.parametrize("d,tail", [(128, 17), (128, 25), (128, 26), (64, 17), (64, 20)])
@pytest.mark.parametrize("decay", ["ssd", "rfa"])
def test_prefill_ragged_tail_in_multi_segment_state(d, tail, decay):
    # Regression: stage 1 reads each row's log-decay prefix from the lane of
    # its token.  With these tails the last valid rows take that value from
    # lanes whose own rows lie past the end; the read must still run in those
    # lanes, or the weights of the last tokens (and the final state) go wrong
    # while every output stays right.
    dev = gpu_device()
    T = 12 * 32 + tail
    x = I.prefill_inputs(1, 2, T, d, dtype="bf16", seed=21, decay=decay, scale=2.0 ** -0.5)
    for segments in (2, 0):
        out, S, z = run_prefill(x, dev, segments=segments)
        o_ref, S_ref, z_ref = oracle_prefill(x)
        e = (rel_err(out, o_ref), rel_err(S, S_ref), rel_err(z, z_ref))
        print(d, tail, decay, segments, e)
        assert max(e) < TOL["bf16"], e


@pytest.mark.parametrize("decay", [None, "ssd"])
def test_prefill_fp16_inputs(decay):
    dev = gpu_device()
    x = I.prefill_inputs(1, 2, 200, 64, dtype="f16", seed=5, decay=decay)
    out, S, z = run_prefill(x, dev)
    o_ref, S_ref, _ = oracle_prefill(x)
    assert rel_err(out, o_ref) < TOL["f16"] and rel_err(S, S_ref) < TOL["f16"]


@pytest.mark.parametrize("dtype,d,decay", [("bf16", 128, None), ("bf16", 64, "ssd"),
                                           ("f16", 128, "rfa"), ("bf16", 32, None)])
def test_prefill_16bit_outputs(dtype, d, decay):
    # A 16-bit output is the fp32 result rounded to nearest even: each element is
    # within half an ulp (at most 2^-8 relative for bf16, 2^-11 for fp16) of the
    # oracle, plus the compute error allowed for 16-bit inputs.
    dev = gpu_device()
    x = I.prefill_inputs(2, 2, 300, d, dtype=dtype, seed=17, decay=decay)
    out, S, z = run_prefill(x, dev, out_dtype=I.DTYPES[dtype])
    assert out.dtype == I.DTYPES[dtype]
    o_ref, S_ref, _ = oracle_prefill(x)
    half_ulp = 2.0 ** -8 if dtype == "bf16" else 2.0 ** -11   # relative, worst case in a binade
    got = out.double().cpu().numpy()
    excess = np.abs(got - o_ref) - half_ulp * np.abs(o_ref)
    assert excess.max() / np.sqrt(np.mean(o_ref ** 2)) < TOL[dtype]
    assert rel_err(S, S_ref) < TOL[dtype]


@pytest.mark.parametrize("dtype,d,decay", [("f32", 64, None), ("f32", 128, "ssd"),
                                           ("f32", 32, "rfa"), ("bf16", 32, None),
                                           ("bf16", 16, "ssd"), ("f16", 8, None)])
def test_prefill_recurrent_path_vs_oracle(dtype, d, decay):
    dev = gpu_device()
    x = I.prefill_inputs(2, 2, 150, d, dtype=dtype, seed=3, decay=decay)
    desc = la.make_desc(2, 2, 150, d, d, {"f32": 0, "bf16": 1, "f16": 2}[dtype],
                        decay=x.decay, gate=x.gate)
    assert la.prefill_plan(desc)[2] == 0
    out, S, z = run_prefill(x, dev)
    o_ref, S_ref, z_ref = oracle_prefill(x)
    e = (rel_err(out, o_ref), rel_err(S, S_ref), rel_err(z, z_ref))
    print(dtype, d, decay, e)
    assert max(e) < TOL[dtype], e


def test_prefill_rff_fp32_vs_oracle():
    dev = gpu_device()
    x = I.prefill_inputs(2, 3, 64, 64, dtype="f32", seed=9, decay="rfa", rff_D=64,
                         unit_norm_qk=True)
    out, S, z = run_prefill(x, dev, phi="rff", W=x.W.to(dev))
    o_ref, S_ref, z_ref = oracle_prefill(x, phi="rff", W=x.W)
    e = (rel_err(out, o_ref), rel_err(S, S_ref), rel_err(z, z_ref))
    print("rff prefill", e)
    assert max(e) < TOL["f32"], e


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("bf16", 64), ("f32", 64)])
def test_prefill_continues_from_state(dtype, d):
    # prefill(T1) then prefill(T2) from the carried state == the oracle over T1 + T2
    dev = gpu_device()
    x = I.prefill_inputs(1, 2, 300, d, dtype=dtype, seed=21, decay="ssd")
    g = lambda t, a, b: t[:, :, a:b].contiguous().to(dev)
    o1, S, z = la.prefill(g(x.q, 0, 130), g(x.k, 0, 130), g(x.v, 0, 130), decay=g(x.decay, 0, 130),
                          out_dtype=torch.float32)
    o2, S, z = la.prefill(g(x.q, 130, 300), g(x.k, 130, 300), g(x.v, 130, 300),
                          decay=g(x.decay, 130, 300), state=(S, z), segments=2,
                          out_dtype=torch.float32)
    torch.cuda.synchronize()
    o_ref, S_ref, z_ref = oracle_prefill(x)
    got = torch.cat([o1, o2], dim=2)
    e = (rel_err(got, o_ref), rel_err(S, S_ref), rel_err(z, z_ref))
    print("continuation", dtype, d, e)
    assert max(e) < TOL[dtype], e


def test_prefill_then_decode_equals_longer_prefill():
    dev = gpu_device()
    x = I.prefill_inputs(2, 2, 96, 64, dtype="f32", seed=4, decay="ssd")
    T1 = 80
    sl = lambda t, a, b: t[:, :, a:b].contiguous().to(dev)
    _, S, z = la.prefill(sl(x.q, 0, T1), sl(x.k, 0, T1), sl(x.v, 0, T1), decay=sl(x.decay, 0, T1))
    outs = []
    for t in range(T1, 96):
        outs.append(la.decode_step(x.q[:, :, t].contiguous().to(dev), x.k[:, :, t].contiguous().to(dev),
                                   x.v[:, :, t].contiguous().to(dev), S, z,
                                   decay=x.decay[:, :, t].contiguous().to(dev)))
    torch.cuda.synchronize()
    o_ref, S_ref, _ = oracle_prefill(x)
    assert rel_err(torch.stack(outs, dim=2), o_ref[:, :, T1:]) < TOL["f32"]
    assert rel_err(S, S_ref) < TOL["f32"]


def test_prefill_edge_shapes():
    dev = gpu_device()
    # T = 0: no-op, state unchanged
    S0 = torch.randn(1, 2, 64, 64, device=dev)
    z0 = torch.rand(1, 2, 64, device=dev)
    S, z = S0.clone(), z0.clone()
    e = torch.empty(1, 2, 0, 64, dtype=torch.bfloat16, device=dev)
    out, S, z = la.prefill(e, e, e, state=(S, z))
    torch.cuda.synchronize()
    assert out.shape == (1, 2, 0, 64) and torch.equal(S, S0) and torch.equal(z, z0)
    # T = 1, T < chunk, B*H = 1, with a carried-in state
    for T in (1, 5, 64, 65):
        x = I.prefill_inputs(1, 1, T, 128, dtype="bf16", seed=T, decay="ssd")
        Sx = torch.rand(1, 1, 128, 128) * 0.1
        zx = torch.rand(1, 1, 128) + 1.0
        out, S, z = la.prefill(x.q.to(dev), x.k.to(dev), x.v.to(dev), decay=x.decay.to(dev),
                               state=(Sx.to(dev), zx.to(dev)), out_dtype=torch.float32)
        torch.cuda.synchronize()
        o_ref, S_ref, _ = O.causal_linear_attention(x.q, x.k, x.v, decay=x.decay, S0=Sx, z0=zx)
        assert rel_err(out, o_ref) < TOL["bf16"] and rel_err(S, S_ref) < TOL["bf16"], T


def test_decay_zero_and_one():
    dev = gpu_device()
    x = I.prefill_inputs(1, 2, 200, 128, dtype="bf16", seed=8)
    # a == 1 everywhere equals no decay (to rounding); a == 0 at t resets the state
    ones = torch.ones(1, 2, 200)
    o1, S1, _ = la.prefill(x.q.to(dev), x.k.to(dev), x.v.to(dev), decay=ones.to(dev),
                           out_dtype=torch.float32)
    o0, S0, _ = la.prefill(x.q.to(dev), x.k.to(dev), x.v.to(dev), out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert rel_err(o1, o0.cpu().numpy()) < 1e-4
    a = torch.full((1, 2, 200), 0.97)
    a[:, :, 100] = 0.0
    o, S, z = la.prefill(x.q.to(dev), x.k.to(dev), x.v.to(dev), decay=a.to(dev), segments=3,
                         out_dtype=torch.float32)
    torch.cuda.synchronize()
    o_ref, S_ref, _ = O.causal_linear_attention(x.q, x.k, x.v, decay=a)
    assert rel_err(o, o_ref) < TOL["bf16"] and rel_err(S, S_ref) < TOL["bf16"]


@pytest.mark.parametrize("kind", ["ssd", "rfa"])
def test_decay_carry_deferred_then_applied(kind):
    """The output stage keeps the chunks' carry factors in a running log
    scale while it stays within a bound, then applies it to the state.
    Decays of 1 (gate 0.999) with sparse strong ones make that scale cross
    the bound at several places inside a segment, once within one chunk
    (a decay of 1e-20); every output and the final state against the oracle."""
    dev = gpu_device()
    T = 1500
    x = I.prefill_inputs(1, 2, T, 128, dtype="bf16", seed=21)
    a = torch.full((1, 2, T), 1.0 if kind == "ssd" else 0.999)
    a[:, :, 37::37] = 0.02
    a[:, 1, 900] = 1e-20
    kw = dict(decay=a) if kind == "ssd" else dict(gate=a)
    o_ref, S_ref, z_ref = O.causal_linear_attention(x.q, x.k, x.v, **kw)
    for segments in (1, 0, 3):
        o, S, z = la.prefill(x.q.to(dev), x.k.to(dev), x.v.to(dev), segments=segments,
                             out_dtype=torch.float32, **{n: t.to(dev) for n, t in kw.items()})
        torch.cuda.synchronize()
        e = (rel_err(o, o_ref), rel_err(S, S_ref), rel_err(z, z_ref))
        print(kind, segments, e)
        assert max(e) < TOL["bf16"], e


def test_prefill_stages_compose_to_prefill():
    dev = gpu_device()
    x = I.prefill_inputs(1, 4, 700, 128, dtype="bf16", seed=2)
    q, k, v = x.q.to(dev), x.k.to(dev), x.v.to(dev)
    ref, _, _ = la.prefill(q, k, v, segments=5)
    desc = la.make_desc(1, 4, 700, 128, 128, 1, segments=5)
    assert la.prefill_plan(desc)[1] == 5   # 22 chunks of 32, 5 per segment
    ws = torch.empty(la.prefill_workspace_size(desc), dtype=torch.uint8, device=dev)
    S, z = la.state_init(1, 4, 128, 128, dev)
    out = torch.empty_like(q)
    for st in (1, 2, 3):
        la.prefill_stage(st, q, k, v, S, z, out, ws, segments=5)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)


@pytest.mark.parametrize("phi,dtype,gate", [("rff", "f32", True), ("elu1", "f32", False),
                                            ("elu1", "bf16", True)])
def test_decode_steps_vs_oracle(phi, dtype, gate):
    dev = gpu_device()
    N, H, dh = 16, 4, 64
    W = I.rff_projection(H, 64, dh, seed=1) if phi == "rff" else None
    dp = 128 if phi == "rff" else dh
    S, z = la.state_init(N, H, dp, dh, dev)
    S_ref = np.zeros((N, H, dp, dh)); z_ref = np.zeros((N, H, dp))
    sd = I.DTYPES[dtype]
    for step in range(6):
        st = I.rfa_decode_step_inputs(N, H, dh, step=step, seed=1)
        q, k, v = st.q.to(sd), st.k.to(sd), st.v.to(sd)
        o = la.decode_step(q.to(dev), k.to(dev), v.to(dev), S, z, phi=phi,
                           W=None if W is None else W.to(dev),
                           gate=st.gate.to(dev) if gate else None, out_dtype=torch.float32)
        torch.cuda.synchronize()
        o_ref, S_ref, z_ref = O.decode_step(q, k, v, S_ref, z_ref, phi=phi, W=W,
                                            gate=st.gate if gate else None)
        e = rel_err(o, o_ref)
        assert e < TOL[dtype], (step, e)
    assert rel_err(S, S_ref) < TOL[dtype] and rel_err(z, z_ref) < TOL[dtype]


# ---------------------------------------------- the normaliser-free read-out

@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("decay", [None, "ssd", "rfa"])
def test_prefill_unnormalised_mfma(d, decay):
    # o_t = phi(q_t)^T S_t: the chunked path with the division left out, over
    # one, the default and three segments
    dev = gpu_device()
    x = I.prefill_inputs(2, 3, 301, d, dtype="bf16", seed=7 + d, decay=decay)
    o_ref, S_ref, z_ref = oracle_prefill(x, normalize=False)
    for segments in (1, 0, 3):
        out, S, z = run_prefill(x, dev, segments=segments, normalize=False)
        e = (rel_err(out, o_ref), rel_err(S, S_ref), rel_err(z, z_ref))
        print("unnormalised", d, decay, segments, e)
        assert max(e) < TOL["bf16"], e


@pytest.mark.parametrize("phi", ["elu1", "rff"])
def test_prefill_unnormalised_per_token_fp32(phi):
    dev = gpu_device()
    x = I.prefill_inputs(2, 2, 70, 32, dtype="f32", seed=3, decay="rfa")
    W = I.rff_projection(2, 16, 32, seed=4) if phi == "rff" else None
    out, S, z = run_prefill(x, dev, phi=phi, W=None if W is None else W.to(dev),
                            normalize=False)
    o_ref, S_ref, z_ref = oracle_prefill(x, phi=phi, W=W, normalize=False)
    e = (rel_err(out, o_ref), rel_err(S, S_ref), rel_err(z, z_ref))
    assert max(e) < TOL["f32"], e


@pytest.mark.parametrize("phi,dh,D", [("rff", 64, 64), ("elu1", 128, 0)])
def test_decode_unnormalised(phi, dh, D):
    dev = gpu_device()
    N, H = 9, 3
    W = I.rff_projection(H, D, dh, seed=1) if phi == "rff" else None
    dp = 2 * D if phi == "rff" else dh
    S, z = la.state_init(N, H, dp, 64, dev)
    S_ref, z_ref = np.zeros((N, H, dp, 64)), np.zeros((N, H, dp))
    for step in range(3):
        st = I.rfa_decode_step_inputs(N, H, dh, 64, step=step, seed=2)
        o = la.decode_step(st.q.to(dev), st.k.to(dev), st.v.to(dev), S, z, phi=phi,
                           W=None if W is None else W.to(dev), gate=st.gate.to(dev),
                           normalize=False)
        torch.cuda.synchronize()
        o_ref, S_ref, z_ref = O.decode_step(st.q, st.k, st.v, S_ref, z_ref, phi=phi, W=W,
                                            gate=st.gate, normalize=False)
        assert rel_err(o, o_ref) < TOL["f32"]
    assert rel_err(S, S_ref) < TOL["f32"] and rel_err(z, z_ref) < TOL["f32"]


# ------------------------------------------------------------ the non-causal form

def oracle_noncausal(x, **kw):
    return O.noncausal_linear_attention(x.q, x.k, x.v, **kw)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("normalize", [True, False])
@pytest.mark.parametrize("chunk", [32, 64])
def test_prefill_noncausal_mfma(d, normalize, chunk):
    # every output reads the whole sequence's state, from one, the default
    # and three segments, with and without a carried-in state
    dev = gpu_device()
    x = I.prefill_inputs(2, 3, 333, d, dtype="bf16", seed=11 + d + chunk)
    o_ref, S_ref, z_ref = oracle_noncausal(x, normalize=normalize)
    for segments in (1, 0, 3):
        out, S, z = run_prefill(x, dev, chunk=chunk, segments=segments, normalize=normalize,
                                causal=False)
        e = (rel_err(out, o_ref), rel_err(S, S_ref), rel_err(z, z_ref))
        print("noncausal", d, normalize, chunk, segments, e)
        assert max(e) < TOL["bf16"], e
    S0 = torch.rand(2, 3, d, d) * 0.1
    z0 = torch.rand(2, 3, d) + 1.0
    o_ref, S_ref, _ = oracle_noncausal(x, normalize=normalize, S0=S0, z0=z0)
    out, S, z = run_prefill(x, dev, chunk=chunk, normalize=normalize, causal=False,
                            state=(S0.to(dev), z0.to(dev)))
    assert rel_err(out, o_ref) < TOL["bf16"] and rel_err(S, S_ref) < TOL["bf16"]


@pytest.mark.parametrize("phi", ["elu1", "rff"])
def test_prefill_noncausal_per_token_fp32(phi):
    # random features with unit-norm q, k, as in the gated decode workload:
    # with raw N(0, 1) inputs the kernel estimates sit near 0 and so do the
    # denominators
    dev = gpu_device()
    rff = phi == "rff"
    x = I.prefill_inputs(2, 2, 90, 32, dtype="f32", seed=8, rff_D=16 if rff else None,
                         unit_norm_qk=rff)
    W = x.W if rff else None
    out, S, z = run_prefill(x, dev, phi=phi, W=None if W is None else W.to(dev), causal=False)
    o_ref, S_ref, z_ref = oracle_noncausal(x, phi=phi, W=W)
    e = (rel_err(out, o_ref), rel_err(S, S_ref), rel_err(z, z_ref))
    assert max(e) < TOL["f32"], e



def test_stage1_fold_on_16x16x32_mfma():
    """The stage-1 fold built on v_mfma_f32_16x16x32_bf16 (selected by
    LA_STAGE1_MFMA=16x16x32, kept to measure the MFMA shape choice) gives the
    same segment states as the 32x32x16 fold up to summation order: outputs
    and final state against the oracle at the bf16 bar, and against the
    default fold to well under the bar (the read-out rounds the state to
    bf16, so an fp32 difference can flip a rounding)."""
    import os
    dev = gpu_device()
    x = I.prefill_inputs(1, 4, 3000, 128, dtype="bf16", seed=17, scale=2.0 ** -0.5)
    ref = run_prefill(x, dev, segments=6)
    os.environ["LA_STAGE1_MFMA"] = "16x16x32"
    try:
        got = run_prefill(x, dev, segments=6)
    finally:
        del os.environ["LA_STAGE1_MFMA"]
    o_ref, S_ref, z_ref = oracle_prefill(x)
    e = (rel_err(got[0], o_ref), rel_err(got[1], S_ref), rel_err(got[2], z_ref))
    d = tuple(rel_err(g, r.cpu().numpy()) for g, r in zip(got, ref))
    print("16x16x32 stage 1: vs oracle", e, "vs 32x32x16", d)
    assert max(e) < TOL["bf16"], e
    assert max(d) < 1e-3, d   # a state rounding to bf16 the other way moves an output ~1e-5
