"""Decode step on the GPU vs the fp64 oracle: every (d', d_v) the one-wave-per-state
kernel specialises, every decay kind and input type, a sequence count that
leaves the last workgroup partly empty, and the gated random-feature decode
workload at full size (256 sequences x 16 heads, 1024 steps) on sampled
states.  Tolerance: max |gpu - oracle| / rms(oracle) <= 1e-4 (fp32 inputs),
2e-2 (bf16/fp16 inputs)."""
import numpy as np
import pytest
import torch

import fixed_state_sequence_amd as la
from fixed_state_sequence_amd import inputs as I
from oracle import linattn_oracle as O
from conftest import rel_err, TOL, gpu_device

pytestmark = pytest.mark.gpu


def _run_steps(N, H, dh, dv, phi, D, decay, dtype, steps, seed, out_dtype=torch.float32):
    dev = gpu_device()
    W = I.rff_projection(H, D, dh, seed=seed) if phi == "rff" else None
    dp = 2 * D if phi == "rff" else dh
    S, z = la.state_init(N, H, dp, dv, dev)
    S_ref, z_ref = np.zeros((N, H, dp, dv)), np.zeros((N, H, dp))
    sd = I.DTYPES[dtype]
    worst = 0.0
    for step in range(steps):
        st = I.rfa_decode_step_inputs(N, H, dh, dv, step=step, seed=seed)
        q, k, v = st.q.to(sd), st.k.to(sd), st.v.to(sd)
        kw = {}
        if decay == "ssd":
            kw["decay"] = st.gate * 0.5 + 0.5     # a in (0.5, 1)
        elif decay == "rfa":
            kw["gate"] = st.gate
        o = la.decode_step(q.to(dev), k.to(dev), v.to(dev), S, z, phi=phi,
                           W=None if W is None else W.to(dev),
                           **{n: t.to(dev) for n, t in kw.items()}, out_dtype=out_dtype)
        torch.cuda.synchronize()
        o_ref, S_ref, z_ref = O.decode_step(q, k, v, S_ref, z_ref, phi=phi, W=W, **kw)
        worst = max(worst, rel_err(o, o_ref))
    return worst, rel_err(S, S_ref), rel_err(z, z_ref)


@pytest.mark.parametrize("dv", [64, 128])
@pytest.mark.parametrize("phi,dh,D", [("elu1", 64, 0), ("elu1", 128, 0), ("elu1", 256, 0),
                                      ("rff", 64, 32), ("rff", 64, 64), ("rff", 100, 128)])
@pytest.mark.parametrize("decay", [None, "ssd", "rfa"])
def test_decode_shapes_fp32(dv, phi, dh, D, decay):
    e = _run_steps(N=7, H=3, dh=dh, dv=dv, phi=phi, D=D, decay=decay, dtype="f32", steps=4,
                   seed=dh + dv + D)
    print(dv, phi, dh, D, decay, e)
    assert max(e) < TOL["f32"], e


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("phi,dh,D", [("elu1", 128, 0), ("rff", 64, 64)])
def test_decode_16bit_inputs(dtype, phi, dh, D):
    e = _run_steps(N=9, H=2, dh=dh, dv=64, phi=phi, D=D, decay="rfa", dtype=dtype, steps=3,
                   seed=5)
    assert max(e) < TOL[dtype], e


def test_decode_16bit_output_rounding():
    # a bf16 output is the fp32 result rounded to nearest even
    dev = gpu_device()
    N, H, dh = 5, 2, 64
    st = I.rfa_decode_step_inputs(N, H, dh, step=0, seed=2)
    q, k, v = (t.to(torch.bfloat16) for t in (st.q, st.k, st.v))
    S, z = la.state_init(N, H, dh, dh, dev)
    S2, z2 = la.state_init(N, H, dh, dh, dev)
    o16 = la.decode_step(q.to(dev), k.to(dev), v.to(dev), S, z, gate=st.gate.to(dev))
    o32 = la.decode_step(q.to(dev), k.to(dev), v.to(dev), S2, z2, gate=st.gate.to(dev),
                         out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert o16.dtype == torch.bfloat16
    assert torch.equal(o16, o32.to(torch.bfloat16))
    assert torch.equal(S, S2) and torch.equal(z, z2)


def test_decode_rff_workload_full_size_sampled():
    """256 sequences x 16 heads, d_h = d_v = 64, D = 64 pairs, gate, fp32, 1024
    steps: the GPU runs every state; the oracle follows 48 sampled states and
    checks their outputs at every step and their final state."""
    dev = gpu_device()
    N, H, dh, D, steps = 256, 16, 64, 64, 1024
    W = I.rff_projection(H, D, dh, seed=0)
    x = I.rfa_decode_batch(steps, N, H, dh, seed=1, device=dev)
    rng = np.random.default_rng(0)
    ns = torch.as_tensor(rng.integers(0, N, 48))
    hs = torch.as_tensor(rng.integers(0, H, 48))
    S, z = la.state_init(N, H, 2 * D, dh, dev)
    outs = torch.empty(steps, 48, dh, device=dev)
    Wd = W.to(dev)
    for t in range(steps):
        o = la.decode_step(x.q[t], x.k[t], x.v[t], S, z, phi="rff", W=Wd, gate=x.gate[t])
        outs[t] = o[ns, hs]
    torch.cuda.synchronize()
    q = x.q[:, ns, hs].cpu().numpy()
    k = x.k[:, ns, hs].cpu().numpy()
    v = x.v[:, ns, hs].cpu().numpy()
    g = x.gate[:, ns, hs].cpu().numpy()
    Wn = W.numpy()[hs.numpy()]                              # [48, D, dh]
    # the sampled states as 48 "heads" of one batch entry, tokens = steps
    fq = O.phi_rff(q.transpose(1, 0, 2)[None], Wn)[0]     # [48, steps, 2D]
    fk = O.phi_rff(k.transpose(1, 0, 2)[None], Wn)[0]
    a, b = O.decay_coefficients(gate=g.T)
    o_ref, S_ref, z_ref = O.recurrence(fq, fk, v.transpose(1, 0, 2), a, b)
    got = outs.cpu().numpy().transpose(1, 0, 2)
    e = (rel_err(got, o_ref), rel_err(S[ns, hs], S_ref), rel_err(z[ns, hs], z_ref))
    print("rff decode full size", e)
    assert max(e) < TOL["f32"], e


@pytest.mark.parametrize("decay", ["rfa", "ssd", None])
def test_decode_state_set_beyond_the_last_level_cache(decay):
    """1027 sequences x 16 heads of 128 x 64 states (568 MB, more than the
    256 MB last-level cache: the four-wave split of each state), 24 steps
    from a zero state (random-feature denominators stay away from 0 as in the
    decode workload); 40 sampled states (the last, partly filled workgroup
    among them) followed by the oracle step by step."""
    dev = gpu_device()
    N, H, dh, D, steps = 1027, 16, 64, 64, 24
    W = I.rff_projection(H, D, dh, seed=5)
    S, z = la.state_init(N, H, 2 * D, dh, dev)
    rng = np.random.default_rng(7)
    ns = np.concatenate([rng.integers(0, N, 36), [N - 1, N - 2, N - 3, 0]])
    hs = np.concatenate([rng.integers(0, H, 36), [15, 0, 7, 3]])
    S_ref = S[ns, hs].double().cpu().numpy()
    z_ref = z[ns, hs].double().cpu().numpy()
    Wd = W.to(dev)
    worst = 0.0
    for t in range(steps):
        st = I.rfa_decode_step_inputs(N, H, dh, step=t, seed=8, device=dev)
        kw = {} if decay is None else ({"gate": st.gate} if decay == "rfa" else
                                       {"decay": st.gate * 0.5 + 0.5})
        o = la.decode_step(st.q, st.k, st.v, S, z, phi="rff", W=Wd, **kw)
        torch.cuda.synchronize()
        kwr = {n: t_[ns, hs].cpu() for n, t_ in kw.items()}
        o_ref, S_ref, z_ref = O.decode_step(st.q[ns, hs].cpu(), st.k[ns, hs].cpu(),
                                            st.v[ns, hs].cpu(), S_ref, z_ref, phi="rff",
                                            W=W[torch.as_tensor(hs)], **kwr)
        worst = max(worst, rel_err(o[ns, hs], o_ref))
    e = (worst, rel_err(S[ns, hs], S_ref), rel_err(z[ns, hs], z_ref))
    print("decode beyond the LLC", decay, e)
    assert max(e) < TOL["f32"], e


def test_mis_shaped_W_raises_before_any_launch():
    # W must be [H, rff_D, d_h]: fewer heads or a wrong input width would be
    # read out of bounds by the kernels, so the binding refuses it.
    dev = gpu_device()
    N, H, dh, dv, D = 4, 8, 64, 64, 64
    st = I.rfa_decode_step_inputs(N, H, dh, dv, step=0, seed=0)
    S, z = la.state_init(N, H, 2 * D, dv, dev)
    q, k, v, g = (t.to(dev) for t in (st.q, st.k, st.v, st.gate))
    for shape in ((H - 1, D, dh), (H, D, dh + 1), (D, dh)):
        W = torch.zeros(shape, device=dev)
        with pytest.raises(ValueError, match="W has shape"):
            la.decode_step(q, k, v, S, z, phi="rff", W=W, gate=g)
        with pytest.raises(ValueError, match="W has shape"):
            la.prefill(q[:, :, None], k[:, :, None], v[:, :, None], phi="rff", W=W)
    torch.cuda.synchronize()
    assert torch.count_nonzero(S).item() == 0 and torch.count_nonzero(z).item() == 0
