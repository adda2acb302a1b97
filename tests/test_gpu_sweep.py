"""Seeded random sweeps of the GPU path against the fp64 oracle: shapes,
chunk lengths, segment counts, decay kinds and strengths, read-outs, output
types and carried-in states drawn together, so that combinations no
hand-written case names are covered too (forward, mLSTM forward, gradients
with and without the mLSTM gates, decode).  Every case prints its draw before
it runs.  Bars as everywhere: max |gpu - oracle| / rms(oracle) < 2e-2 for
bf16 inputs (16-bit outputs: after half an ulp of the oracle per element).
"""
import random

import numpy as np
import pytest
import torch

import fixed_state_sequence_amd as la
from fixed_state_sequence_amd import inputs as I
from oracle import linattn_oracle as O
from conftest import rel_err, TOL, gpu_device

pytestmark = pytest.mark.gpu


def _out_err(out, ref):
    got = out.detach().double().cpu().numpy()
    if out.dtype == torch.float32:
        return rel_err(got, ref)
    excess = np.abs(got - ref) - 2.0 ** -8 * np.abs(ref)   # half a bf16 ulp, worst case
    return float(excess.max() / np.sqrt(np.mean(ref ** 2)))


def _decay(x, kind, mean, rng_t):
    """Replace the decay/gate draw by one of the given strength."""
    a = torch.sigmoid(torch.randn(x.q.shape[:3], generator=rng_t) + mean).float()
    if kind == "ssd":
        x.decay, x.gate = a, None
    elif kind == "rfa":
        x.decay, x.gate = None, a
    else:
        x.decay = x.gate = None


def _forward_cases(n, seed):
    r = random.Random(seed)
    for i in range(n):
        d = r.choice([64, 128])
        yield dict(i=i, B=r.choice([1, 2, 3]), H=r.choice([1, 2, 3]), T=r.choice(
            [1, 2, 31, 32, 33, 63, 64, 95, 160, 257, 333] + [r.randint(1, 900) for _ in range(4)]),
            d=d, chunk=r.choice([0, 32, 64] + ([128] if d == 64 else [])),
            segments=r.choice([0, 1, 2, 3, 7]), kind=r.choice([None, "ssd", "rfa"]),
            mean=r.choice([-1.0, 1.0, 3.0, 6.0]), normalize=r.choice([True, True, False]),
            out=r.choice(["f32", "bf16"]), state=r.random() < 0.4, seed=1000 + i)


@pytest.mark.parametrize("case", list(_forward_cases(40, 7)), ids=lambda c: f"f{c['i']}")
def test_prefill_sweep(case):
    dev = gpu_device()
    c = case
    print(c, flush=True)
    x = I.prefill_inputs(c["B"], c["H"], c["T"], c["d"], dtype="bf16", seed=c["seed"],
                         scale=2.0 ** -0.5)
    _decay(x, c["kind"], c["mean"], torch.Generator().manual_seed(c["seed"]))
    S0 = z0 = None
    st = None
    if c["state"]:
        rng = np.random.default_rng(c["seed"])
        S0 = rng.standard_normal((c["B"], c["H"], c["d"], c["d"])) * 0.3
        z0 = np.abs(rng.standard_normal((c["B"], c["H"], c["d"]))) * 0.3 + 0.5
        st = (torch.tensor(S0, dtype=torch.float32, device=dev),
              torch.tensor(z0, dtype=torch.float32, device=dev))
        S0, z0 = st[0].cpu().double().numpy(), st[1].cpu().double().numpy()
    g = lambda t: None if t is None else t.to(dev)
    out, S, z = la.prefill(g(x.q), g(x.k), g(x.v), decay=g(x.decay), gate=g(x.gate), state=st,
                           chunk=c["chunk"], segments=c["segments"], normalize=c["normalize"],
                           out_dtype=torch.float32 if c["out"] == "f32" else torch.bfloat16)
    torch.cuda.synchronize()
    o_ref, S_ref, z_ref = O.causal_linear_attention(x.q, x.k, x.v, decay=x.decay, gate=x.gate,
                                                    S0=S0, z0=z0, normalize=c["normalize"])
    e = (_out_err(out, o_ref), rel_err(S, S_ref), rel_err(z, z_ref))
    print("errors", e)
    assert max(e) < TOL["bf16"], (c, e)


def _mlstm_cases(n, seed):
    r = random.Random(seed)
    for i in range(n):
        yield dict(i=i, B=r.choice([1, 2]), H=r.choice([1, 2, 3]),
                   T=r.choice([1, 33, 100, 257, r.randint(1, 700), r.randint(1, 700)]),
                   d=r.choice([64, 128]), chunk=r.choice([0, 32, 64]),
                   segments=r.choice([0, 1, 2, 3, 5]), fmean=r.choice([0.0, 3.0, 6.0]),
                   ishift=r.choice([0.0, 0.0, 4.0]), fexp=r.random() < 0.3,
                   state=r.random() < 0.4, seed=2000 + i)


@pytest.mark.parametrize("case", list(_mlstm_cases(16, 11)), ids=lambda c: f"m{c['i']}")
def test_mlstm_prefill_sweep(case):
    dev = gpu_device()
    c = case
    print(c, flush=True)
    x = I.prefill_inputs(c["B"], c["H"], c["T"], c["d"], dtype="bf16", seed=c["seed"],
                         decay="mlstm", decay_mean=c["fmean"], scale=2.0 ** -0.5)
    x.igate = x.igate + c["ishift"]
    if c["fexp"]:
        x.fgate = -torch.nn.functional.softplus(-x.fgate)   # log sigmoid: the exp form's input
    st = S0 = z0 = m0 = None
    if c["state"]:
        rng = np.random.default_rng(c["seed"])
        S0 = rng.standard_normal((c["B"], c["H"], c["d"], c["d"])) * 0.3
        z0 = rng.standard_normal((c["B"], c["H"], c["d"])) * 0.3
        m0 = rng.standard_normal((c["B"], c["H"]))
        st = tuple(torch.tensor(a, dtype=torch.float32, device=dev) for a in (S0, z0, m0))
        S0, z0, m0 = (t.cpu().double().numpy() for t in st)
    g = lambda t: None if t is None else t.to(dev)
    out, S, z, m = la.prefill(g(x.q), g(x.k), g(x.v), phi="identity", igate=g(x.igate),
                              fgate=g(x.fgate), fgate_exp=c["fexp"], normalize="max1",
                              state=st, chunk=c["chunk"], segments=c["segments"],
                              out_dtype=torch.float32)
    torch.cuda.synchronize()
    o_ref, S_ref, z_ref, m_ref = O.mlstm_recurrence(x.q, x.k, x.v, x.igate, x.fgate, c["fexp"],
                                                    1e-6, S0, z0, m0, "max1")
    e = (rel_err(out, o_ref), rel_err(S, S_ref), rel_err(z, z_ref),
         float(np.abs(m.cpu().double().numpy() - m_ref).max()))
    print("errors", e)
    assert max(e[:3]) < TOL["bf16"] and e[3] < 1e-3, (c, e)


def _backward_cases(n, seed):
    """With the sum read-out and no carried state the first token's output is
    v_0 itself up to eps, so dq_0 and dk_0 are O(eps): differences of O(1)
    terms that no fp32 arithmetic resolves.  In a long sequence they vanish
    against the other tokens' gradients; with a handful of tokens they are
    most of the rms, so short sequences of that kind carry a state."""
    r = random.Random(seed)
    for i in range(n):
        c = dict(i=i, B=r.choice([1, 2]), H=r.choice([1, 2, 3]),
                 T=r.choice([1, 32, 33, 95, 200, r.randint(1, 500), r.randint(1, 500)]),
                 d=r.choice([64, 128]), segments=r.choice([0, 1, 2, 3, 5]),
                 kind=r.choice([None, "ssd", "rfa"]), mean=r.choice([-1.0, 1.0, 3.0, 6.0]),
                 normalize=r.choice([True, True, False]), state=r.random() < 0.5,
                 seed=3000 + i)
        if c["normalize"] is True and c["T"] < 16:
            c["state"] = True
        yield c


@pytest.mark.parametrize("case", list(_backward_cases(16, 13)), ids=lambda c: f"b{c['i']}")
def test_backward_sweep(case):
    dev = gpu_device()
    c = case
    print(c, flush=True)
    B, H, T, d = c["B"], c["H"], c["T"], c["d"]
    x = I.prefill_inputs(B, H, T, d, dtype="bf16", seed=c["seed"], scale=2.0 ** -0.5)
    _decay(x, c["kind"], c["mean"], torch.Generator().manual_seed(c["seed"]))
    do = torch.randn(B, H, T, d, generator=torch.Generator().manual_seed(c["seed"] + 1))
    do = do.to(torch.bfloat16)
    st = S0 = z0 = None
    if c["state"]:
        rng = np.random.default_rng(c["seed"])
        S0 = rng.standard_normal((B, H, d, d)) * 0.3
        z0 = np.abs(rng.standard_normal((B, H, d))) * 0.3 + 0.5
        st = (torch.tensor(S0, dtype=torch.float32, device=dev),
              torch.tensor(z0, dtype=torch.float32, device=dev))
        S0, z0 = st[0].cpu().double().numpy(), st[1].cpu().double().numpy()
    g = lambda t: None if t is None else t.to(dev)
    got = la.prefill_backward(g(x.q), g(x.k), g(x.v), g(do), decay=g(x.decay), gate=g(x.gate),
                              state=st, normalize=c["normalize"], state_grad=True,
                              segments=c["segments"])
    torch.cuda.synchronize()
    ref = O.prefill_gradients_recurrent(x.q, x.k, x.v, do, decay=x.decay, gate=x.gate, S0=S0,
                                        z0=z0, normalize=c["normalize"])
    errs = {k: rel_err(got[k], ref[k]) for k in got}
    print("errors", errs)
    assert max(errs.values()) < TOL["bf16"], (c, errs)


def _decode_cases(n, seed):
    r = random.Random(seed)
    for i in range(n):
        phi = r.choice(["elu1", "elu1", "rff"])
        yield dict(i=i, N=r.choice([1, 3, 7, 33]), H=r.choice([1, 2, 4]),
                   dh=r.choice([16, 32, 64, 100, 128, 256]), dv=r.choice([16, 32, 64, 128]),
                   phi=phi, D=r.choice([16, 32, 64, 128]) if phi == "rff" else 0,
                   decay=r.choice([None, "ssd", "rfa"]), dtype=r.choice(["f32", "f32", "bf16"]),
                   steps=r.randint(2, 6), seed=4000 + i)


@pytest.mark.parametrize("case", list(_decode_cases(24, 17)), ids=lambda c: f"d{c['i']}")
def test_decode_sweep(case):
    """Decode steps from a zero state (the specialised kernels and the
    per-token one, by shape), output of every step and the final state."""
    dev = gpu_device()
    c = case
    print(c, flush=True)
    N, H, dh, dv, phi, D = c["N"], c["H"], c["dh"], c["dv"], c["phi"], c["D"]
    W = I.rff_projection(H, D, dh, seed=c["seed"]) if phi == "rff" else None
    dp = 2 * D if phi == "rff" else dh
    S, z = la.state_init(N, H, dp, dv, dev)
    S_ref, z_ref = np.zeros((N, H, dp, dv)), np.zeros((N, H, dp))
    sd = I.DTYPES[c["dtype"]]
    worst = 0.0
    for step in range(c["steps"]):
        st = I.rfa_decode_step_inputs(N, H, dh, dv, step=step, seed=c["seed"])
        q, k, v = st.q.to(sd), st.k.to(sd), st.v.to(sd)
        kw = {}
        if c["decay"] == "ssd":
            kw["decay"] = st.gate * 0.5 + 0.5
        elif c["decay"] == "rfa":
            kw["gate"] = st.gate
        o = la.decode_step(q.to(dev), k.to(dev), v.to(dev), S, z, phi=phi,
                           W=None if W is None else W.to(dev),
                           **{n: t.to(dev) for n, t in kw.items()}, out_dtype=torch.float32)
        torch.cuda.synchronize()
        o_ref, S_ref, z_ref = O.decode_step(q, k, v, S_ref, z_ref, phi=phi, W=W, **kw)
        worst = max(worst, rel_err(o, o_ref))
    e = (worst, rel_err(S, S_ref), rel_err(z, z_ref))
    print("errors", e)
    assert max(e) < TOL[c["dtype"]], (c, e)


def _mlstm_backward_cases(n, seed):
    """Gradients with the mLSTM gates, bf16 inputs (the chunked passes).  The
    sum read-out, and input gates shifted up (where the max1 floor e^{-m}
    falls far below |q.z|), take positive features and start states, which
    keep q.z away from 0; short sum read-out draws carry a state, as in the
    gradient sweep above."""
    r = random.Random(seed)
    for i in range(n):
        c = dict(i=i, B=r.choice([1, 2]), H=r.choice([1, 2, 3]),
                 T=r.choice([1, 31, 33, 96, 257, r.randint(1, 600), r.randint(1, 600)]),
                 d=r.choice([64, 128]), segments=r.choice([0, 1, 2, 3, 5]),
                 fmean=r.choice([0.0, 3.0, 6.0]), ishift=r.choice([0.0, 0.0, 3.0]),
                 fexp=r.random() < 0.3, normalize=r.choice(["max1", "max1", True, False]),
                 state=r.random() < 0.5, seed=5000 + i)
        if c["normalize"] is True and c["T"] < 16:
            c["state"] = True   # as in the gradient sweep above: the first tokens' O(eps) terms
        yield c


@pytest.mark.parametrize("case", list(_mlstm_backward_cases(16, 19)), ids=lambda c: f"mb{c['i']}")
def test_mlstm_backward_sweep(case):
    dev = gpu_device()
    c = case
    print(c, flush=True)
    B, H, T, d = c["B"], c["H"], c["T"], c["d"]
    positive = c["normalize"] is True or c["ishift"] > 0
    x = I.prefill_inputs(B, H, T, d, dtype="bf16", seed=c["seed"], decay="mlstm",
                         decay_mean=c["fmean"], scale=0.7)
    x.igate = x.igate + c["ishift"]
    if positive:
        x.q, x.k = x.q.abs(), x.k.abs()
    if c["fexp"]:
        x.fgate = -torch.nn.functional.softplus(-x.fgate)   # log sigmoid: the exp form's input
    do = torch.randn(B, H, T, d, generator=torch.Generator().manual_seed(c["seed"] + 1))
    do = do.to(torch.bfloat16)
    st = S0 = z0 = m0 = None
    if c["state"]:
        rng = np.random.default_rng(c["seed"])
        S0 = rng.standard_normal((B, H, d, d)) * 0.3
        z0 = rng.standard_normal((B, H, d)) * 0.3
        if positive:
            S0, z0 = np.abs(S0), np.abs(z0)
        m0 = c["ishift"] + rng.standard_normal((B, H))
        st = tuple(torch.tensor(a, dtype=torch.float32, device=dev) for a in (S0, z0, m0))
        S0, z0, m0 = (t.cpu().double().numpy() for t in st)
    g = lambda t: None if t is None else t.to(dev)
    got = la.prefill_backward(g(x.q), g(x.k), g(x.v), g(do), phi="identity", igate=g(x.igate),
                              fgate=g(x.fgate), fgate_exp=c["fexp"], state=st,
                              normalize=c["normalize"], state_grad=True, segments=c["segments"])
    torch.cuda.synchronize()
    ref = O.mlstm_gradients(x.q, x.k, x.v, do, x.igate, x.fgate, c["fexp"], 1e-6, S0, z0, m0,
                            c["normalize"])
    errs = {k: rel_err(got[k], ref[k]) for k in got}
    print("errors", errs)
    assert max(errs.values()) < TOL["bf16"], (c, errs)
