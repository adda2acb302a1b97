"""Pins for the oracle's prefill gradients: central finite differences of
L = sum_t <dout_t, o_t> through the forward oracle (the recurrence, a
different algorithm from the gradients' quadratic form), closed forms, and
planted mistakes.  CPU only, float64, tiny inputs.
"""
import numpy as np
import pytest

from oracle import linattn_oracle as O

H_FD = 1e-6


def loss(q, k, v, do, phi, decay, gate, S0, z0, normalize, eps=1e-6):
    o, _, _ = O.causal_linear_attention(q, k, v, phi=phi, decay=decay, gate=gate, eps=eps,
                                        S0=S0, z0=z0, normalize=normalize)
    return float((o * do).sum())


def fd(f, x):
    g = np.zeros_like(x)
    for i in np.ndindex(x.shape):
        xp, xm = x.copy(), x.copy()
        xp[i] += H_FD
        xm[i] -= H_FD
        g[i] = (f(xp) - f(xm)) / (2 * H_FD)
    return g


def case(seed, T=7, d=3, dv=2, kind="none", scale=1.0):
    rng = np.random.default_rng(seed)
    q, k = rng.standard_normal((T, d)) * scale, rng.standard_normal((T, d)) * scale
    v, do = rng.standard_normal((T, dv)), rng.standard_normal((T, dv))
    S0, z0 = rng.standard_normal((d, dv)) * 0.3, np.abs(rng.standard_normal(d)) * 0.3
    a = 1.0 / (1.0 + np.exp(-rng.standard_normal(T) - 1.0))
    decay = a if kind == "ssd" else None
    gate = a if kind == "rfa" else None
    return q, k, v, do, S0, z0, decay, gate


@pytest.mark.parametrize("phi", ["elu1", "identity"])
@pytest.mark.parametrize("kind", ["none", "ssd", "rfa"])
@pytest.mark.parametrize("normalize", [True, False, "max1"])
def test_gradients_match_finite_differences(phi, kind, normalize):
    q, k, v, do, S0, z0, decay, gate = case(3, kind=kind)
    if phi == "identity" and normalize is True:
        q, k = np.abs(q), np.abs(k)       # keep q.z away from 0 (signed features)
    g = O.prefill_gradients(q, k, v, do, phi=phi, decay=decay, gate=gate, S0=S0, z0=z0,
                            normalize=normalize)
    f = lambda **kw: loss(**{**dict(q=q, k=k, v=v, do=do, phi=phi, decay=decay, gate=gate,
                                    S0=S0, z0=z0, normalize=normalize), **kw})
    checks = [("dq", q, lambda x: f(q=x)), ("dk", k, lambda x: f(k=x)),
              ("dv", v, lambda x: f(v=x)), ("dS0", S0, lambda x: f(S0=x)),
              ("dz0", z0, lambda x: f(z0=x))]
    if decay is not None:
        checks.append(("ddecay", decay, lambda x: f(decay=x)))
    if gate is not None:
        checks.append(("dgate", gate, lambda x: f(gate=x)))
    for name, x, fn in checks:
        ref = fd(fn, x)
        np.testing.assert_allclose(g[name], ref, rtol=1e-6, atol=1e-7, err_msg=name)


def test_gradients_are_linear_in_dout():
    q, k, v, do, S0, z0, decay, _ = case(5, kind="ssd")
    do2 = np.random.default_rng(9).standard_normal(do.shape)
    g1 = O.prefill_gradients(q, k, v, do, decay=decay, S0=S0, z0=z0)
    g2 = O.prefill_gradients(q, k, v, do2, decay=decay, S0=S0, z0=z0)
    g12 = O.prefill_gradients(q, k, v, do + 2 * do2, decay=decay, S0=S0, z0=z0)
    for n in ("dq", "dk", "dv", "dS0", "dz0", "ddecay"):
        np.testing.assert_allclose(g12[n], g1[n] + 2 * g2[n], rtol=1e-10, atol=1e-12)


def test_unnormalised_closed_forms():
    # no normaliser, no decay: o_t = sum_{s<=t} (fq_t.fk_s) v_s + fq_t^T S0, so
    # dv_s = sum_{t>=s} (fq_t.fk_s) do_t and dS0 = sum_t fq_t do_t^T
    q, k, v, do, S0, z0, _, _ = case(7)
    g = O.prefill_gradients(q, k, v, do, S0=S0, z0=z0, normalize=False)
    fq, fk = O.phi_elu1(q), O.phi_elu1(k)
    T = q.shape[0]
    dv = np.zeros_like(v)
    for s in range(T):
        for t in range(s, T):
            dv[s] += float(fq[t] @ fk[s]) * do[t]
    np.testing.assert_allclose(g["dv"], dv, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(g["dS0"], fq.T @ do, rtol=1e-12, atol=1e-13)
    np.testing.assert_array_equal(g["dz0"], 0.0)


def test_single_token_closed_form():
    # T = 1, zero state: o = v (fq.fk) / ((fq.fk) + eps); with eps -> the
    # output is v whatever q and k, so dq, dk vanish up to O(eps), dv = do
    rng = np.random.default_rng(2)
    q, k = rng.standard_normal((1, 4)), rng.standard_normal((1, 4))
    v, do = rng.standard_normal((1, 3)), rng.standard_normal((1, 3))
    g = O.prefill_gradients(q, k, v, do, eps=0.0)
    np.testing.assert_allclose(g["dv"], do, rtol=1e-14)
    assert np.abs(g["dq"]).max() < 1e-12 and np.abs(g["dk"]).max() < 1e-12


def _mutant(q, k, v, do, decay, mistake):
    """A copy of the gradient with one plausible mistake (no decay, sum read-out)."""
    fq, fk = O.phi_elu1(q), O.phi_elu1(k)
    T = q.shape[0]
    M = np.tril(np.ones((T, T)))
    A = fq @ fk.T
    W = A * M
    num, den = W @ v, W.sum(1) + 1e-6
    o = num / den[:, None]
    g_num, g_den = do / den[:, None], -(do * o).sum(1) / den
    if mistake == "no_den_term":
        g_den = 0 * g_den
    dW = g_num @ v.T + g_den[:, None]
    dA = dW * M
    if mistake == "mask_transposed":
        dA = dW * M.T
    dfq = dA @ fk
    dq = dfq * O.phi_derivative(q)
    if mistake == "no_phi_derivative":
        dq = dfq
    return dq


@pytest.mark.parametrize("mistake", ["no_den_term", "mask_transposed", "no_phi_derivative"])
def test_planted_mistakes_fail_finite_differences(mistake):
    q, k, v, do, _, _, _, _ = case(11, scale=1.5)
    ref = fd(lambda x: loss(x, k, v, do, "elu1", None, None, None, None, True), q)
    assert np.abs(_mutant(q, k, v, do, None, mistake) - ref).max() > 1e-4
    assert np.abs(_mutant(q, k, v, do, None, None) - ref).max() < 1e-7


# ---------------------------------------------------------------------------
# The recurrent gradients (reverse mode through the state, for long
# sequences): finite differences directly, and the quadratic-form gradients
# on the same inputs.

@pytest.mark.parametrize("phi", ["elu1", "identity"])
@pytest.mark.parametrize("normalize", [True, False, "max1"])
def test_recurrent_gradients_match_finite_differences(phi, normalize):
    q, k, v, do, S0, z0, _, _ = case(11)
    if phi == "identity" and normalize is True:
        q, k = np.abs(q), np.abs(k)
    g = O.prefill_gradients_recurrent(q, k, v, do, phi=phi, S0=S0, z0=z0, normalize=normalize)
    f = lambda **kw: loss(**{**dict(q=q, k=k, v=v, do=do, phi=phi, decay=None, gate=None,
                                    S0=S0, z0=z0, normalize=normalize), **kw})
    for name, x, fn in [("dq", q, lambda x: f(q=x)), ("dk", k, lambda x: f(k=x)),
                        ("dv", v, lambda x: f(v=x)), ("dS0", S0, lambda x: f(S0=x)),
                        ("dz0", z0, lambda x: f(z0=x))]:
        ref = fd(fn, x)
        assert np.abs(g[name] - ref).max() <= 1e-6 * max(1.0, np.abs(ref).max()), name


@pytest.mark.parametrize("normalize", [True, False, "max1"])
@pytest.mark.parametrize("kind", ["none", "ssd", "rfa"])
@pytest.mark.parametrize("T", [50, 150])    # one checkpoint block of the walk back, three
def test_recurrent_gradients_equal_quadratic_form(normalize, kind, T):
    rng = np.random.default_rng(5)
    B, H, d, dv = 2, 2, 5, 3
    q, k = rng.standard_normal((B, H, T, d)), rng.standard_normal((B, H, T, d))
    v, do = rng.standard_normal((B, H, T, dv)), rng.standard_normal((B, H, T, dv))
    S0, z0 = rng.standard_normal((B, H, d, dv)) * 0.3, np.abs(rng.standard_normal((B, H, d)))
    a_ = 1.0 / (1.0 + np.exp(-rng.standard_normal((B, H, T)) - 1.0))
    decay = a_ if kind == "ssd" else None
    gate = a_ if kind == "rfa" else None
    a = O.prefill_gradients(q, k, v, do, decay=decay, gate=gate, S0=S0, z0=z0, normalize=normalize)
    b = O.prefill_gradients_recurrent(q, k, v, do, decay=decay, gate=gate, S0=S0, z0=z0,
                                      normalize=normalize)
    assert set(a) == set(b)
    for n in b:
        assert np.abs(a[n] - b[n]).max() <= 1e-11 * np.abs(a[n]).max(), n


@pytest.mark.parametrize("kind", ["ssd", "rfa"])
def test_recurrent_decay_gradient_matches_finite_differences(kind):
    q, k, v, do, S0, z0, decay, gate = case(12, kind=kind)
    g = O.prefill_gradients_recurrent(q, k, v, do, decay=decay, gate=gate, S0=S0, z0=z0)
    f = lambda **kw: loss(**{**dict(q=q, k=k, v=v, do=do, phi="elu1", decay=decay, gate=gate,
                                    S0=S0, z0=z0, normalize=True), **kw})
    if kind == "ssd":
        name, x, fn = "ddecay", decay, lambda x: f(decay=x)
    else:
        name, x, fn = "dgate", gate, lambda x: f(gate=x)
    ref = fd(fn, x)
    assert np.abs(g[name] - ref).max() <= 1e-6 * max(1.0, np.abs(ref).max()), name


def test_recurrent_gradients_planted_mistake_is_caught():
    # the gradient state gathered after the read-out of token t instead of
    # before it (G missing phi(q_t) g_t^T at t) must fail the quadratic form
    rng = np.random.default_rng(6)
    T, d = 20, 4
    q, k, v, do = (rng.standard_normal((T, d)) for _ in range(4))
    ref = O.prefill_gradients(q, k, v, do)
    fq, fk = O.features(q), O.features(k)
    g = O.prefill_gradients_recurrent(q, k, v, do)
    # rebuild dk with the shifted accumulation from the oracle's own g, h
    o, _, _ = O.causal_linear_attention(q, k, v)
    z = np.cumsum(fk, axis=0)
    Dv = (fq * z).sum(1) + 1e-6
    gg = do / Dv[:, None]
    h = -(do * o).sum(1) / Dv
    G, gz, dfk = np.zeros((d, d)), np.zeros(d), np.zeros((T, d))
    for t in range(T - 1, -1, -1):
        dfk[t] = G @ v[t] + gz
        G += np.outer(fq[t], gg[t])
        gz += fq[t] * h[t]
    wrong = dfk * O.phi_derivative(k)
    assert np.abs(g["dk"] - ref["dk"]).max() < 1e-12 * np.abs(ref["dk"]).max()
    assert np.abs(wrong - ref["dk"]).max() > 1e-3 * np.abs(ref["dk"]).max()


# ---------------------------------------------------------------------------
# A decay or gate of exactly 0 is a full reset of the state.  L is a
# polynomial in each alpha_r over the denominators, smooth through 0, so its
# gradient there is finite and central differences around 0 pin it.  Both
# gradient oracles take it as a product over the other decays (no division).

def _zero_case(seed, kind, zeros, T=9):
    q, k, v, do, S0, z0, decay, gate = case(seed, T=T, kind=kind)
    a = decay if kind == "ssd" else gate
    a[list(zeros)] = 0.0
    return q, k, v, do, S0, z0, decay, gate


@pytest.mark.parametrize("fn", ["quadratic", "recurrent"])
@pytest.mark.parametrize("kind", ["ssd", "rfa"])
@pytest.mark.parametrize("zeros", [(0,), (4,), (8,), (2, 3, 6)])
def test_decay_gradient_at_zero_matches_finite_differences(fn, kind, zeros):
    q, k, v, do, S0, z0, decay, gate = _zero_case(21, kind, zeros)
    grad = O.prefill_gradients if fn == "quadratic" else O.prefill_gradients_recurrent
    with np.errstate(all="raise"):          # no division by the zero decay anywhere
        g = grad(q, k, v, do, decay=decay, gate=gate, S0=S0, z0=z0)
    name = "ddecay" if kind == "ssd" else "dgate"
    f = lambda x: loss(q, k, v, do, "elu1", x if kind == "ssd" else None,
                       x if kind == "rfa" else None, S0, z0, True)
    ref = fd(f, decay if kind == "ssd" else gate)
    assert np.all(np.isfinite(g[name]))
    np.testing.assert_allclose(g[name], ref, rtol=1e-6, atol=1e-7, err_msg=name)
    # the other gradients stay those of the reset sequence
    for other, x, fo in (("dq", q, lambda x: loss(x, k, v, do, "elu1", decay, gate, S0, z0, True)),
                         ("dS0", S0, lambda x: loss(q, k, v, do, "elu1", decay, gate, x, z0, True))):
        np.testing.assert_allclose(g[other], fd(fo, x), rtol=1e-6, atol=1e-7, err_msg=other)


def test_decay_gradient_at_zero_is_the_state_product():
    # With alpha_r = 0 nothing before r reaches the loss, yet dL/dalpha_r is
    # the inner product of the gradient state after r with the state before
    # r: here both are written out from their definitions, so a gradient
    # that returned 0 (or dropped either state's start term) would fail.
    rng = np.random.default_rng(31)
    T, d, dv, r = 8, 3, 2, 5
    q, k = rng.standard_normal((T, d)), rng.standard_normal((T, d))
    v, do = rng.standard_normal((T, dv)), rng.standard_normal((T, dv))
    S0, z0 = rng.standard_normal((d, dv)) * 0.3, np.abs(rng.standard_normal(d))
    a = 1.0 / (1.0 + np.exp(-rng.standard_normal(T)))
    a[r] = 0.0
    fq, fk = O.phi_elu1(q), O.phi_elu1(k)
    o, _, _ = O.causal_linear_attention(q, k, v, decay=a, S0=S0, z0=z0)
    # S_{r-1}, z_{r-1} by the plain sums
    Sm = np.prod(a[:r]) * S0 + sum(np.prod(a[s + 1:r]) * np.outer(fk[s], v[s]) for s in range(r))
    zm = np.prod(a[:r]) * z0 + sum(np.prod(a[s + 1:r]) * fk[s] for s in range(r))
    # G_r, gz_r: the read-outs at t >= r, through the state after r
    Sr = np.zeros((d, dv)) + np.outer(fk[r], v[r])   # alpha_r = 0
    zr = fk[r].copy()
    G, gz = np.zeros((d, dv)), np.zeros(d)
    for t in range(r, T):
        if t > r:
            Sr = a[t] * Sr + np.outer(fk[t], v[t])
            zr = a[t] * zr + fk[t]
        D = fq[t] @ zr + 1e-6
        w = np.prod(a[r + 1:t + 1])
        G += w * np.outer(fq[t], do[t] / D)
        gz += w * fq[t] * (-(do[t] @ o[t]) / D)
    expect = (G * Sm).sum() + gz @ zm
    for grad in (O.prefill_gradients, O.prefill_gradients_recurrent):
        got = grad(q, k, v, do, decay=a, S0=S0, z0=z0)["ddecay"][r]
        assert abs(got - expect) <= 1e-12 * max(1.0, abs(expect)), (grad.__name__, got, expect)
    assert abs(expect) > 1e-3
