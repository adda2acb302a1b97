"""Pins for the oracle's mLSTM functions (wikillm "Linear attention",
Variants / "Matrix memory with exponential gates (mLSTM)"): the literal
recurrence against a pure-Python double loop and closed forms, the stabilised
recurrence against the literal one, the stabiliser against its max-plus
unrolling, and planted mistakes that these pins must catch.  CPU only.
"""
import math

import numpy as np
import pytest

from oracle import linattn_oracle as O

RNG = np.random.default_rng(4321)


def rand(*shape, rng=RNG):
    return rng.standard_normal(shape)


def sigmoid(x):
    return 1.0 / (1.0 + np.exp(-np.asarray(x, dtype=np.float64)))


def gates(shape, rng=RNG, imean=0.0, fmean=3.0):
    return rng.standard_normal(shape) + imean, rng.standard_normal(shape) + fmean


# ------------------------------------------------------------ gates, read-out

def test_log_forget_closed_forms():
    # (log(sigmoid(x)) taken literally loses digits for large x: moderate x here)
    x = np.array([-40.0, -3.0, 0.0, 0.5, 3.0, 8.0])
    np.testing.assert_allclose(O.log_forget(x), np.log(sigmoid(x)), rtol=1e-11, atol=0)
    assert O.log_forget(np.array([0.0]))[0] == pytest.approx(math.log(0.5), abs=1e-15)
    # far in the saturated tails: log sigmoid(x) ~ -e^{-x} and ~ x
    assert O.log_forget(np.array([60.0]))[0] == pytest.approx(-math.exp(-60.0), rel=1e-12)
    assert O.log_forget(np.array([-800.0]))[0] == pytest.approx(-800.0, rel=1e-15)
    np.testing.assert_array_equal(O.log_forget(x, exp_form=True), x)


def test_max1_readout_closed_forms():
    num = np.array([[2.0, -4.0], [2.0, -4.0], [2.0, -4.0], [2.0, -4.0]])
    den = np.array([0.5, -0.5, 4.0, -4.0])
    got = O.readout(num, den, normalize="max1")
    # |den| < 1: the numerator itself; |den| >= 1: divided by |den| (sign kept)
    np.testing.assert_array_equal(got, [[2.0, -4.0], [2.0, -4.0], [0.5, -1.0], [0.5, -1.0]])


def test_single_token_closed_form():
    # T = 1 from a zero state: o = (q.k) e^{itilde} v / max(|q.k| e^{itilde}, 1)
    for it, ft in ((0.3, 2.0), (-4.0, -1.0), (2.5, 0.0)):
        q, k, v = rand(1, 5), rand(1, 5), rand(1, 3)
        o, S, z, m = O.mlstm_recurrence(q, k, v, np.array([it]), np.array([ft]))
        s = float(q[0] @ k[0]) * math.exp(it)
        np.testing.assert_allclose(o[0], s * v[0] / max(abs(s), 1.0), rtol=1e-13)
        # the stabiliser of a zero state (m = 0) after one token
        assert m == pytest.approx(max(math.log(sigmoid(ft)), it), abs=1e-15)


# ------------------------------------------- literal recurrence vs definition

@pytest.mark.parametrize("exp_form", [False, True])
@pytest.mark.parametrize("normalize", ["max1", True, False])
@pytest.mark.parametrize("T,d,dv", [(1, 3, 2), (6, 4, 3), (11, 3, 5)])
def test_definition_equals_bruteforce(exp_form, normalize, T, d, dv):
    q, k, v = rand(T, d), rand(T, d), rand(T, dv)
    it, ft = gates((T,), fmean=0.0 if exp_form else 3.0)
    f = np.exp(ft) if exp_form else sigmoid(ft)
    o, _, _ = O.mlstm_by_definition(q, k, v, it, ft, exp_form, normalize=normalize)
    ref = O.kernel_attention_by_definition(q, k, v, alpha=f, beta=np.exp(it), normalize=normalize)
    np.testing.assert_allclose(o, ref, rtol=1e-11, atol=1e-12)


def test_unit_gates_are_plain_identity_attention():
    # f = e^0 = 1 and i = e^0 = 1: plain causal attention with identity
    # features and the max1 read-out; the stabiliser stays at 0
    q, k, v = rand(2, 20, 6), rand(2, 20, 6), rand(2, 20, 4)
    zero = np.zeros((2, 20))
    o, _, _, m = O.mlstm_recurrence(q, k, v, zero, zero, exp_form=True)
    np.testing.assert_allclose(o, O.masked_quadratic(q, k, v, normalize="max1"),
                               rtol=1e-11, atol=1e-12)
    np.testing.assert_array_equal(m, 0.0)


# --------------------------------------------- stabilised vs literal recurrence

@pytest.mark.parametrize("exp_form", [False, True])
@pytest.mark.parametrize("normalize", ["max1", True, False])
def test_stabilised_equals_literal(exp_form, normalize):
    T, d, dv = 40, 6, 5
    q, k, v = rand(3, T, d), rand(3, T, d), rand(3, T, dv)
    it, ft = gates((3, T), imean=1.0, fmean=0.0 if exp_form else 2.0)
    if exp_form:
        ft = -np.abs(ft) * 0.2     # f = e^{ft} <= 1 keeps the literal state moderate
    S0, z0 = rand(3, d, dv), rand(3, d)
    o_def, S_def, z_def = O.mlstm_by_definition(q, k, v, it, ft, exp_form, S0=S0, z0=z0,
                                                normalize=normalize)
    o, S, z, m = O.mlstm_recurrence(q, k, v, it, ft, exp_form, S0=S0, z0=z0,
                                    m0=np.zeros(3), normalize=normalize)
    np.testing.assert_allclose(o, o_def, rtol=1e-10, atol=1e-11)
    np.testing.assert_allclose(np.exp(m)[:, None, None] * S, S_def, rtol=1e-10, atol=1e-11)
    np.testing.assert_allclose(np.exp(m)[:, None] * z, z_def, rtol=1e-10, atol=1e-11)


def test_stabilised_survives_input_gates_beyond_overflow():
    # i = e^{1000 + x} overflows float64; the quotient does not depend on a
    # common factor of all weights once |den| >= 1, so the stabilised
    # outputs must equal num / |den| of the unshifted weights
    T, d, dv = 30, 5, 4
    q, k, v = rand(T, d), rand(T, d), rand(T, dv)
    it, ft = gates((T,))
    o, S, z, m = O.mlstm_recurrence(q, k, v, it + 1000.0, ft)
    assert np.isfinite(o).all() and np.isfinite(S).all() and 999 < m < 1010
    f, i = sigmoid(ft), np.exp(it)
    w = (q @ k.T) * np.tril(np.ones((T, T)))
    for t in range(T):
        for s in range(t + 1):
            w[t, s] *= i[s] * np.prod(f[s + 1: t + 1])
    ref = (w @ v) / np.abs(w.sum(-1))[:, None]
    np.testing.assert_allclose(o, ref, rtol=1e-9, atol=1e-12)


def test_stabiliser_is_its_max_plus_unrolling():
    # m_T = max(m0 + sum_r log f_r, max_s (itilde_s + sum_{r > s} log f_r)),
    # enumerated term by term
    T = 25
    for exp_form in (False, True):
        it, ft = gates((T,), imean=-1.0, fmean=1.0)
        lf = np.log(np.exp(ft)) if exp_form else np.log(sigmoid(ft))
        m0 = 0.7
        terms = [m0 + lf.sum()] + [it[s] + lf[s + 1:].sum() for s in range(T)]
        _, _, _, m = O.mlstm_recurrence(rand(T, 3), rand(T, 3), rand(T, 2), it, ft, exp_form,
                                        S0=np.zeros((3, 2)), z0=np.zeros(3), m0=np.array(m0))
        assert float(m) == pytest.approx(max(terms), abs=1e-12)


def test_final_state_closed_form_matches_recurrence():
    T, d, dv = 37, 4, 6
    k, v = rand(2, T, d), rand(2, T, dv)
    it, ft = gates((2, T))
    S0, z0, m0 = rand(2, d, dv), rand(2, d), np.array([0.5, -2.0])
    _, S, z, m = O.mlstm_recurrence(rand(2, T, d), k, v, it, ft, S0=S0, z0=z0, m0=m0)
    Sc, zc, mc = O.mlstm_final_state(k, v, it, ft, S0=S0, z0=z0, m0=m0)
    np.testing.assert_allclose(mc, m, rtol=0, atol=1e-12)
    np.testing.assert_allclose(Sc, S, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(zc, z, rtol=1e-10, atol=1e-12)


def test_start_scale_does_not_change_outputs():
    # (S0 e^{-c}, z0 e^{-c}, m0 + c) is the same state as (S0, z0, m0)
    T, d, dv = 15, 4, 3
    q, k, v = rand(T, d), rand(T, d), rand(T, dv)
    it, ft = gates((T,))
    S0, z0 = rand(d, dv), rand(d)
    for normalize in ("max1", True, False):
        a = O.mlstm_recurrence(q, k, v, it, ft, S0=S0, z0=z0, m0=np.array(0.0), normalize=normalize)
        c = 7.5
        b = O.mlstm_recurrence(q, k, v, it, ft, S0=S0 * math.exp(-c), z0=z0 * math.exp(-c),
                               m0=np.array(c), normalize=normalize)
        np.testing.assert_allclose(b[0], a[0], rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(np.exp(b[3]) * b[1], np.exp(a[3]) * a[1], rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("normalize", ["max1", True, False])
def test_output_at_matches_recurrence(normalize):
    T, d, dv = 50, 5, 4
    q, k, v = rand(2, T, d), rand(2, T, d), rand(2, T, dv)
    it, ft = gates((2, T))
    S0, z0, m0 = rand(2, d, dv), rand(2, d), np.array([1.0, -3.0])
    o, _, _, _ = O.mlstm_recurrence(q, k, v, it, ft, S0=S0, z0=z0, m0=m0, normalize=normalize)
    for t in (0, 1, 17, T - 1):
        got = O.mlstm_output_at(q[:, t], k, v, t, it, ft, S0=S0, z0=z0, m0=m0,
                                normalize=normalize)
        np.testing.assert_allclose(got, o[:, t], rtol=1e-10, atol=1e-12)


def test_continuation_is_bitwise():
    T, T1, d, dv = 30, 13, 4, 4
    q, k, v = rand(T, d), rand(T, d), rand(T, dv)
    it, ft = gates((T,))
    o, S, z, m = O.mlstm_recurrence(q, k, v, it, ft)
    o1, S1, z1, m1 = O.mlstm_recurrence(q[:T1], k[:T1], v[:T1], it[:T1], ft[:T1])
    o2, S2, z2, m2 = O.mlstm_recurrence(q[T1:], k[T1:], v[T1:], it[T1:], ft[T1:], S0=S1, z0=z1,
                                        m0=m1)
    np.testing.assert_array_equal(np.concatenate([o1, o2]), o)
    np.testing.assert_array_equal(S2, S)
    np.testing.assert_array_equal(m2, m)


# --------------------------------------------------- planted mistakes caught

def _stab_loop(q, k, v, it, ft, mistake):
    T, d = q.shape
    S = np.zeros((d, v.shape[1])); z = np.zeros(d); m = 0.0; out = []
    lf = np.log(sigmoid(ft))
    for t in range(T):
        m_new = max(lf[t] + m, it[t])
        fs = math.exp(lf[t] + m - m_new)
        is_ = math.exp(it[t] - m_new)
        if mistake == "forget_uses_new_m":
            fs = math.exp(lf[t] + m_new - m_new)
        if mistake == "input_not_exponential":
            is_ = it[t] * math.exp(-m_new)
        if mistake == "other_stabiliser":
            # a different but consistent stabiliser: the same outputs
            m_new = max(m, it[t]); fs = math.exp(lf[t] + m - m_new); is_ = math.exp(it[t] - m_new)
        if mistake == "normaliser_not_forgotten":
            z = z * math.exp(m - m_new) / fs
        S = fs * S + is_ * np.outer(k[t], v[t]); z = fs * z + is_ * k[t]
        if mistake == "m_not_carried":
            m_keep = m
        m = m_new
        num, den = q[t] @ S, q[t] @ z
        floor = math.exp(-m)
        if mistake == "m_not_carried":
            m = m_keep
        if mistake == "floor_not_rescaled":
            floor = 1.0
        if mistake == "no_abs":
            out.append(num / max(den, floor))
            continue
        out.append(num / max(abs(den), floor))
    return np.array(out)


def test_any_consistent_stabiliser_gives_the_same_outputs():
    rng = np.random.default_rng(12)
    T, d, dv = 24, 4, 3
    q, k, v = (rng.standard_normal((T, d)), rng.standard_normal((T, d)),
               rng.standard_normal((T, dv)))
    it, ft = rng.standard_normal(T) + 1.5, rng.standard_normal(T) + 1.0
    np.testing.assert_allclose(_stab_loop(q, k, v, it, ft, "other_stabiliser"),
                               O.mlstm_recurrence(q, k, v, it, ft)[0], rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("mistake", ["forget_uses_new_m", "input_not_exponential",
                                     "normaliser_not_forgotten", "m_not_carried",
                                     "floor_not_rescaled", "no_abs"])
def test_planted_mistakes_fail_the_definition_pin(mistake):
    rng = np.random.default_rng(11)
    T, d, dv = 24, 4, 3
    q, k, v = (rng.standard_normal((T, d)), rng.standard_normal((T, d)),
               rng.standard_normal((T, dv)))
    it, ft = rng.standard_normal(T) + 1.5, rng.standard_normal(T) + 1.0
    ref = O.kernel_attention_by_definition(q, k, v, alpha=sigmoid(ft), beta=np.exp(it),
                                           normalize="max1")
    got = _stab_loop(q, k, v, it, ft, mistake)
    assert np.abs(got - ref).max() > 1e-6
    # the same loop without a mistake, and the oracle, pass the same check
    assert np.abs(_stab_loop(q, k, v, it, ft, None) - ref).max() < 1e-10
    assert np.abs(O.mlstm_recurrence(q, k, v, it, ft)[0] - ref).max() < 1e-10
