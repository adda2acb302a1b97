"""Pins of the oracle's mLSTM gradients (oracle.mlstm_gradients) to facts
other than itself (CPU):

* central finite differences of L = sum_t <dout_t, o_t>, with o from the
  stabilised forward oracle (mlstm_recurrence, pinned in
  test_oracle_mlstm_pins.py), for every input: q, k, v, both gate
  pre-activations, and the scaled start state (S0', z0', m0); every read-out,
  both forget-gate forms, input gates shifted far up (where the stabiliser
  carries the state);
* with input pre-activations of 0 and the sigmoid forget gate the recurrence
  is the SSD decay a = sigmoid(fgate) with identity features, whose
  gradients the generic oracle gives (pinned in test_oracle_backward_pins.py):
  dq, dk, dv equal, and dL/dfgate = dL/da a (1 - a).
"""
import numpy as np
import pytest

from oracle import linattn_oracle as O


def _inputs(seed, T=7, d=3, dv=2, ishift=0.0, fmean=1.0, state=True):
    g = np.random.default_rng(seed)
    x = dict(q=g.standard_normal((2, T, d)), k=g.standard_normal((2, T, d)),
             v=g.standard_normal((2, T, dv)), dout=g.standard_normal((2, T, dv)),
             igate=g.standard_normal((2, T)) + ishift, fgate=g.standard_normal((2, T)) + fmean)
    if state:
        x.update(S0=g.standard_normal((2, d, dv)) * 0.5, z0=g.standard_normal((2, d)) * 0.5,
                 m0=g.standard_normal(2))
    return x


def _loss(x, exp_form, normalize):
    o = O.mlstm_recurrence(x["q"], x["k"], x["v"], x["igate"], x["fgate"], exp_form, 1e-6,
                           x.get("S0"), x.get("z0"), x.get("m0"), normalize)[0]
    return float((o * x["dout"]).sum())


def _fd(x, name, exp_form, normalize, h=1e-6):
    base = x[name]
    out = np.zeros_like(base)
    for i in np.ndindex(*base.shape):
        xp = dict(x); xm = dict(x)
        bp = base.copy(); bp[i] += h
        bm = base.copy(); bm[i] -= h
        xp[name], xm[name] = bp, bm
        out[i] = (_loss(xp, exp_form, normalize) - _loss(xm, exp_form, normalize)) / (2 * h)
    return out


KEYS = {"q": "dq", "k": "dk", "v": "dv", "igate": "digate", "fgate": "dfgate", "S0": "dS0",
        "z0": "dz0", "m0": "dm0"}


@pytest.mark.parametrize("exp_form", [False, True])
@pytest.mark.parametrize("normalize", ["max1", True, False])
@pytest.mark.parametrize("ishift,state", [(0.0, True), (0.0, False), (25.0, True)])
def test_mlstm_gradients_match_finite_differences(exp_form, normalize, ishift, state):
    x = _inputs(3 + int(exp_form) + 7 * int(ishift), ishift=ishift, state=state,
                fmean=-0.5 if exp_form else 1.0)
    if normalize is True:
        # the sum read-out has no floor: positive q and k keep q.z away from 0
        x["q"], x["k"] = np.abs(x["q"]), np.abs(x["k"])
        if state:
            x["z0"] = np.abs(x["z0"])
    got = O.mlstm_gradients(x["q"], x["k"], x["v"], x["dout"], x["igate"], x["fgate"], exp_form,
                            1e-6, x.get("S0"), x.get("z0"), x.get("m0"), normalize)
    refs = {name: _fd(x, name, exp_form, normalize) for name in KEYS if name in x}
    # bound: 2e-5 of the gradient's largest element, plus the differences'
    # own resolution (fp64 rounding of L over the step h, with margin), which
    # is what is left of a gradient as small as the start state's once input
    # gates of e^25 swamp it
    noise = 100 * np.finfo(np.float64).eps * max(1.0, abs(_loss(x, exp_form, normalize))) / 1e-6
    for name, ref in refs.items():
        err = np.abs(got[KEYS[name]] - ref).max()
        assert err < 2e-5 * np.abs(ref).max() + noise, (name, err, np.abs(ref).max())


def test_mlstm_gradients_with_unit_input_gates_are_the_ssd_decay_gradients():
    x = _inputs(11, T=40, d=4, dv=3, state=False)
    x["igate"] = np.zeros_like(x["igate"])
    a = 1.0 / (1.0 + np.exp(-x["fgate"]))
    for normalize in ("max1", True, False):
        q, k = (np.abs(x["q"]), np.abs(x["k"])) if normalize is True else (x["q"], x["k"])
        got = O.mlstm_gradients(q, k, x["v"], x["dout"], x["igate"], x["fgate"], False, 1e-6,
                                normalize=normalize)
        ref = O.prefill_gradients_recurrent(q, k, x["v"], x["dout"], phi="identity", decay=a,
                                            normalize=normalize)
        for key in ("dq", "dk", "dv"):
            np.testing.assert_allclose(got[key], ref[key], rtol=1e-9, atol=1e-9 * np.abs(ref[key]).max())
        np.testing.assert_allclose(got["dfgate"], ref["ddecay"] * a * (1 - a), rtol=1e-8,
                                   atol=1e-9 * np.abs(ref["ddecay"]).max())


def test_planted_mistake_is_caught():
    """A gate gradient without the chain rule through the sigmoid (dL/dlog f
    reported as dL/dfgate) fails the finite differences."""
    x = _inputs(5, state=False)
    got = O.mlstm_gradients(x["q"], x["k"], x["v"], x["dout"], x["igate"], x["fgate"], False,
                            1e-6, normalize="max1")
    f = 1.0 / (1.0 + np.exp(-x["fgate"]))
    wrong = got["dfgate"] / (1.0 - f)
    ref = _fd(x, "fgate", False, "max1")
    assert np.abs(got["dfgate"] - ref).max() < 1e-5 * np.abs(ref).max()
    assert np.abs(wrong - ref).max() > 1e-2 * np.abs(ref).max()
