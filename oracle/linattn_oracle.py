"""fp64 CPU oracle for causal linear attention.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, calls or
links this module: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the
HIP library and never imports it.

Everything is plain numpy in float64.  Inputs are taken exactly as the GPU
path receives them (bf16/fp16/fp32 values) and upcast to float64 here.

Sources (the three pages the method is described on):

* [kb]     llm-arch-kb "Linear Attention", section 2 "Derivation" (causal
           recurrence, symbol legend, compute cost) and section 3 "Reference
           implementation" (non-causal and causal sketches).
* [lesson] efficient-attention lesson "Linear attention": Researcher level,
           "Derivation" (the general sim-attention sum, its factorised form,
           the recurrence for S_i and z_i, and the read-out); Developer level,
           "The regrouping, and the recurrence it implies" (bracketings,
           masked-quadratic check, eps = 1e-6 in the divisor) and "Try it
           yourself" (constant decay and its weighted quadratic form).
* [card]   wikillm "Linear attention": "Implementation sketch" (scalar decay
           applied to the old state and normaliser; current term undecayed),
           "Variants / Random Fourier features (RFA)" (Gaussian random
           projections, sigmoid gate that decays the old state and scales the
           new term by one minus the gate), "Decaying linear attention with a
           scalar state (SSD)" (decay 1 is the plain causal case),
           "Variants / Matrix memory with exponential gates (mLSTM)" (matrix
           memory and normaliser with a forget and an exponential input gate,
           a read-out divided by max(|n^T q|, 1), a stabiliser state against
           overflow) and, in "Implementation sketch", the remark that the
           mLSTM step is this loop with the identity feature map.

Every function is pinned by ``tests/test_oracle_pins.py``,
``tests/test_oracle_mlstm_pins.py`` and (the gradients)
``tests/test_oracle_backward_pins.py`` and
``tests/test_oracle_mlstm_backward_pins.py`` against facts the pages or the
mathematics fix (closed forms, brute force, printed values, central finite
differences of the forward definition).

Layout convention: ``[..., T, d]`` with any leading dims (batch, head);
decay/gate arrays are ``[..., T]``.  Feature dimension ``d'`` is ``d_h`` for
elu+1 and the identity map, and ``2 * D`` for random Fourier features.
"""
from __future__ import annotations

import numpy as np

F64 = np.float64


def _f64(x):
    """Upcast a numpy array or torch tensor (any float dtype) to float64."""
    if x is None:
        return None
    if hasattr(x, "detach"):  # torch tensor: bf16 has no numpy dtype
        x = x.detach().cpu().double().numpy()
    return np.asarray(x, dtype=F64)


# --------------------------------------------------------------------------
# Feature maps
# --------------------------------------------------------------------------

def phi_elu1(x):
    """elu(x) + 1 with alpha = 1, element-wise, so d' = d_h.

    [kb] section 2, symbol legend (phi(x) = elu(x) + 1, d' = d_h in the
    paper's experiments); [lesson] Developer level (PyTorch's elu default).
    elu(x) = x for x > 0 and exp(x) - 1 otherwise, hence phi = x + 1 or exp(x).
    """
    x = _f64(x)
    return np.where(x > 0, x + 1.0, np.exp(np.minimum(x, 0.0)))


def phi_rff(x, W):
    """Random Fourier features: D^{-1/2} [sin(W x); cos(W x)].

    [card] Variants / RFA: Gaussian random projections whose feature inner
    products estimate a Gaussian kernel.  ``x``: [..., H, T, d_h];
    ``W``: [H, D, d_h] (one projection per head).  Output: [..., H, T, 2D],
    sines first, then cosines.  No bias/phase term, sigma = 1.
    """
    x = _f64(x)
    W = _f64(W)
    D = W.shape[-2]
    proj = np.einsum("...htd,hjd->...htj", x, W)
    return np.concatenate([np.sin(proj), np.cos(proj)], axis=-1) / np.sqrt(D)


def phi_identity(x):
    """The identity feature map of the mLSTM step ([card] Implementation
    sketch: mLSTM fits the loop with the identity as its feature map)."""
    return _f64(x).copy()


def features(x, phi="elu1", W=None):
    if phi == "elu1":
        return phi_elu1(x)
    if phi == "identity":
        return phi_identity(x)
    if phi == "rff":
        if W is None:
            raise ValueError("rff feature map needs W")
        return phi_rff(x, W)
    raise ValueError(f"unknown feature map {phi!r}")


def decay_coefficients(decay=None, gate=None):
    """Per-token (alpha, beta) of S_t = alpha_t S_{t-1} + beta_t phi(k_t) v_t^T.

    * no decay: alpha = beta = 1 (returned as None, i.e. no multiply at all);
    * SSD scalar decay a_t: alpha = a_t, beta = 1 ([card] Implementation
      sketch: the decay multiplies the old state and the old normaliser);
    * RFA gate g_t: alpha = g_t, beta = 1 - g_t ([card] Variants / RFA and
      Implementation sketch: the gate decays the old state and scales the
      new term by one minus the gate).
    """
    if decay is not None and gate is not None:
        raise ValueError("decay and gate are exclusive")
    if decay is not None:
        return _f64(decay), None
    if gate is not None:
        g = _f64(gate)
        return g, 1.0 - g
    return None, None


def readout(num, den, eps=1e-6, normalize=True):
    """The read-out from the numerator phi(q)^T S and the denominator
    phi(q)^T z:
      normalize=True  -- num / (den + eps) ([kb] section 3 sketch);
      normalize=False -- num alone, the normaliser-free form ([card] SSD);
      "max1"          -- num / max(|den|, 1) ([card] mLSTM read-out).
    num: [..., d_v]; den: [...]."""
    num, den = _f64(num), _f64(den)
    if normalize is True:
        return num / (den + eps)[..., None]
    if normalize is False:
        return num
    if normalize == "max1":
        return num / np.maximum(np.abs(den), 1.0)[..., None]
    raise ValueError(f"unknown read-out {normalize!r}")


def _readout_scalar(num, den, eps, normalize):
    if normalize is True:
        return num / (den + eps)
    if normalize is False:
        return num
    if normalize == "max1":
        return num / max(abs(den), 1.0)
    raise ValueError(f"unknown read-out {normalize!r}")


# --------------------------------------------------------------------------
# The recurrence (the method's algorithm)
# --------------------------------------------------------------------------

def recurrence(fq, fk, v, alpha=None, beta=None, eps=1e-6, S0=None, z0=None, normalize=True):
    """Causal linear attention as an RNN over t, in float64.

    For each t (in order):
        S_t = alpha_t S_{t-1} + beta_t phi(k_t) v_t^T      (d' x d_v)
        z_t = alpha_t z_{t-1} + beta_t phi(k_t)            (d')
        o_t = S_t^T phi(q_t) / (z_t^T phi(q_t) + eps)
    The read-out uses the state after token t is added (inclusive causal
    sum).  [lesson] Researcher level, Derivation (recurrence and read-out);
    [kb] section 3 causal sketch (eps added to the denominator);
    [card] Implementation sketch (decay on the old state only).
    normalize=False returns the numerator S_t^T phi(q_t) alone, the
    normaliser-free read-out of [card] "Decaying linear attention with a
    scalar state (SSD)"; z is still carried.  normalize="max1" divides by
    max(|z_t^T phi(q_t)|, 1) instead ([card] mLSTM read-out).

    fq, fk: [..., T, d'] features; v: [..., T, d_v]; alpha, beta: [..., T]
    or None.  S0: [..., d', d_v], z0: [..., d'] (default zero state).
    Returns (o [..., T, d_v], S_T, z_T).
    """
    fq, fk, v = _f64(fq), _f64(fk), _f64(v)
    lead = fq.shape[:-2]
    T, dp = fq.shape[-2], fq.shape[-1]
    dv = v.shape[-1]
    S = np.zeros(lead + (dp, dv), F64) if S0 is None else _f64(S0).copy()
    z = np.zeros(lead + (dp,), F64) if z0 is None else _f64(z0).copy()
    alpha = _f64(alpha)
    beta = _f64(beta)
    o = np.empty(lead + (T, dv), F64)
    for t in range(T):
        k_t = fk[..., t, :]
        new_S = k_t[..., :, None] * v[..., t, None, :]
        new_z = k_t
        if beta is not None:
            b = beta[..., t]
            new_S = b[..., None, None] * new_S
            new_z = b[..., None] * new_z
        if alpha is not None:
            a = alpha[..., t]
            S = a[..., None, None] * S + new_S
            z = a[..., None] * z + new_z
        else:
            S = S + new_S
            z = z + new_z
        q_t = fq[..., t, :]
        num = np.einsum("...d,...dv->...v", q_t, S)
        den = np.einsum("...d,...d->...", q_t, z)
        o[..., t, :] = readout(num, den, eps, normalize)
    return o, S, z


def causal_linear_attention(q, k, v, phi="elu1", W=None, decay=None, gate=None,
                            eps=1e-6, S0=None, z0=None, normalize=True):
    """Feature map, then the recurrence.  Returns (o, S, z) in float64.

    q, k: [..., H, T, d_h]; v: [..., H, T, d_v]; W: [H, D, d_h] for RFF.
    [card] Implementation sketch (the pluggable-feature-map loop).
    """
    fq = features(q, phi, W)
    fk = features(k, phi, W)
    alpha, beta = decay_coefficients(decay, gate)
    return recurrence(fq, fk, v, alpha, beta, eps, S0, z0, normalize)


def decode_step(q, k, v, S, z, phi="elu1", W=None, decay=None, gate=None, eps=1e-6,
                normalize=True):
    """One autoregressive step from state (S, z): q, k [..., H, d_h], v [..., H, d_v],
    decay/gate [..., H].  Returns (o [..., H, d_v], S', z').

    [kb] section 2, causal recurrence (constant-state RNN step).
    """
    q, k, v = _f64(q)[..., None, :], _f64(k)[..., None, :], _f64(v)[..., None, :]
    decay = None if decay is None else _f64(decay)[..., None]
    gate = None if gate is None else _f64(gate)[..., None]
    o, S, z = causal_linear_attention(q, k, v, phi, W, decay, gate, eps, S, z, normalize)
    return o[..., 0, :], S, z


# --------------------------------------------------------------------------
# The definition (masked quadratic form), used to pin the recurrence and to
# compute sampled outputs at full size one by one
# --------------------------------------------------------------------------

def decay_products(alpha, T):
    """P[..., t, s] = prod_{r=s+1..t} alpha_r for s <= t, else 0 (products
    taken directly, no logarithms, so alpha = 0 is exact)."""
    if alpha is None:
        return np.tril(np.ones((T, T), F64))
    alpha = _f64(alpha)
    lead = alpha.shape[:-1]
    P = np.zeros(lead + (T, T), F64)
    for t in range(T):
        run = np.ones(lead, F64)
        for s in range(t, -1, -1):
            P[..., t, s] = run
            run = run * alpha[..., s]
    return P


def masked_quadratic(fq, fk, v, alpha=None, beta=None, eps=1e-6, normalize=True):
    """o_t = sum_{s<=t} w_ts v_s / (sum_{s<=t} w_ts + eps) with
    w_ts = (phi(q_t) . phi(k_s)) * beta_s * prod_{r=s+1..t} alpha_r.

    With no decay this is scores * tril(1) ([lesson] Developer level, the
    masked quadratic check; Researcher level, the sim-attention sum over
    j <= i).  With a constant decay it is the weighted quadratic form asked
    for in [lesson] "Try it yourself".  Zero initial state.  O(T^2).
    """
    fq, fk, v = _f64(fq), _f64(fk), _f64(v)
    T = fq.shape[-2]
    scores = fq @ np.swapaxes(fk, -1, -2)
    w = scores * decay_products(alpha, T)
    if beta is not None:
        w = w * _f64(beta)[..., None, :]
    return readout(w @ v, w.sum(axis=-1), eps, normalize)


def kernel_attention_by_definition(fq, fk, v, alpha=None, beta=None, eps=1e-6, normalize=True):
    """Pure-Python double loop over one head: o_i = sum_{j<=i} sim_ij v_j /
    (sum_{j<=i} sim_ij + eps), sim_ij = phi(q_i).phi(k_j) times the decay
    weight.  Tiny inputs only.  [lesson] Researcher level, Derivation."""
    fq, fk, v = _f64(fq), _f64(fk), _f64(v)
    T, dv = fq.shape[0], v.shape[1]
    out = np.zeros((T, dv), F64)
    for i in range(T):
        num = [0.0] * dv
        den = 0.0
        for j in range(i + 1):
            sim = sum(float(fq[i, c]) * float(fk[j, c]) for c in range(fq.shape[1]))
            wgt = 1.0 if beta is None else float(beta[j])
            for r in range(j + 1, i + 1):
                wgt *= 1.0 if alpha is None else float(alpha[r])
            sim *= wgt
            den += sim
            for c in range(dv):
                num[c] += sim * float(v[j, c])
        for c in range(dv):
            out[i, c] = _readout_scalar(num[c], den, eps, normalize)
    return out


def output_at(fq_t, fk, v, t, alpha=None, beta=None, eps=1e-6, S0=None, z0=None,
              normalize=True):
    """The definition evaluated at one position t (O(t d)), including the
    carried-in state (S0, z0) decayed by prod_{r=0..t} alpha_r.

    fq_t: [..., d'] (features of query t); fk: [..., T, d']; v: [..., T, d_v].
    """
    fq_t, fk, v = _f64(fq_t), _f64(fk)[..., : t + 1, :], _f64(v)[..., : t + 1, :]
    sims = np.einsum("...d,...sd->...s", fq_t, fk)
    lead = sims.shape[:-1]
    if alpha is not None:
        a = _f64(alpha)[..., : t + 1]
        # weight of key s: prod_{r=s+1..t} alpha_r  (reverse cumulative product)
        rev = np.cumprod(a[..., :0:-1], axis=-1)[..., ::-1]
        wts = np.concatenate([rev, np.ones(lead + (1,), F64)], axis=-1)
        carry = np.prod(a, axis=-1)
    else:
        wts = np.ones(lead + (t + 1,), F64)
        carry = np.ones(lead, F64)
    if beta is not None:
        wts = wts * _f64(beta)[..., : t + 1]
    w = sims * wts
    num = np.einsum("...s,...sv->...v", w, v)
    den = w.sum(axis=-1)
    if S0 is not None:
        num = num + carry[..., None] * np.einsum("...d,...dv->...v", fq_t, _f64(S0))
    if z0 is not None:
        den = den + carry * np.einsum("...d,...d->...", fq_t, _f64(z0))
    return readout(num, den, eps, normalize)


def final_state(fk, v, alpha=None, beta=None, S0=None, z0=None):
    """S_T = (prod alpha) S0 + sum_s w_s phi(k_s) v_s^T and likewise z_T, with
    w_s = beta_s prod_{r=s+1..T-1} alpha_r: the closed form of the state after
    T tokens ([lesson] Researcher level: both sums are prefix sums)."""
    fk, v = _f64(fk), _f64(v)
    T = fk.shape[-2]
    lead = fk.shape[:-2]
    if alpha is not None:
        a = _f64(alpha)
        rev = np.cumprod(a[..., :0:-1], axis=-1)[..., ::-1]
        w = np.concatenate([rev, np.ones(lead + (1,), F64)], axis=-1)
        carry = np.prod(a, axis=-1)
    else:
        w = np.ones(lead + (T,), F64)
        carry = np.ones(lead, F64)
    if beta is not None:
        w = w * _f64(beta)
    # optimize=True lets numpy contract pairwise through BLAS; same sums
    S = np.einsum("...s,...sd,...sv->...dv", w, fk, v, optimize=True)
    z = np.einsum("...s,...sd->...d", w, fk)
    if S0 is not None:
        S = S + carry[..., None, None] * _f64(S0)
    if z0 is not None:
        z = z + carry[..., None] * _f64(z0)
    return S, z


# --------------------------------------------------------------------------
# mLSTM: matrix memory with exponential gates ([card] Variants / "Matrix
# memory with exponential gates (mLSTM)"; [card] Implementation sketch: the
# mLSTM step is the loop above with the identity feature map,
# input-dependent gates and a normaliser read-out)
#
# Per token, with forget gate f_t and input gate i_t = exp(itilde_t):
#     C_t = f_t C_{t-1} + i_t k_t v_t^T,   n_t = f_t n_{t-1} + i_t k_t,
#     o_t = C_t^T q_t / max(|n_t^T q_t|, 1),
# i.e. the recurrence with phi = identity, alpha = f, beta = i and the
# "max1" read-out (the page's C is this library's S transposed, n is z).
# f_t = sigmoid(ftilde_t), or exp(ftilde_t) in the exponential form.
#
# The stabiliser: the page says only that a stabiliser state keeps the
# exponentials from overflowing.  Reading: a log-domain running maximum
#     m_t = max(log f_t + m_{t-1}, itilde_t),
# with the state kept as (S', z', m) = (e^{-m} S, e^{-m} z, m):
#     S'_t = e^{log f_t + m_{t-1} - m_t} S'_{t-1} + e^{itilde_t - m_t} k_t v_t^T,
# both factors <= 1, and the read-out floor 1 becoming e^{-m_t}
#     o_t = q_t^T S'_t / max(|q_t^T z'_t|, e^{-m_t}),
# which is the same number as the unstabilised read-out.  A zero state has
# m = 0.
# --------------------------------------------------------------------------

def log_forget(fgate, exp_form=False):
    """log f_t from the forget-gate pre-activation: log sigmoid(x) =
    -log(1 + e^{-x}), or x itself for the exponential forget gate."""
    x = _f64(fgate)
    return x.copy() if exp_form else -np.logaddexp(0.0, -x)


def mlstm_coefficients(igate, fgate, exp_form=False):
    """Unstabilised (alpha, beta) = (f_t, i_t) = (sigmoid or exp of the forget
    pre-activation, exp of the input pre-activation), for the definition."""
    return np.exp(log_forget(fgate, exp_form)), np.exp(_f64(igate))


def mlstm_by_definition(q, k, v, igate, fgate, exp_form=False, eps=1e-6, S0=None, z0=None,
                        normalize="max1"):
    """The mLSTM recurrence taken literally (no stabiliser), in float64:
    identity features, alpha = f, beta = i.  Returns (o, S, z) with the true
    (unscaled) state.  Overflows for input pre-activations beyond ~700."""
    f, i = mlstm_coefficients(igate, fgate, exp_form)
    return recurrence(phi_identity(q), phi_identity(k), v, f, i, eps, S0, z0, normalize)


def _scaled_readout(num, den, eps, normalize, m):
    """Read-out of a state scaled by e^{-m}: the same number as readout() of
    the unscaled numerator and denominator."""
    if normalize is True:
        return num / (den + eps * np.exp(-m))[..., None]
    if normalize is False:
        return num * np.exp(m)[..., None]
    if normalize == "max1":
        return num / np.maximum(np.abs(den), np.exp(-m))[..., None]
    raise ValueError(f"unknown read-out {normalize!r}")


def mlstm_recurrence(q, k, v, igate, fgate, exp_form=False, eps=1e-6, S0=None, z0=None,
                     m0=None, normalize="max1"):
    """The stabilised mLSTM recurrence (the reading in the comment above),
    token by token in float64.

    q, k: [..., T, d]; v: [..., T, d_v]; igate, fgate: [..., T] (input and
    forget pre-activations).  (S0, z0, m0): the scaled start state (zero, and
    m0 = 0, by default).  Returns (o, S', z', m) with S = e^m S'.
    """
    fq, fk, v = phi_identity(q), phi_identity(k), _f64(v)
    lead = fq.shape[:-2]
    T, dp = fq.shape[-2], fq.shape[-1]
    dv = v.shape[-1]
    S = np.zeros(lead + (dp, dv), F64) if S0 is None else _f64(S0).copy()
    z = np.zeros(lead + (dp,), F64) if z0 is None else _f64(z0).copy()
    m = np.zeros(lead, F64) if m0 is None else _f64(m0).copy()
    lf = log_forget(fgate, exp_form)
    it = _f64(igate)
    o = np.empty(lead + (T, dv), F64)
    for t in range(T):
        m_new = np.maximum(lf[..., t] + m, it[..., t])
        fs = np.exp(lf[..., t] + m - m_new)      # stabilised forget factor
        is_ = np.exp(it[..., t] - m_new)         # stabilised input factor
        k_t = fk[..., t, :]
        S = fs[..., None, None] * S + is_[..., None, None] * (k_t[..., :, None] * v[..., t, None, :])
        z = fs[..., None] * z + is_[..., None] * k_t
        m = m_new
        q_t = fq[..., t, :]
        num = np.einsum("...d,...dv->...v", q_t, S)
        den = np.einsum("...d,...d->...", q_t, z)
        o[..., t, :] = _scaled_readout(num, den, eps, normalize, m)
    return o, S, z, m


def mlstm_log_weights(igate, fgate, t, exp_form=False):
    """lambda_s = itilde_s + sum_{r=s+1..t} log f_r for s = 0..t (the log
    weight of key s at step t) and the log decay of the start state,
    sum_{r=0..t} log f_r.  [..., t+1] and [...]."""
    lf = log_forget(fgate, exp_form)[..., : t + 1]
    it = _f64(igate)[..., : t + 1]
    # suffix sums of log f after s: total - inclusive prefix
    pref = np.cumsum(lf, axis=-1)
    total = pref[..., -1]
    return it + (total[..., None] - pref), total


def mlstm_output_at(q_t, k, v, t, igate, fgate, exp_form=False, eps=1e-6, S0=None, z0=None,
                    m0=None, normalize="max1"):
    """The mLSTM output at one position t by its definition, O(t d):
    o_t = sum_{s<=t} w_s (q_t.k_s) v_s / max(|sum_s w_s q_t.k_s|, 1) with
    w_s = i_s prod_{r=s+1..t} f_r, plus the start state decayed by
    prod_{r<=t} f_r.  Numerator and denominator are both scaled by e^{-M},
    M the largest log weight, so nothing overflows; the quotient is
    unchanged."""
    q_t, k, v = _f64(q_t), _f64(k)[..., : t + 1, :], _f64(v)[..., : t + 1, :]
    lam, carry = mlstm_log_weights(igate, fgate, t, exp_form)
    lead = lam.shape[:-1]
    m0 = np.zeros(lead, F64) if m0 is None else _f64(m0)
    lc = carry + m0                                   # log scale of the start state's term
    M = np.maximum(lam.max(axis=-1), lc)
    w = np.exp(lam - M[..., None]) * np.einsum("...d,...sd->...s", q_t, k)
    num = np.einsum("...s,...sv->...v", w, v)
    den = w.sum(axis=-1)
    if S0 is not None:
        num = num + np.exp(lc - M)[..., None] * np.einsum("...d,...dv->...v", q_t, _f64(S0))
    if z0 is not None:
        den = den + np.exp(lc - M) * np.einsum("...d,...d->...", q_t, _f64(z0))
    return _scaled_readout(num, den, eps, normalize, M)


def mlstm_final_state(k, v, igate, fgate, exp_form=False, S0=None, z0=None, m0=None):
    """The scaled state after T tokens in closed form: the stabiliser is the
    max-plus unrolling of its recurrence,
        m_T = max(m0 + sum_r log f_r, max_s (itilde_s + sum_{r>s} log f_r)),
    and S' = sum_s e^{lambda_s - m_T} k_s v_s^T + e^{m0 + sum log f - m_T} S0'
    (z' likewise).  Returns (S', z', m_T)."""
    k, v = _f64(k), _f64(v)
    T = k.shape[-2]
    lam, carry = mlstm_log_weights(igate, fgate, T - 1, exp_form)
    lead = lam.shape[:-1]
    m0 = np.zeros(lead, F64) if m0 is None else _f64(m0)
    lc = carry + m0
    m = np.maximum(lam.max(axis=-1), lc)
    w = np.exp(lam - m[..., None])
    S = np.einsum("...s,...sd,...sv->...dv", w, k, v, optimize=True)
    z = np.einsum("...s,...sd->...d", w, k)
    if S0 is not None:
        S = S + np.exp(lc - m)[..., None, None] * _f64(S0)
    if z0 is not None:
        z = z + np.exp(lc - m)[..., None] * _f64(z0)
    return S, z, m


# --------------------------------------------------------------------------
# Non-causal bracketings ([kb] section 3 non-causal sketch; [lesson] Developer
# level, "Two ways to bracket the same product")
# --------------------------------------------------------------------------

def noncausal_left(fq, fk, v, eps=1e-6):
    """((phi(Q) phi(K)^T) V) / ((phi(Q) phi(K)^T) 1 + eps): T x T scores first."""
    fq, fk, v = _f64(fq), _f64(fk), _f64(v)
    A = fq @ np.swapaxes(fk, -1, -2)
    return (A @ v) / (A.sum(axis=-1) + eps)[..., None]


def noncausal_right(fq, fk, v, eps=1e-6):
    """(phi(Q) (phi(K)^T V)) / (phi(Q) (phi(K)^T 1) + eps): d' x d_v state first."""
    fq, fk, v = _f64(fq), _f64(fk), _f64(v)
    S = np.swapaxes(fk, -1, -2) @ v
    z = fk.sum(axis=-2)
    return (fq @ S) / (np.einsum("...td,...d->...t", fq, z) + eps)[..., None]


def noncausal_linear_attention(q, k, v, phi="elu1", W=None, eps=1e-6, S0=None, z0=None,
                               normalize=True):
    """Non-causal linear attention ([kb] section 3, non-causal sketch; [lesson]
    Developer level, the phi(Q) (phi(K)^T V) bracketing): every query reads
    the state of the whole sequence, S = S0 + phi(K)^T V and z = z0 +
    phi(K)^T 1, as o_t = phi(q_t)^T S / (phi(q_t)^T z + eps), or the
    numerator alone with normalize=False.  The state is the one a causal pass
    over the same tokens ends with.  Returns (o, S, z) in float64.

    q, k: [..., H, T, d_h]; v: [..., H, T, d_v]; S0, z0 as for the causal form.
    """
    fq = features(q, phi, W)
    fk = features(k, phi, W)
    v = _f64(v)
    S = np.swapaxes(fk, -1, -2) @ v
    z = fk.sum(axis=-2)
    if S0 is not None:
        S = S + _f64(S0)
    if z0 is not None:
        z = z + _f64(z0)
    num = fq @ S
    den = np.einsum("...td,...d->...t", fq, z)
    return readout(num, den, eps, normalize), S, z


def noncausal_by_definition(fq, fk, v, eps=1e-6, normalize=True):
    """Pure-Python double loop over one head: o_i = sum_j sim_ij v_j /
    (sum_j sim_ij + eps) over every key j.  Tiny inputs only."""
    fq, fk, v = _f64(fq), _f64(fk), _f64(v)
    T, dv = fq.shape[0], v.shape[1]
    out = np.zeros((T, dv), F64)
    for i in range(T):
        num = [0.0] * dv
        den = 0.0
        for j in range(T):
            sim = sum(float(fq[i, c]) * float(fk[j, c]) for c in range(fq.shape[1]))
            den += sim
            for c in range(dv):
                num[c] += sim * float(v[j, c])
        for c in range(dv):
            out[i, c] = _readout_scalar(num[c], den, eps, normalize)
    return out


# --------------------------------------------------------------------------
# Gradients of the causal prefill (training; [lesson] Developer level and
# "Implementation reality": training runs the chunked form, which computes
# the same function, so its gradients are those of the definition)
# --------------------------------------------------------------------------

def phi_derivative(x, phi="elu1"):
    """d phi / dx element-wise: elu+1 has slope 1 for x > 0 and e^x below;
    the identity has slope 1."""
    x = _f64(x)
    if phi == "elu1":
        return np.where(x > 0, 1.0, np.exp(np.minimum(x, 0.0)))
    if phi == "identity":
        return np.ones_like(x)
    raise ValueError(f"no derivative for feature map {phi!r}")


def prefill_gradients(q, k, v, dout, phi="elu1", decay=None, gate=None, eps=1e-6, S0=None,
                      z0=None, normalize=True):
    """Gradients of L = sum_t <dout_t, o_t> for the causal prefill, from the
    masked quadratic form (the definition) in float64, one head at a time
    (leading dims are looped):

        W_ts = (phi(q_t).phi(k_s)) beta_s prod_{r=s+1..t} alpha_r   (s <= t)
        num_t = sum_s W_ts v_s + c_t phi(q_t)^T S0,  den_t = sum_s W_ts + c_t phi(q_t).z0
        o_t = num_t / (den_t + eps)   (or num_t, or num_t / max(|den_t|, 1))

    with c_t = prod_{r<=t} alpha_r.  Reverse-mode by hand:
        g_num = dout / D,  g_den = -(dout . o) / D   (D the read-out's divisor)
        dW = g_num V^T + g_den 1^T,   dphi(Q) = (dW o M) phi(K) + c (g_num S0^T + g_den z0^T)
        dphi(K) = (dW o M)^T phi(Q) ..., dV = W^T g_num,
    and the decay through the products M.  Returns a dict with dq, dk, dv,
    dS0, dz0 and (with decay/gate) ddecay or dgate, all float64.
    """
    fq_all, fk_all = features(q, phi), features(k, phi)
    dphq, dphk = phi_derivative(q, phi), phi_derivative(k, phi)
    v_all, do_all = _f64(v), _f64(dout)
    alpha_all, beta_all = decay_coefficients(decay, gate)
    lead = fq_all.shape[:-2]
    T, dp = fq_all.shape[-2:]
    dv_ = v_all.shape[-1]
    out = {n: np.zeros(lead + shp) for n, shp in (("dq", (T, q.shape[-1])), ("dk", (T, k.shape[-1])),
                                                  ("dv", (T, dv_)), ("dS0", (dp, dv_)), ("dz0", (dp,)),
                                                  ("dalpha", (T,)), ("dbeta", (T,)))}
    for idx in np.ndindex(*lead):
        fq, fk, vv, do = fq_all[idx], fk_all[idx], v_all[idx], do_all[idx]
        al = np.ones(T) if alpha_all is None else alpha_all[idx]
        be = np.ones(T) if beta_all is None else beta_all[idx]
        S0i = np.zeros((dp, dv_)) if S0 is None else _f64(S0)[idx]
        z0i = np.zeros(dp) if z0 is None else _f64(z0)[idx]
        # P[t, s] = prod_{r=s+1..t} alpha_r (s <= t); c[t] = prod_{r<=t} alpha_r
        P = decay_products(al, T)
        c = np.cumprod(al)
        A = fq @ fk.T                                   # raw scores
        M = P * be[None, :]                             # decay and beta weights
        W = A * M
        num = W @ vv + c[:, None] * (fq @ S0i)
        den = W.sum(1) + c * (fq @ z0i)
        if normalize is True:
            Dv = den + eps
            o = num / Dv[:, None]
            g_num = do / Dv[:, None]
            g_den = -(do * o).sum(1) / Dv
        elif normalize is False:
            g_num = do.copy()
            g_den = np.zeros(T)
        elif normalize == "max1":
            Dv = np.maximum(np.abs(den), 1.0)
            o = num / Dv[:, None]
            g_num = do / Dv[:, None]
            # d/d den of max(|den|, 1): sign(den) where |den| > 1, else 0
            g_den = np.where(np.abs(den) > 1.0, -np.sign(den) * (do * o).sum(1) / Dv, 0.0)
        else:
            raise ValueError(f"unknown read-out {normalize!r}")
        dW = g_num @ vv.T + g_den[:, None]              # dL/dW_ts (s <= t used through M)
        dA = dW * M
        dfq = dA @ fk + c[:, None] * (g_num @ S0i.T + g_den[:, None] * z0i[None, :])
        dfk = dA.T @ fq
        out["dq"][idx] = dfq * dphq[idx]
        out["dk"][idx] = dfk * dphk[idx]
        out["dv"][idx] = W.T @ g_num
        out["dS0"][idx] = (c[:, None] * fq).T @ g_num
        out["dz0"][idx] = (c * g_den) @ fq
        # decay: dL/dM_ts = dW_ts A_ts.  M_ts = beta_s prod_{r'=s+1..t}
        # alpha_r' holds alpha_r exactly when s < r <= t, as the factor
        # between P[r-1, s] and P[t, r]; the start-state carry c_t holds it
        # when r <= t, between c_{r-1} and P[t, r].  So, as the product over
        # r' != r with no division (alpha_r = 0, a full reset, included):
        #   dL/dalpha_r = sum_{t>=r} P[t, r] (sum_{s<r} dM_ts beta_s P[r-1, s]
        #                                     + dc_t c_{r-1}),
        # and dL/dbeta_s = sum_t dM_ts P_ts.
        dM = dW * A
        dc = (g_num * (fq @ S0i)).sum(1) + g_den * (fq @ z0i)
        for r in range(T):
            c_prev = c[r - 1] if r > 0 else 1.0
            inner = dM[r:, :r] @ (be[:r] * P[r - 1, :r]) if r > 0 else np.zeros(T)
            out["dalpha"][idx][r] = P[r:, r] @ (inner + dc[r:] * c_prev)
        out["dbeta"][idx] = (dM * P).sum(0)
    res = {n: out[n] for n in ("dq", "dk", "dv", "dS0", "dz0")}
    if decay is not None:
        res["ddecay"] = out["dalpha"]
    if gate is not None:
        # alpha = g, beta = 1 - g
        res["dgate"] = out["dalpha"] - out["dbeta"]
    return res


def _reverse_mode_head(fq, fk, vv, do, al, be, S, z, readout):
    """Reverse mode through S_t = al_t S_{t-1} + be_t phi(k_t) v_t^T (z
    likewise) for one head, in float64.  readout(t, num, den) gives the
    read-out's (g_t, h_t): the gradients of L with respect to the numerator
    and the divisor's dot product.  Returns (dphi(q), dphi(k), dv, dL/dal,
    dL/dbe, G, gz) with G, gz the gradient state before the first token, and
    dL/dal_r = <G_r, S_{r-1}> + <gz_r, z_{r-1}> (no division by al_r).  The
    walk back needs S_{r-1} beside G_r: the forward walk keeps the state
    every CKPT tokens, and each block of CKPT tokens is walked forward again
    from its checkpoint before it is walked back."""
    CKPT = 64
    T, dp = fq.shape
    dv_ = vv.shape[-1]
    g = np.empty((T, dv_))
    h = np.empty(T)
    dfq = np.empty((T, dp))
    ckpt = {}                 # the state before token t, every CKPT tokens
    for t in range(T):
        if t % CKPT == 0:
            ckpt[t] = (S.copy(), z.copy())
        S = al[t] * S + be[t] * np.outer(fk[t], vv[t])
        z = al[t] * z + be[t] * fk[t]
        g[t], h[t] = readout(t, fq[t] @ S, fq[t] @ z)
        dfq[t] = S @ g[t] + z * h[t]
    G = np.zeros((dp, dv_))
    gz = np.zeros(dp)
    dfk = np.empty((T, dp))
    dvv = np.empty((T, dv_))
    dal = np.empty(T)
    dbe = np.empty(T)
    for b0 in sorted(ckpt, reverse=True):
        b1 = min(b0 + CKPT, T)
        Sp, zp = ckpt[b0]
        prev = []             # (S_{t-1}, z_{t-1}) for t in [b0, b1)
        for t in range(b0, b1):
            prev.append((Sp, zp))
            Sp = al[t] * Sp + be[t] * np.outer(fk[t], vv[t])
            zp = al[t] * zp + be[t] * fk[t]
        for t in range(b1 - 1, b0 - 1, -1):
            a_next = al[t + 1] if t + 1 < T else 0.0
            G = a_next * G + np.outer(fq[t], g[t])
            gz = a_next * gz + fq[t] * h[t]
            u = G @ vv[t] + gz
            dfk[t] = be[t] * u
            dvv[t] = be[t] * (fk[t] @ G)
            dbe[t] = fk[t] @ u
            Sm, zm = prev[t - b0]
            dal[t] = (G * Sm).sum() + gz @ zm
    return dfq, dfk, dvv, dal, dbe, G, gz


def _readout_grads(normalize, eps, floor=1.0):
    """(g_t, h_t) of the read-out from its numerator and divisor dot product:
    the sum form num / (den + eps), the numerator alone, or num / max(|den|,
    floor).  With a state held scaled by e^{-m_t} (the mLSTM gates) the same
    read-outs of the true state are num' / (den' + eps e^{-m_t}), e^{m_t}
    num' and num' / max(|den'|, e^{-m_t}): eps, the scale and the floor
    given per token."""
    def grads(do, num, den, eps_t, scale_t, floor_t):
        if normalize is True:
            Dv = den + eps_t
            return do / Dv, -(do @ (num / Dv)) / Dv
        if normalize is False:
            return do * scale_t, 0.0
        if normalize == "max1":
            Dv = max(abs(den), floor_t)
            return do / Dv, (-np.sign(den) * (do @ (num / Dv)) / Dv if abs(den) > floor_t else 0.0)
        raise ValueError(f"unknown read-out {normalize!r}")
    return grads


def prefill_gradients_recurrent(q, k, v, dout, phi="elu1", decay=None, gate=None, eps=1e-6,
                                S0=None, z0=None, normalize=True):
    """The same gradients as prefill_gradients, by reverse mode through the
    recurrence instead of the quadratic form (O(T d' d_v) per head, for long
    sequences), in float64.

    Forward over t ([lesson] Researcher level, Derivation; [card]
    Implementation sketch: S_t = alpha_t S_{t-1} + beta_t phi(k_t) v_t^T, z_t
    likewise, o_t read from the state after token t):
        D_t the read-out's divisor, g_t = dout_t / D_t, h_t its gradient
        (-(dout_t . o_t) / D_t for the sum read-out),
        dphi(q_t) = S_t g_t + z_t h_t.
    Backward over t, with the gradient state G (d' x d_v) and gz (d'):
        G <- alpha_{t+1} G + phi(q_t) g_t^T,  gz likewise with h_t
        u_t = G v_t + gz,  dphi(k_t) = beta_t u_t,  dv_t = beta_t G^T phi(k_t).
    The decay multiplies the previous state in S_r = alpha_r S_{r-1} + ...,
    and G_r is the gradient of S_r, so
        dL/dalpha_r = <G_r, S_{r-1}> + <gz_r, z_{r-1}>,
        dL/dbeta_t = phi(k_t) . u_t,
    with no division by alpha (alpha_r = 0, a full reset, included).
    The initial state enters S_t as prod_{r<=t} alpha_r S0: dS0 = alpha_0 G,
    dz0 = alpha_0 gz after the walk.  Returns a dict with dq, dk, dv, dS0,
    dz0 and ddecay (with decay) or dgate (with gate).
    """
    fq_all, fk_all = features(q, phi), features(k, phi)
    dphq, dphk = phi_derivative(q, phi), phi_derivative(k, phi)
    v_all, do_all = _f64(v), _f64(dout)
    alpha_all, beta_all = decay_coefficients(decay, gate)
    lead = fq_all.shape[:-2]
    T, dp = fq_all.shape[-2:]
    dv_ = v_all.shape[-1]
    res = {n: np.zeros(lead + shp) for n, shp in (("dq", (T, q.shape[-1])), ("dk", (T, k.shape[-1])),
                                                  ("dv", (T, dv_)), ("dS0", (dp, dv_)), ("dz0", (dp,)),
                                                  ("dalpha", (T,)), ("dbeta", (T,)))}
    grads = _readout_grads(normalize, eps)
    for idx in np.ndindex(*lead):
        do = do_all[idx]
        al = np.ones(T) if alpha_all is None else alpha_all[idx]
        be = np.ones(T) if beta_all is None else beta_all[idx]
        S = np.zeros((dp, dv_)) if S0 is None else _f64(S0)[idx].copy()
        z = np.zeros(dp) if z0 is None else _f64(z0)[idx].copy()
        rd = lambda t, num, den: grads(do[t], num, den, eps, 1.0, 1.0)
        dfq, dfk, dvv, dal, dbe, G, gz = _reverse_mode_head(fq_all[idx], fk_all[idx], v_all[idx],
                                                            do, al, be, S, z, rd)
        res["dq"][idx] = dfq * dphq[idx]
        res["dk"][idx] = dfk * dphk[idx]
        res["dv"][idx] = dvv
        res["dS0"][idx] = al[0] * G
        res["dz0"][idx] = al[0] * gz
        res["dalpha"][idx] = dal
        res["dbeta"][idx] = dbe
    out = {n: res[n] for n in ("dq", "dk", "dv", "dS0", "dz0")}
    if decay is not None:
        out["ddecay"] = res["dalpha"]
    if gate is not None:
        out["dgate"] = res["dalpha"] - res["dbeta"]
    return out


def mlstm_gradients(q, k, v, dout, igate, fgate, exp_form=False, eps=1e-6, S0=None, z0=None,
                    m0=None, normalize="max1"):
    """Gradients of L = sum_t <dout_t, o_t> for the mLSTM gates ([card]
    "Variants / Matrix memory with exponential gates (mLSTM)"), o from
    mlstm_recurrence, in float64: with respect to q, k, v, the forget and
    input pre-activations, and the scaled start state (S0', z0', m0).

    L depends on the true state S_t = e^{m_t} S'_t, whose recurrence has
    alpha_t = f_t and beta_t = i_t = e^{itilde_t}; the stabiliser only picks
    the scale it is held at.  Reverse mode runs in that scale: the scaled
    recurrence S'_t = alpha'_t S'_{t-1} + beta'_t k_t v_t^T (alpha'_t =
    e^{log f_t + m_{t-1} - m_t}, beta'_t = e^{itilde_t - m_t}, as in
    mlstm_recurrence) with the scaled read-out, whose factors g'_t = e^{m_t}
    g_t give the gradient state G'_t = e^{m_t} G_t.  Then
        dq_t = S'_t g'_t + z'_t h'_t,  dk_t = beta'_t (G'_t v_t + gz'_t),
        dv_t = beta'_t G'_t^T k_t,
        dL/dlog f_r = f_r <G_r, S_{r-1}> + ... = alpha'_r (<G'_r, S'_{r-1}>
                      + <gz'_r, z'_{r-1}>),
        dL/ditilde_t = i_t k_t . (G_t v_t + gz_t) = beta'_t k_t . (G'_t v_t + gz'_t),
        dL/dS0' = alpha'_0 G'_0 (S_init = e^{m0} S0'), dz0' alike,
        dL/dm0 = <dS0', S0'> + <dz0', z0'>,
    and dL/dfgate = dL/dlog f times d log f / dfgate: 1 - f for the sigmoid
    gate, 1 for the exponential one.  Returns a dict with dq, dk, dv, dfgate,
    digate, dS0, dz0 and dm0.
    """
    fq_all, fk_all, v_all, do_all = phi_identity(q), phi_identity(k), _f64(v), _f64(dout)
    lf_all = log_forget(fgate, exp_form)
    it_all = _f64(igate)
    lead = fq_all.shape[:-2]
    T, dp = fq_all.shape[-2:]
    dv_ = v_all.shape[-1]
    res = {n: np.zeros(lead + shp) for n, shp in (("dq", (T, dp)), ("dk", (T, dp)), ("dv", (T, dv_)),
                                                  ("dfgate", (T,)), ("digate", (T,)),
                                                  ("dS0", (dp, dv_)), ("dz0", (dp,)), ("dm0", ()))}
    grads = _readout_grads(normalize, eps)
    for idx in np.ndindex(*lead):
        lf, it, do = lf_all[idx], it_all[idx], do_all[idx]
        S = np.zeros((dp, dv_)) if S0 is None else _f64(S0)[idx].copy()
        z = np.zeros(dp) if z0 is None else _f64(z0)[idx].copy()
        m_prev = 0.0 if m0 is None else float(_f64(m0)[idx])
        m = np.empty(T)
        for t in range(T):
            m[t] = max(lf[t] + m_prev, it[t])
            m_prev = m[t]
        m_before = np.concatenate([[0.0 if m0 is None else float(_f64(m0)[idx])], m[:-1]])
        al = np.exp(lf + m_before - m)
        be = np.exp(it - m)
        rd = lambda t, num, den: grads(do[t], num, den, eps * np.exp(-m[t]), np.exp(m[t]),
                                       np.exp(-m[t]))
        S_init, z_init = S.copy(), z.copy()
        dfq, dfk, dvv, dal, dbe, G, gz = _reverse_mode_head(fq_all[idx], fk_all[idx], v_all[idx],
                                                            do, al, be, S, z, rd)
        dlogf = al * dal
        f = np.exp(lf)
        res["dq"][idx] = dfq
        res["dk"][idx] = dfk
        res["dv"][idx] = dvv
        res["dfgate"][idx] = dlogf if exp_form else dlogf * (1.0 - f)
        res["digate"][idx] = be * dbe
        res["dS0"][idx] = al[0] * G
        res["dz0"][idx] = al[0] * gz
        res["dm0"][idx] = (res["dS0"][idx] * S_init).sum() + res["dz0"][idx] @ z_init
    return res


# --------------------------------------------------------------------------
# Accounting the pages print
# --------------------------------------------------------------------------

def state_update_ops(T, d_prime, d_h):
    """T rank-one updates of O(d' d_h) each ([kb] section 2, compute cost)."""
    return T * d_prime * d_h


def softmax_ops(T, d_h):
    """The T x T score matrix times d_h ([kb] section 2, compute cost)."""
    return T * T * d_h


def state_numbers(d_prime, d_v):
    """Numbers held by S ([lesson] Developer level: S is d x d, never grows)."""
    return d_prime * d_v


def kv_cache_numbers(t, d):
    """A softmax KV cache at step t holds 2 t d numbers ([lesson] Developer level)."""
    return 2 * t * d


def worked_example_report(q, k, v, eps=1e-6):
    """The checks of the pages' T=8, d=4 example, evaluated in float64:
    bracketing agreement, shapes of (q k^T) and (k^T V), recurrent vs masked
    quadratic agreement and their max difference, state size, KV-cache size.
    ([lesson] Developer level, "The regrouping, and the recurrence it implies")."""
    fq, fk, vv = phi_elu1(q), phi_elu1(k), _f64(v)
    left = (fq @ fk.T) @ vv
    right = fq @ (fk.T @ vv)
    o_rnn, S, _ = recurrence(fq, fk, vv, eps=eps)
    o_quad = masked_quadratic(fq, fk, vv, eps=eps)
    T, d = fq.shape
    return dict(
        associative=bool(np.allclose(left, right, rtol=1e-5, atol=1e-5)),
        qkT_shape=tuple((fq @ fk.T).shape),
        kTv_shape=tuple((fk.T @ vv).shape),
        recurrent_matches_quadratic=bool(np.allclose(o_rnn, o_quad, rtol=1e-5, atol=1e-4)),
        max_difference=float(np.abs(o_rnn - o_quad).max()),
        state_numel=int(S.size),
        kv_cache_numbers=kv_cache_numbers(T, d),
    )
