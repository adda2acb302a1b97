"""The measured prefill workloads at their full sizes, in the launch
configuration the benchmark times (default chunk and segment plan, output in
the input type), against the fp64 oracle.

* elu+1 prefill, B=4, H=8, T=2048, d=64, bf16: every output and the final
  state, element by element.
* SSD-decay prefill, B=2, H=16, T=8192, d=128, bf16: four (b, h) sequences
  end to end through the oracle's recurrence, sampled positions of every
  other sequence through the definition, and every final state through its
  closed form.
* long-context prefill, B=1, H=8, T=102400, d=128, bf16 scaled by 1/sqrt(2):
  two heads end to end, sampled positions (chunk, sub-segment and segment
  edges among them) of the other six, every final state in closed form; and
  the same workload with the normaliser-free read-out, two heads end to end,
  and in the non-causal form, every output.
* mLSTM gates on the long-context shape (identity features, sigmoid forget
  and exponential input gates, max(|q.z|, 1) read-out): two heads end to
  end, sampled positions of the other six, every final state (S', z', m) in
  closed form.

A 16-bit output is the fp32 result rounded to nearest even, so each element
may sit up to half an ulp (2^-8 relative, worst case in a binade) from the
oracle beyond the compute error; the metric subtracts that allowance before
dividing by rms(oracle).  Bar: 2e-2 (bf16 inputs).

The long-context and SSD-decay workloads also run with fp32 outputs, where
no output rounding intervenes: there the bar applies to the plain metric,
max |gpu - oracle| / rms(oracle), on the end-to-end heads, the sampled
positions and the final states, and to the worst single position measured
against its own rms.
"""
import numpy as np
import pytest
import torch

import fixed_state_sequence_amd as la
from fixed_state_sequence_amd import inputs as I
from oracle import linattn_oracle as O
from conftest import rel_err, TOL, gpu_device

pytestmark = pytest.mark.gpu

HALF_ULP_BF16 = 2.0 ** -8


def excess_err(got, ref, rms):
    """max(|got - ref| - half an ulp of ref) / rms, for outputs rounded to bf16."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    ex = np.abs(got - ref) - HALF_ULP_BF16 * np.abs(ref)
    return float(max(ex.max(), 0.0) / rms)


def rms(x):
    return float(np.sqrt(np.mean(np.asarray(x, dtype=np.float64) ** 2)))


def run_workload(name, normalize=True, causal=True, out_dtype=torch.bfloat16):
    """Inputs drawn on the host (seed 0) and the prefill as the benchmark runs it."""
    dev = gpu_device()
    x = I.workload_inputs(name, seed=0)
    B, H, T, d = x.q.shape
    desc = la.make_desc(B, H, T, d, d, la._lib.LA_BF16,
                        decay=x.decay)
    chunk, segments, path = la.prefill_plan(desc)
    assert path == 1
    g = lambda t: None if t is None else t.to(dev)
    out, S, z = la.prefill(g(x.q), g(x.k), g(x.v), decay=g(x.decay), normalize=normalize,
                           causal=causal, out_dtype=out_dtype)
    torch.cuda.synchronize()
    assert out.dtype == out_dtype
    print(name, "plan", chunk, segments)
    return x, out.double().cpu().numpy(), S.cpu().numpy(), z.cpu().numpy(), (chunk, segments)


def sample_positions(T, chunk, segments, n_random, rng):
    cps = -(-T // chunk) // segments * chunk        # tokens per segment (full segments)
    edges = {0, 1, chunk - 1, chunk, T - 1, T - 2}
    for s in range(1, min(segments, 4)):
        for off in (-1, 0, 1):
            edges.add(s * cps + off)
            edges.add(s * cps - cps // 2 + off)     # sub-segment edge inside segment s-1
    edges |= set(int(t) for t in rng.integers(0, T, n_random))
    return sorted(t for t in edges if 0 <= t < T)


def plain_err(got, ref, rms):
    """max |got - ref| / rms, for fp32 outputs."""
    return float(np.abs(np.asarray(got, np.float64) - np.asarray(ref, np.float64)).max() / rms)


def worst_per_position(got, ref):
    """The worst position's max |got - ref| over its own rms(ref)."""
    return float((np.abs(got - ref).max(axis=-1) / np.sqrt(np.mean(ref ** 2, axis=-1))).max())


def check_sampled(x, out, S, z, full, others, positions, rms_ref, metric=None):
    """Outputs at `positions` of the (b, h) pairs in `others` by the definition,
    and every final state by its closed form.  Also returns the worst sampled
    position's error over its own rms."""
    metric = metric or excess_err
    B, H, T, _ = x.q.shape
    alpha = None if x.decay is None else O._f64(x.decay)
    worst = pos_worst = 0.0
    for b, h in others:
        fq = O.features(x.q[b, h])
        fk = O.features(x.k[b, h])
        v = O._f64(x.v[b, h])
        a = None if alpha is None else alpha[b, h]
        for t in positions:
            ref = O.output_at(fq[t], fk, v, t, alpha=a)
            worst = max(worst, metric(out[b, h, t], ref, rms_ref))
            pos_worst = max(pos_worst, worst_per_position(out[b, h, t][None], ref[None]))
    s_worst = z_worst = 0.0
    for b in range(B):
        for h in range(H):
            if (b, h) in full:
                continue
            S_ref, z_ref = O.final_state(O.features(x.k[b, h]), x.v[b, h],
                                         alpha=None if alpha is None else alpha[b, h])
            s_worst = max(s_worst, rel_err(S[b, h], S_ref))
            z_worst = max(z_worst, rel_err(z[b, h], z_ref))
    return worst, s_worst, z_worst, pos_worst


def test_elu_prefill_b4_h8_t2048_d64_full():
    x, out, S, z, _ = run_workload("elu_prefill_b4_h8_t2048_d64")
    o_ref, S_ref, z_ref = O.causal_linear_attention(x.q, x.k, x.v)
    r = rms(o_ref)
    e = (excess_err(out, o_ref, r), rel_err(S, S_ref), rel_err(z, z_ref))
    print("elu prefill 4x8x2048x64", e, "plain max|err|/rms", rel_err(out, o_ref))
    assert max(e) < TOL["bf16"], e


def test_ssd_prefill_b2_h16_t8192_d128_sampled():
    x, out, S, z, (chunk, segments) = run_workload("ssd_prefill_b2_h16_t8192_d128")
    B, H, T, _ = x.q.shape
    full = [(0, 0), (0, 15), (1, 7), (1, 15)]
    bs, hs = [p[0] for p in full], [p[1] for p in full]
    o_ref, S_ref, z_ref = O.causal_linear_attention(x.q[bs, hs], x.k[bs, hs], x.v[bs, hs],
                                                    decay=x.decay[bs, hs])
    r = rms(o_ref)
    e_full = (excess_err(out[bs, hs], o_ref, r), rel_err(S[bs, hs], S_ref),
              rel_err(z[bs, hs], z_ref))
    rng = np.random.default_rng(3)
    others = [(int(b), int(h)) for b, h in zip(rng.integers(0, B, 4), rng.integers(0, H, 4))]
    pos = sample_positions(T, chunk, segments, 8, rng)
    e_s = check_sampled(x, out, S, z, full, others, pos, r)
    print("ssd prefill 2x16x8192x128 full", e_full, "sampled", e_s)
    assert max(e_full + e_s[:3]) < TOL["bf16"], (e_full, e_s)


def test_long_prefill_b1_h8_t102400_d128_sampled():
    x, out, S, z, (chunk, segments) = run_workload("long_prefill_b1_h8_t102400_d128")
    B, H, T, _ = x.q.shape
    full = [(0, 0), (0, 5)]
    hs = [p[1] for p in full]
    o_ref, S_ref, z_ref = O.causal_linear_attention(x.q[0, hs], x.k[0, hs], x.v[0, hs])
    r = rms(o_ref)
    got = out[0, hs]
    e_full = (excess_err(got, o_ref, r), rel_err(S[0, hs], S_ref), rel_err(z[0, hs], z_ref))
    # the outputs shrink like 1/sqrt(t): also report the worst error of a position
    # relative to that position's own rms
    per_pos = (np.abs(got - o_ref).max(axis=-1) /
               np.sqrt(np.mean(o_ref ** 2, axis=-1))).max()
    rng = np.random.default_rng(4)
    others = [(0, 1), (0, 2), (0, 7)]
    pos = sample_positions(T, chunk, segments, 12, rng)
    e_s = check_sampled(x, out, S, z, full, others, pos, r)
    print("long prefill 1x8x102400x128 full", e_full, "sampled", e_s,
          "worst per-position", per_pos)
    assert max(e_full + e_s[:3]) < TOL["bf16"], (e_full, e_s)


# fp32 outputs: no output rounding, so the bar applies to the plain metric,
# max |gpu - oracle| / rms(oracle) over the checked tensor, and to the worst
# single position measured against that position's own rms.

def test_long_prefill_b1_h8_t102400_d128_fp32_out_plain_metric():
    x, out, S, z, (chunk, segments) = run_workload("long_prefill_b1_h8_t102400_d128",
                                                   out_dtype=torch.float32)
    B, H, T, _ = x.q.shape
    full = [(0, 1), (0, 6)]
    hs = [p[1] for p in full]
    o_ref, S_ref, z_ref = O.causal_linear_attention(x.q[0, hs], x.k[0, hs], x.v[0, hs])
    r = rms(o_ref)
    got = out[0, hs]
    e_full = (plain_err(got, o_ref, r), rel_err(S[0, hs], S_ref), rel_err(z[0, hs], z_ref))
    per_pos = worst_per_position(got, o_ref)
    rng = np.random.default_rng(14)
    others = [(0, 0), (0, 3), (0, 4)]
    pos = sample_positions(T, chunk, segments, 12, rng)
    e_s = check_sampled(x, out, S, z, full, others, pos, r, metric=plain_err)
    print("long prefill fp32 out: full", e_full, "worst per-position", per_pos, "sampled", e_s)
    assert max(e_full) < TOL["bf16"], e_full
    assert max(e_s) < TOL["bf16"], e_s
    assert per_pos < TOL["bf16"], per_pos


def test_ssd_prefill_b2_h16_t8192_d128_fp32_out_plain_metric():
    x, out, S, z, (chunk, segments) = run_workload("ssd_prefill_b2_h16_t8192_d128",
                                                   out_dtype=torch.float32)
    B, H, T, _ = x.q.shape
    full = [(0, 3), (0, 12), (1, 0), (1, 9)]
    bs, hs = [p[0] for p in full], [p[1] for p in full]
    o_ref, S_ref, z_ref = O.causal_linear_attention(x.q[bs, hs], x.k[bs, hs], x.v[bs, hs],
                                                    decay=x.decay[bs, hs])
    r = rms(o_ref)
    got = out[bs, hs]
    e_full = (plain_err(got, o_ref, r), rel_err(S[bs, hs], S_ref), rel_err(z[bs, hs], z_ref))
    per_pos = worst_per_position(got, o_ref)
    rng = np.random.default_rng(15)
    others = [(int(b), int(h)) for b, h in zip(rng.integers(0, B, 4), rng.integers(0, H, 4))]
    pos = sample_positions(T, chunk, segments, 8, rng)
    e_s = check_sampled(x, out, S, z, full, others, pos, r, metric=plain_err)
    print("ssd prefill fp32 out: full", e_full, "worst per-position", per_pos, "sampled", e_s)
    assert max(e_full) < TOL["bf16"], e_full
    assert max(e_s) < TOL["bf16"], e_s
    assert per_pos < TOL["bf16"], per_pos


def test_long_prefill_unnormalised_two_heads():
    """The long-context workload with the normaliser-free read-out, in the
    benchmark's launch configuration: two heads end to end against the
    oracle's numerator, and their final states."""
    x, out, S, z, _ = run_workload("long_prefill_b1_h8_t102400_d128", normalize=False)
    hs = [3, 6]
    o_ref, S_ref, z_ref = O.causal_linear_attention(x.q[0, hs], x.k[0, hs], x.v[0, hs],
                                                    normalize=False)
    r = rms(o_ref)
    e = (excess_err(out[0, hs], o_ref, r), rel_err(S[0, hs], S_ref), rel_err(z[0, hs], z_ref))
    print("long prefill unnormalised", e)
    assert max(e) < TOL["bf16"], e


def test_long_prefill_noncausal_full():
    """The long-context workload in the non-causal form, in the benchmark's
    launch configuration: every output and every final state."""
    x, out, S, z, _ = run_workload("long_prefill_b1_h8_t102400_d128", causal=False)
    o_ref, S_ref, z_ref = O.noncausal_linear_attention(x.q, x.k, x.v)
    r = rms(o_ref)
    e = (excess_err(out, o_ref, r), rel_err(S, S_ref), rel_err(z, z_ref))
    print("long prefill non-causal", e, "plain", rel_err(out, o_ref))
    assert max(e) < TOL["bf16"], e



def test_mlstm_prefill_b1_h8_t102400_d128_sampled():
    dev = gpu_device()
    x = I.workload_inputs("mlstm_prefill_b1_h8_t102400_d128", seed=0)
    B, H, T, d = x.q.shape
    desc = la.make_desc(B, H, T, d, d, la._lib.LA_BF16, phi="identity", igate=x.igate,
                        fgate=x.fgate, normalize="max1", stab=torch.empty(1))
    chunk, segments, path = la.prefill_plan(desc)
    assert path == 1
    g = lambda t: t.to(dev)
    out, S, z, m = la.prefill(g(x.q), g(x.k), g(x.v), phi="identity", igate=g(x.igate),
                              fgate=g(x.fgate), normalize="max1")
    torch.cuda.synchronize()
    assert out.dtype == torch.bfloat16
    out, S, z, m = (out.double().cpu().numpy(), S.cpu().numpy(), z.cpu().numpy(),
                    m.cpu().double().numpy())
    hs = [2, 5]
    o_ref, S_ref, z_ref, m_ref = O.mlstm_recurrence(x.q[0, hs], x.k[0, hs], x.v[0, hs],
                                                    x.igate[0, hs], x.fgate[0, hs])
    r = rms(o_ref)
    e_full = (excess_err(out[0, hs], o_ref, r), rel_err(S[0, hs], S_ref),
              rel_err(z[0, hs], z_ref), float(np.abs(m[0, hs] - m_ref).max()))
    rng = np.random.default_rng(6)
    pos = sample_positions(T, chunk, segments, 12, rng)
    worst = 0.0
    for h in (0, 1, 3, 4, 6, 7):
        for t in pos:
            ref = O.mlstm_output_at(x.q[0, h, t], x.k[0, h], x.v[0, h], t, x.igate[0, h],
                                    x.fgate[0, h])
            worst = max(worst, excess_err(out[0, h, t], ref, r))
    Sc, zc, mc = O.mlstm_final_state(x.k[0], x.v[0], x.igate[0], x.fgate[0])
    e_state = (rel_err(S[0], Sc), rel_err(z[0], zc), float(np.abs(m[0] - mc).max()))
    print("mlstm prefill 1x8x102400x128 full", e_full, "sampled", worst, "states", e_state)
    assert max(e_full[:3]) < TOL["bf16"] and e_full[3] < 1e-3, e_full
    assert worst < TOL["bf16"], worst
    assert max(e_state[:2]) < TOL["bf16"] and e_state[2] < 1e-3, e_state
