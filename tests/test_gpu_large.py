"""Tensors of more than 2^31 elements (byte offsets past 2^32), against the
fp64 oracle: the offset of every (b, h) is 64-bit on every path, and these
tests reach sequences that start at, and lie wholly beyond, element 2^31.

* prefill and its gradients: the SSD-decay workload's sequence shape (T=8192,
  d=128, bf16, decay a = sigmoid(N(3, 1))) with 2100 sequences, B=4 x H=525:
  2.2e9 elements per input.  Element 2^31 is the first of sequence 2048, so
  sequences 2047 (the last below it), 2048 and 2099 (the last) are checked
  end to end, in the default plan, with 16-bit and with fp32 outputs and
  fp32 gradients.
* decode: the RFA decode step (RFF, D=64 pairs over d_h=64, d'=128, d_v=64,
  fp32) over 16400 sequences x 16 heads: a state of 2.15e9 floats.  The state
  element 2^31 is the first of sequence 16384; sequences 16383, 16384 and
  16399 start from states built by the oracle's recurrence (16 tokens each),
  the others from N(0, 1) values, which an output read from a wrong address
  would show.

Inputs are drawn on the GPU (one seeded torch CUDA generator; the values
checked are copied back to the host for the oracle).  Bars as for the other
workloads: 2e-2 of rms (bf16 inputs, with half an ulp of a bf16 output
allowed), 1e-4 for fp32.
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
B, H, T, D = 4, 525, 8192, 128
SEQS = (2047, 2048, 2099)   # flattened b * H + h


def _excess_err(got, ref):
    """max(|got - ref| - half an ulp of ref) / rms(ref), for bf16 outputs."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    ex = np.abs(got - ref) - HALF_ULP_BF16 * np.abs(ref)
    return float(max(ex.max(), 0.0) / np.sqrt(np.mean(ref * ref)))


def _host(x, n):
    """Sequence n (flattened b * H + h) of a [B, H, ...] device tensor, on the host."""
    return x[n // x.shape[1], n % x.shape[1]].cpu()


@pytest.fixture(scope="module")
def big_inputs():
    dev = gpu_device()
    assert B * H * T * D > 2 ** 31
    assert (SEQS[1] * T * D == 2 ** 31) and ((SEQS[1] - 1) * T * D < 2 ** 31)
    x = I.prefill_inputs(B, H, T, D, dtype="bf16", seed=0, decay="ssd", device=dev)
    torch.cuda.synchronize()
    yield x
    del x
    torch.cuda.empty_cache()


@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
def test_prefill_beyond_2pow31_elements(big_inputs, out_dtype):
    """16-bit outputs (half an ulp allowed) and fp32 outputs (the plain
    metric, max |gpu - oracle| / rms(oracle)); the output tensor itself has
    more than 2^31 elements either way."""
    x = big_inputs
    out, S, z = la.prefill(x.q, x.k, x.v, decay=x.decay, out_dtype=out_dtype)
    torch.cuda.synchronize()
    errs = {}
    for n in SEQS:
        o_ref, S_ref, z_ref = O.causal_linear_attention(
            _host(x.q, n)[None], _host(x.k, n)[None], _host(x.v, n)[None],
            decay=_host(x.decay, n)[None])
        got = _host(out, n).double().numpy()
        e_o = (_excess_err(got, o_ref[0]) if out_dtype == torch.bfloat16 else rel_err(got, o_ref[0]))
        errs[n] = (e_o, rel_err(_host(S, n), S_ref[0]), rel_err(_host(z, n), z_ref[0]))
    print("prefill 4x525x8192x128 (2.2e9 elements), out", out_dtype, "sequences", errs)
    del out, S, z
    torch.cuda.empty_cache()
    assert max(max(e) for e in errs.values()) < TOL["bf16"], errs


def test_prefill_backward_beyond_2pow31_elements(big_inputs):
    x = big_inputs
    dev = x.q.device
    g = torch.Generator(device=dev)
    g.manual_seed(1)
    do = torch.randn(x.q.shape, generator=g, device=dev).to(torch.bfloat16)
    got = la.prefill_backward(x.q, x.k, x.v, do, decay=x.decay)
    torch.cuda.synchronize()
    errs = {}
    for n in SEQS:
        ref = O.prefill_gradients_recurrent(
            _host(x.q, n)[None], _host(x.k, n)[None], _host(x.v, n)[None],
            _host(do, n)[None], decay=_host(x.decay, n)[None])
        errs[n] = {k: rel_err(_host(got[k], n), ref[k][0]) for k in ("dq", "dk", "dv", "ddecay")}
    print("backward 4x525x8192x128 (2.2e9 elements), sequences", errs)
    del got, do
    torch.cuda.empty_cache()
    assert max(max(e.values()) for e in errs.values()) < TOL["bf16"], errs


def test_decode_beyond_2pow31_state_elements():
    dev = gpu_device()
    N, Hd, dh, Dr, dv = 16400, 16, 64, 64, 64
    dp = 2 * Dr
    checked = (16383, 16384, 16399)
    assert N * Hd * dp * dv > 2 ** 31 and checked[1] * Hd * dp * dv == 2 ** 31
    W = I.rff_projection(Hd, Dr, dh, seed=3)
    gen = torch.Generator(device=dev)
    gen.manual_seed(5)
    S = torch.randn(N, Hd, dp, dv, generator=gen, device=dev)
    z = torch.randn(N, Hd, dp, generator=gen, device=dev)
    starts = {}
    for i, n in enumerate(checked):
        # a state the recurrence reaches: 16 RFA tokens from zero
        p = I.prefill_inputs(1, Hd, 16, dh, dtype="f32", seed=40 + i, decay="rfa",
                             unit_norm_qk=True)
        _, S0, z0 = O.causal_linear_attention(p.q, p.k, p.v, phi="rff", W=W, gate=p.gate)
        starts[n] = (S0[0], z0[0])
        S[n] = torch.as_tensor(S0[0], dtype=torch.float32, device=dev)
        z[n] = torch.as_tensor(z0[0], dtype=torch.float32, device=dev)
    st = I.rfa_decode_step_inputs(N, Hd, dh, dv, step=0, seed=3, device=dev)
    o = la.decode_step(st.q, st.k, st.v, S, z, phi="rff", W=W.to(dev), gate=st.gate)
    torch.cuda.synchronize()
    errs = {}
    for n in checked:
        o_ref, S_ref, z_ref = O.decode_step(st.q[n].cpu(), st.k[n].cpu(), st.v[n].cpu(),
                                            starts[n][0], starts[n][1], phi="rff", W=W,
                                            gate=st.gate[n].cpu())
        errs[n] = (rel_err(o[n].cpu(), o_ref), rel_err(S[n].cpu(), S_ref),
                   rel_err(z[n].cpu(), z_ref))
    print("decode 16400x16, d'=128, d_v=64 (2.15e9 state elements), sequences", errs)
    del S, z, o, st
    torch.cuda.empty_cache()
    assert max(max(e) for e in errs.values()) < TOL["f32"], errs
