"""Seeded input generators: deterministic, right shapes/dtypes/distributions."""
import torch

from fixed_state_sequence_amd import inputs as I


def test_prefill_inputs_deterministic_and_shaped():
    a = I.prefill_inputs(2, 3, 50, 16, dtype="bf16", seed=5, decay="ssd")
    b = I.prefill_inputs(2, 3, 50, 16, dtype="bf16", seed=5, decay="ssd")
    for x, y in [(a.q, b.q), (a.k, b.k), (a.v, b.v), (a.decay, b.decay)]:
        assert torch.equal(x, y)
    assert a.q.shape == (2, 3, 50, 16) and a.q.dtype == torch.bfloat16
    assert a.decay.shape == (2, 3, 50) and a.decay.dtype == torch.float32
    assert (a.decay > 0).all() and (a.decay < 1).all()
    c = I.prefill_inputs(2, 3, 50, 16, dtype="bf16", seed=6)
    assert not torch.equal(a.q, c.q)


def test_bf16_rounding_is_nearest_even():
    # 1 + 2^-8 lies exactly between two bf16 values (1 and 1 + 2^-7): ties go to even (1)
    x = torch.tensor([1 + 2 ** -8, 1 + 3 * 2 ** -8, 1 + 2 ** -8 + 2 ** -20])
    y = x.to(torch.bfloat16).float()
    assert y.tolist() == [1.0, 1 + 2 ** -6, 1 + 2 ** -7]


def test_long_prefill_scale_and_ssd_decay_distribution():
    w = I.prefill_inputs(1, 2, 4096, 32, dtype="bf16", seed=0, scale=2 ** -0.5)
    std = w.q.float().std().item()
    assert abs(std - 2 ** -0.5) < 0.02
    s = I.prefill_inputs(1, 4, 8192, 8, dtype="bf16", seed=0, decay="ssd")
    x = torch.logit(s.decay.double())
    assert abs(x.mean().item() - 3.0) < 0.05 and abs(x.std().item() - 1.0) < 0.05


def test_rfa_decode_inputs_unit_norm_and_per_step():
    s0 = I.rfa_decode_step_inputs(8, 4, 64, step=0)
    s1 = I.rfa_decode_step_inputs(8, 4, 64, step=1)
    assert torch.allclose(s0.q.double().norm(dim=-1), torch.ones(8, 4, dtype=torch.float64), atol=1e-6)
    assert torch.allclose(s0.k.double().norm(dim=-1), torch.ones(8, 4, dtype=torch.float64), atol=1e-6)
    assert not torch.equal(s0.q, s1.q)
    assert torch.equal(s0.v, I.rfa_decode_step_inputs(8, 4, 64, step=0).v)
    assert ((s0.gate > 0) & (s0.gate < 1)).all()
    W = I.rff_projection(16, 64, 64, seed=0)
    assert W.shape == (16, 64, 64)


def test_worked_example_inputs():
    q, k, v = I.tiny_worked_example()
    assert q.shape == k.shape == v.shape == (8, 4) and q.dtype == torch.float32
    w = I.workload_inputs("tiny_causal_t8_d4")
    assert torch.equal(w.q[0, 0], q)
