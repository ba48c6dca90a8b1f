"""The gradient tolerance helper against real bf16 rounding (round to nearest even from fp32)."""
import numpy as np
import torch

from parity import MAX_ABS, bf16_halfulp, grad_bound, strict_summary


def test_halfulp_is_the_largest_rounding_error():
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(400000) * np.exp(rng.uniform(-8, 4, 400000))).astype(np.float32)
    r = torch.from_numpy(x).to(torch.bfloat16).float().numpy().astype(np.float64)
    err = np.abs(r - x.astype(np.float64))
    hu = bf16_halfulp(np.abs(x.astype(np.float64)))
    assert (err <= hu).all()
    assert (err / hu).max() > 0.99          # attained: it is the bound, not a loose one


def test_halfulp_values():
    got = bf16_halfulp(np.array([1.0, 1.99, 2.0, 7.99, 8.0, 15.9, 0.0]))
    assert got.tolist() == [2 ** -8, 2 ** -8, 2 ** -7, 2 ** -6, 2 ** -5, 2 ** -5, 0.0]


def test_grad_bound_covers_rounding_of_a_value_within_the_strict_bound():
    """A result within 2e-2 of ref, then rounded to bf16, always meets grad_bound(ref)."""
    rng = np.random.default_rng(1)
    ref = rng.uniform(-17, 17, 200000)
    x = (ref + rng.uniform(-MAX_ABS, MAX_ABS, ref.size)).astype(np.float32)
    r = torch.from_numpy(x).to(torch.bfloat16).float().numpy().astype(np.float64)
    assert (np.abs(r - ref) <= grad_bound(ref)).all()
    # and below |ref| = 2 the added term never exceeds 2^-8
    small = np.abs(ref) < 2 - MAX_ABS
    assert (grad_bound(ref[small]) <= MAX_ABS + 2 ** -8).all()


def test_strict_summary():
    err = np.array([0.0, 0.03, 0.01, 0.025])
    ref = np.array([1.0, 9.0, 3.0, -5.0])
    assert strict_summary(err, ref) == (2, 5.0, 0.03)
