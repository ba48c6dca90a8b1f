"""Comparison helpers for the GPU-vs-oracle parity tests.

Tolerances for bf16 outputs: max |gpu - ref| <= 2e-2 and mean |gpu - ref| <= 2e-3 (elementwise over the
compared set); the sink gradient within 1e-2 relative.

Gradients (dq, dk, dv) are bf16 numbers whose exact values reach 10-17 on the first keys of a long causal
sequence, where one bf16 half-ulp (2^-4 in [8, 16)) exceeds 2e-2 by itself.  Their bound is the stated 2e-2
on the unrounded result plus the largest error of rounding a value within 2e-2 of the exact one to bf16:
    |gpu - ref| <= 2e-2 + halfulp(|ref| + 2e-2),   halfulp(y) = 2^(floor(log2 y) - 8)
(bf16 keeps 8 significant bits, so a number in [2^e, 2^(e+1)) rounds with an error of at most 2^(e-8)).
Below |ref| = 2 the added term is at most 2^-8.  Every compare also counts the elements beyond the strict
2e-2 and records the smallest |ref| among them; the session summary (conftest.py) prints those counts.
"""
import numpy as np
import torch

MAX_ABS = 2e-2
MEAN_ABS = 2e-3
DSINK_REL = 1e-2

# (tensor name, elements compared, elements beyond the strict bound, smallest |ref| among them, largest error)
STRICT_LOG = []


def to_np(x):
    if isinstance(x, torch.Tensor):
        return x.detach().float().cpu().numpy().astype(np.float64)
    return np.asarray(x, np.float64)


def bf16_halfulp(y):
    """Largest error of rounding a number of magnitude y to bf16 (round to nearest even): 2^(floor(log2 y) - 8)
    for y > 0, 0 for y = 0."""
    y = np.asarray(y, np.float64)
    _, e = np.frexp(y)               # y = m 2^e with m in [0.5, 1): floor(log2 y) = e - 1
    return np.where(y > 0, np.ldexp(1.0, e - 9), 0.0)


def grad_bound(ref, max_abs=MAX_ABS):
    """Elementwise bound for a bf16 gradient: the stated max_abs plus the bf16 rounding of a value within
    max_abs of ref."""
    return max_abs + bf16_halfulp(np.abs(ref) + max_abs)


def strict_summary(err, ref, max_abs=MAX_ABS):
    """(count beyond max_abs, smallest |ref| among them or None, largest error)."""
    over = err > max_abs
    n = int(over.sum())
    return n, (float(np.abs(ref[over]).min()) if n else None), (float(err.max()) if err.size else 0.0)


def compare(name, gpu, ref, max_abs=MAX_ABS, mean_abs=MEAN_ABS, grad=False):
    """Elementwise parity of a bf16 output (grad=True: the gradient bound above)."""
    g, r = to_np(gpu), to_np(ref)
    assert g.shape == r.shape, (name, g.shape, r.shape)
    assert np.isfinite(g).all(), f"{name}: non-finite values"
    err = np.abs(g - r)
    bound = grad_bound(r, max_abs) if grad else np.full_like(r, max_abs)
    worst = float(err.max()) if err.size else 0.0
    mean = float(err.mean()) if err.size else 0.0
    n_over, min_ref, _ = strict_summary(err, r, max_abs)
    if grad:
        STRICT_LOG.append((name.split()[0], err.size, n_over, min_ref, worst))
    msg = (f"{name}: max|err|={worst:.3e} mean|err|={mean:.3e} max|ref|={np.abs(r).max() if r.size else 0:.3f} "
           f"n={err.size} strict>{max_abs:g}: {n_over}" + (f" (min|ref| {min_ref:.3f})" if n_over else ""))
    print(msg, flush=True)
    assert (err <= bound).all(), msg
    assert mean <= mean_abs, msg
    return worst, mean


def compare_rel(name, gpu, ref, rel=DSINK_REL):
    g, r = to_np(gpu), to_np(ref)
    denom = np.maximum(np.abs(r), 1e-30)
    relerr = np.abs(g - r) / denom
    nrel = np.linalg.norm(g - r) / max(np.linalg.norm(r), 1e-30)
    msg = f"{name}: max rel={relerr.max():.3e} norm rel={nrel:.3e} values={np.round(r[:4], 4)}"
    print(msg, flush=True)
    assert (relerr <= rel).all(), msg
