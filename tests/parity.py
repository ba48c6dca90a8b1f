"""Comparison helpers for the GPU-vs-oracle parity tests.

Tolerances for bf16 outputs: max |gpu - ref| <= 2e-2 and mean |gpu - ref| <= 2e-3 (elementwise over the
compared set); the sink gradient within 1e-2 relative.  For gradients whose exact values exceed the range
where a bf16 half-ulp stays below 2e-2 (|x| >= 8), the bound is widened by that half-ulp, 2^-8 |ref|,
because rounding the exact value to bf16 alone can exceed 2e-2 there; such elements are counted and reported.
"""
import numpy as np
import torch

MAX_ABS = 2e-2
MEAN_ABS = 2e-3
DSINK_REL = 1e-2


def to_np(x):
    if isinstance(x, torch.Tensor):
        return x.detach().float().cpu().numpy().astype(np.float64)
    return np.asarray(x, np.float64)


def compare(name, gpu, ref, max_abs=MAX_ABS, mean_abs=MEAN_ABS, bf16_halfulp=False):
    g, r = to_np(gpu), to_np(ref)
    assert g.shape == r.shape, (name, g.shape, r.shape)
    assert np.isfinite(g).all(), f"{name}: non-finite values"
    err = np.abs(g - r)
    bound = max_abs + (2.0 ** -8) * np.abs(r) if bf16_halfulp else np.full_like(r, max_abs)
    worst = float(err.max()) if err.size else 0.0
    mean = float(err.mean()) if err.size else 0.0
    widened = int(((err > max_abs) & (err <= bound)).sum()) if bf16_halfulp else 0
    msg = (f"{name}: max|err|={worst:.3e} mean|err|={mean:.3e} max|ref|={np.abs(r).max() if r.size else 0:.3f} "
           f"n={err.size} widened={widened}")
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
