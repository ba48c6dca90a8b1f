"""GPU forward parity against the fp64 oracle (bf16 outputs: max-abs 2e-2, mean-abs 2e-3)."""
import numpy as np
import pytest
import torch

import mimo_inputs as mi
import oracle
from parity import compare

pytestmark = pytest.mark.gpu


def _gpu():
    import global_gqa_attention_amd as ga

    if not torch.cuda.is_available():
        pytest.fail("a GPU is required for the -m gpu tests")
    return ga


def _run_fwd(ga, d):
    dev = "cuda"
    q, k, v = d["q"].to(dev), d["k"].to(dev), d["v"].to(dev)
    sink = None if d["sink"] is None else d["sink"].to(dev)
    cu = d["cu_seqlens"].to(dev)
    out, lse = ga.fwd(q, k, v, sink, cu, max(d["lengths"] + [1]), d["window"], d["rope_base"])
    torch.cuda.synchronize()
    return out.cpu(), lse.cpu()


def _case(lengths, hq, hkv, window, base, sink, seed):
    d = mi.make_layer(lengths, hq, hkv, seed, sink)
    d.update(window=window, rope_base=base)
    return d


def test_fwd_swa_512_full():
    """One SWA layer, 512 tokens, 64/8 heads, window 128, sink, base 1e4, seed 0: every output."""
    ga = _gpu()
    d = mi.swa_512()
    print("case swa_512", flush=True)
    out, lse = _run_fwd(ga, d)
    ro, rl = oracle.prefill(d["q"], d["k"], d["v"], d["sink"], d["cu_seqlens"], 128, 1e4)
    compare("out", out, ro)
    compare("lse", lse, rl)


@pytest.mark.parametrize("lengths,hq,hkv,window,base,sink", [
    ([1, 5, 63, 64, 65, 129, 200, 0, 300], 64, 8, 128, 1e4, True),
    ([1, 5, 63, 64, 65, 129, 200, 0, 300], 64, 4, -1, 1e7, False),
    ([17, 130, 1], 64, 4, -1, 1e7, True),
    ([70, 33, 257], 16, 8, 0, 1e4, True),
    ([70, 33, 257], 16, 16, 3, 1e4, False),
    ([100, 29], 12, 4, 40, 1e4, True),
    ([100, 29], 8, 1, -1, 1e4, False),
])
def test_fwd_ragged_small(lengths, hq, hkv, window, base, sink):
    ga = _gpu()
    d = _case(lengths, hq, hkv, window, base, sink, 5)
    print(f"case lengths={lengths} hq={hq} hkv={hkv} window={window}", flush=True)
    out, lse = _run_fwd(ga, d)
    ro, rl = oracle.prefill(d["q"], d["k"], d["v"], d["sink"], d["cu_seqlens"], window, base)
    compare("out", out, ro)
    compare("lse", lse, rl)


def test_fwd_sink_minus_inf_equals_no_sink():
    ga = _gpu()
    d = _case([300, 45], 64, 8, 128, 1e4, True, 6)
    d2 = dict(d)
    d2["sink"] = torch.full((64,), float("-inf"))
    a, la = _run_fwd(ga, d2)
    d3 = dict(d)
    d3["sink"] = None
    b, lb = _run_fwd(ga, d3)
    assert torch.equal(a, b) and torch.equal(la, lb)


def test_fwd_deterministic():
    ga = _gpu()
    d = _case([513, 1000], 64, 4, -1, 1e7, False, 7)
    a, la = _run_fwd(ga, d)
    b, lb = _run_fwd(ga, d)
    assert torch.equal(a, b) and torch.equal(la, lb)


def _sample_rows(lengths, hq, n, seed):
    rng = np.random.default_rng(seed)
    T = sum(lengths)
    starts = np.concatenate([[0], np.cumsum(lengths)])
    toks = set(rng.integers(0, T, n).tolist())
    for b, L in enumerate(lengths):       # first, last and a window edge of every sequence
        if L:
            toks.update([starts[b], starts[b] + L - 1, starts[b] + min(L - 1, 128), starts[b] + min(L - 1, 129)])
    toks = np.array(sorted(toks))
    heads = rng.integers(0, hq, len(toks))
    return toks * hq + heads


def test_fwd_global_2x4096_full():
    """Global layer, 2 x 4096 tokens, 64/4 heads, base 1e7, seed 1: every output row against the oracle (about
    690 GFLOP of fp64 work on the host)."""
    ga = _gpu()
    d = mi.global_2x4096()
    print("case global_2x4096 (every row)", flush=True)
    out, lse = _run_fwd(ga, d)
    ro, rl = oracle.prefill(d["q"], d["k"], d["v"], None, d["cu_seqlens"], -1, 1e7)
    compare("out", out, ro)
    compare("lse", lse, rl)


def test_fwd_thd_32k_sampled():
    """32768-token THD batch (16 lengths in [1024, 2048] + pad), SWA and global layers, seed 2: sampled rows."""
    ga = _gpu()
    both = mi.thd_32k()
    for name in ("swa", "glb"):
        d = both[name]
        print(f"case thd_32k {name}", flush=True)
        out, lse = _run_fwd(ga, d)
        rows = _sample_rows(d["lengths"], 64, 800, 2)
        ro, rl = oracle.prefill_rows(d["q"], d["k"], d["v"], d["sink"], d["cu_seqlens"], d["window"],
                                     d["rope_base"], rows)
        compare(f"{name} out", out.reshape(-1, 128)[rows], ro)
        compare(f"{name} lse", lse.T.reshape(-1)[rows], rl)


@pytest.mark.parametrize("lengths,hkv,window,base", [
    ([1, 5, 63, 64, 65, 129, 200, 0, 300], 8, 128, 1e4),
    ([17, 130, 1], 4, -1, 1e7),
])
def test_fwd_q_rot_output(lengths, hkv, window, base):
    """The optional rotated-q output: RoPE applied at each token's position in its own sequence (the oracle's
    fp64 rotation, to one bf16 rounding), and out / lse unchanged by asking for it."""
    ga = _gpu()
    d = _case(lengths, 64, hkv, window, base, window >= 0, 8)
    print(f"case q_rot lengths={lengths} window={window}", flush=True)
    dev = "cuda"
    q, k, v = d["q"].to(dev), d["k"].to(dev), d["v"].to(dev)
    sink = None if d["sink"] is None else d["sink"].to(dev)
    cu = d["cu_seqlens"].to(dev)
    maxl = max(lengths)
    qr = torch.full_like(q, float("nan"))
    o1, l1 = ga.fwd(q, k, v, sink, cu, maxl, window, base, q_rot=qr)
    o2, l2 = ga.fwd(q, k, v, sink, cu, maxl, window, base)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    T = sum(lengths)
    pos = np.concatenate([np.arange(n) for n in lengths]).astype(np.int32)
    ref = oracle.rope(d["q"].reshape(T * 64, 192), np.repeat(pos, 64), base)
    got = qr.cpu().float().numpy().reshape(T * 64, 192)
    err = np.abs(got - ref)
    assert np.isfinite(got).all()
    assert (err <= 2.0 ** -8 * np.abs(ref) + 1e-6).all(), float(err.max())


@pytest.mark.parametrize("window,hkv,sink", [(128, 8, True), (-1, 4, False)])
def test_fwd_many_sequences(window, hkv, sink):
    """More than 64 sequences (the work-item lookup reads cu_seqlens 64 at a time): 100 ragged sequences,
    lengths 0..40, every output."""
    ga = _gpu()
    rng = np.random.default_rng(21)
    lengths = [int(x) for x in rng.integers(0, 41, 100)]
    d = _case(lengths, 16, hkv, window, 1e4, sink, 13)
    print(f"case many sequences window={window}", flush=True)
    out, lse = _run_fwd(ga, d)
    ro, rl = oracle.prefill(d["q"], d["k"], d["v"], d["sink"], d["cu_seqlens"], window, 1e4)
    compare("out", out, ro)
    compare("lse", lse, rl)
