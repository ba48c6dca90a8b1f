"""GPU parity of the prefill over a cached prefix (mimo_attn_prefill_cached) against the fp64 oracle: bf16
outputs within max-abs 2e-2 and mean-abs 2e-3, LSE likewise."""
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


def _dev(x):
    return None if x is None else x.to("cuda")


def _run(ga, d, window, base):
    out, lse = ga.prefill_cached(_dev(d["q"]), _dev(d["k"]), _dev(d["v"]), _dev(d["k_cache"]), _dev(d["v_cache"]),
                                 _dev(d["sink"]), _dev(d["cu_seqlens"]), _dev(d["cu_cache"]), _dev(d["positions"]),
                                 max(d["lengths"] + [1]), d["max_position"], window, base)
    torch.cuda.synchronize()
    return out.cpu(), lse.cpu()


def _oracle(d, window, base, rows=None):
    return oracle.prefill_cached_rows(d["q"], d["k"], d["v"], d["k_cache"], d["v_cache"], d["cu_seqlens"],
                                      d["cu_cache"], d["positions"], d["sink"], window, base, rows=rows)


@pytest.mark.parametrize("chunks,prefixes,keep,hq,hkv,window,base,sink", [
    ([1, 5, 63, 64, 65, 129, 0, 200], [0, 300, 17, 128, 1000, 5, 40, 64], None, 64, 4, -1, 1e7, False),
    ([1, 5, 63, 64, 65, 129, 0, 200], [0, 300, 17, 128, 1000, 5, 40, 64], 128, 64, 8, 128, 1e4, True),
    ([33, 257, 8], [500, 0, 7], None, 16, 8, 0, 1e4, True),
    ([100, 29], [60, 3], 20, 12, 4, 20, 1e4, True),
    ([70, 1, 16], [130000, 4096, 2], 50, 16, 2, 50, 1e7, True),
    ([40, 40], [0, 0], None, 8, 1, -1, 1e4, False),
])
def test_prefill_cached_matches_oracle(chunks, prefixes, keep, hq, hkv, window, base, sink):
    ga = _gpu()
    d = mi.make_cached(chunks, prefixes, hq, hkv, 6, sink, keep)
    print(f"case chunks={chunks} prefixes={prefixes} keep={keep} hq={hq} hkv={hkv} window={window}", flush=True)
    out, lse = _run(ga, d, window, base)
    T = out.shape[0]
    ro, rl = _oracle(d, window, base)
    compare("out", out, ro.reshape(T, hq, -1))
    compare("lse", lse, rl.reshape(T, hq).T)


@pytest.mark.parametrize("window,base,sink", [(128, 1e4, True), (-1, 1e7, False)])
def test_prefill_cached_without_cache_equals_fwd(window, base, sink):
    """No cache rows and positions 0: the same rows as the plain forward, bit for bit."""
    ga = _gpu()
    lengths = [1, 90, 0, 300, 33]
    d = mi.make_layer(lengths, 64, 8 if window >= 0 else 4, 7, sink)
    print(f"case lengths={lengths} window={window}", flush=True)
    hkv = d["k"].shape[1]
    q, k, v, cu = _dev(d["q"]), _dev(d["k"]), _dev(d["v"]), _dev(d["cu_seqlens"])
    s = _dev(d["sink"])
    o1, l1 = ga.fwd(q, k, v, s, cu, max(lengths), window, base)
    kc = torch.zeros((0, hkv, 192), dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros((0, hkv, 128), dtype=torch.bfloat16, device="cuda")
    zc = torch.zeros(len(lengths) + 1, dtype=torch.int32, device="cuda")
    zp = torch.zeros(len(lengths), dtype=torch.int32, device="cuda")
    o2, l2 = ga.prefill_cached(q, k, v, kc, vc, s, cu, zc, zp, max(lengths), max(lengths), window, base)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1, l2)


@pytest.mark.parametrize("layer", ["glb", "swa"])
def test_prefill_cached_chunked_16_sampled(layer):
    """The 16-sequence chunked prefill (prefixes 2048..8192, chunks 1024..2048) at full size: 96 sampled
    (token, head) rows against the oracle, and every output finite."""
    ga = _gpu()
    d = mi.chunked_16()[layer]
    print(f"case chunked_16 {layer}", flush=True)
    out, lse = _run(ga, d, d["window"], d["rope_base"])
    assert torch.isfinite(out.float()).all() and torch.isfinite(lse).all()
    T, hq = out.shape[0], out.shape[1]
    g = np.random.default_rng(8)
    rows = np.sort(g.choice(T * hq, 96, replace=False))
    cu = d["cu_seqlens"].tolist()
    ends = np.array(cu[1:]) - 1                     # each sequence's last token, the longest key span
    rows = np.unique(np.concatenate([rows, ends[:8] * hq + 5]))
    ro, rl = _oracle(d, d["window"], d["rope_base"], rows)
    t, h = rows // hq, rows % hq
    compare("out", out[t, h], ro)
    compare("lse", lse[h, t], rl)
