"""GPU decode parity against the fp64 oracle (bf16 outputs: max-abs 2e-2, mean-abs 2e-3)."""
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


def _run(ga, d, max_len):
    dev = "cuda"
    g = lambda x: None if x is None else x.to(dev)  # noqa: E731
    out = ga.decode(g(d["q"]), g(d["k_new"]), g(d["v_new"]), g(d["k_cache"]), g(d["v_cache"]), g(d["cu_cache"]),
                    g(d["positions"]), g(d["sink"]), max_len, d["window"], d["rope_base"])
    torch.cuda.synchronize()
    return out.cpu()


def test_decode_swa_ring_full():
    """Batch 64, 128-entry ring + current token, 8 KV heads, sink, base 1e4, seed 3: every output."""
    ga = _gpu()
    d = mi.decode_swa()
    out = _run(ga, d, 128)
    ref, _ = oracle.decode_rows(d["q"], d["k_new"], d["v_new"], d["k_cache"], d["v_cache"], d["cu_cache"],
                                d["positions"], d["sink"], d["window"], d["rope_base"])
    compare("out", out.reshape(-1, 128), ref)


@pytest.mark.parametrize("lens,hkv,window,sink", [
    ([0, 1, 31, 32, 33, 1000, 2049, 5000], 4, -1, False),
    ([0, 1, 31, 32, 33, 1000, 2049, 5000], 8, 128, True),
    ([3000, 7, 129, 128, 127], 8, 50, True),
    ([4096, 1], 1, -1, True),
])
def test_decode_ragged_full(lens, hkv, window, sink):
    ga = _gpu()
    g = torch.Generator().manual_seed(12)
    B, hq = len(lens), 64
    r = lambda *s: torch.randn(*s, generator=g).to(torch.bfloat16)  # noqa: E731
    cu = mi.cu_from_lengths(lens)
    d = dict(q=r(B, hq, 192), k_new=r(B, hkv, 192), v_new=r(B, hkv, 128), k_cache=r(int(cu[-1]), hkv, 192),
             v_cache=r(int(cu[-1]), hkv, 128), cu_cache=cu,
             positions=torch.tensor([n + 17 for n in lens], dtype=torch.int32),
             sink=torch.randn(hq, generator=g) if sink else None, window=window, rope_base=1e4)
    print(f"case lens={lens} hkv={hkv} window={window}", flush=True)
    out = _run(ga, d, max(lens))
    ref, _ = oracle.decode_rows(d["q"], d["k_new"], d["v_new"], d["k_cache"], d["v_cache"], d["cu_cache"],
                                d["positions"], d["sink"], window, 1e4)
    compare("out", out.reshape(-1, 128), ref)


def test_decode_global_full_size_sampled():
    """Batch 64, cached lengths in [8192, 131072], 4 KV heads, base 1e7, seed 3 (cache drawn on the device):
    all 64 heads of 8 sequences against the oracle on the copied cache segments."""
    ga = _gpu()
    d = mi.decode_global(device="cuda")
    cu = d["cu_cache"].cpu()
    lens = (cu[1:] - cu[:-1]).tolist()
    out = ga.decode(d["q"], d["k_new"], d["v_new"], d["k_cache"], d["v_cache"], d["cu_cache"], d["positions"],
                    None, max(lens), -1, 1e7)
    torch.cuda.synchronize()
    out = out.cpu()
    rng = np.random.default_rng(5)
    bs = [int(np.argmax(lens)), int(np.argmin(lens))]
    bs = sorted(set(bs + [int(b) for b in rng.permutation(64) if int(b) not in bs][:6]))
    heads = np.arange(64)
    for b in bs:          # eight sequences (the longest and shortest among them), every query head
        s, e = int(cu[b]), int(cu[b + 1])
        kc = d["k_cache"][s:e].cpu()
        vc = d["v_cache"][s:e].cpu()
        ref, _ = oracle.decode_rows(d["q"][b:b + 1].cpu(), d["k_new"][b:b + 1].cpu(), d["v_new"][b:b + 1].cpu(),
                                    kc, vc, [0, e - s], d["positions"][b:b + 1].cpu(), None, -1, 1e7, rows=heads)
        compare(f"out b={b} len={e - s}", out[b][heads], ref)
