"""GPU parity at the per-GPU shapes of a 4-way head split (16 query heads with 2 KV heads on sliding-window
layers and 1 on global layers) and for decode against one 1,048,576-row cache (the configured 1M context),
against the fp64 oracle: bf16 outputs within max-abs 2e-2 and mean-abs 2e-3 (gradients widened by a bf16
half-ulp where |ref| >= 8), dsink 1e-2 relative per head."""
import numpy as np
import pytest
import torch

import mimo_inputs as mi
import oracle
from parity import compare, compare_rel

pytestmark = pytest.mark.gpu


def _gpu():
    import global_gqa_attention_amd as ga

    if not torch.cuda.is_available():
        pytest.fail("a GPU is required for the -m gpu tests")
    return ga


SHARDS = [(16, 2, 128, 1e4, True), (16, 1, -1, 1e7, False)]


@pytest.mark.parametrize("hq,hkv,window,base,sink", SHARDS)
def test_shard_fwd_bwd_full(hq, hkv, window, base, sink):
    ga = _gpu()
    lengths = [1, 64, 129, 300, 0, 77]
    d = mi.make_layer(lengths, hq, hkv, 13, sink)
    print(f"case shard hq={hq} hkv={hkv} window={window}", flush=True)
    dev = "cuda"
    q, k, v, cu = d["q"].to(dev), d["k"].to(dev), d["v"].to(dev), d["cu_seqlens"].to(dev)
    s = None if d["sink"] is None else d["sink"].to(dev)
    out, lse = ga.fwd(q, k, v, s, cu, max(lengths), window, base)
    torch.cuda.synchronize()
    ro, rl = oracle.prefill(d["q"], d["k"], d["v"], d["sink"], d["cu_seqlens"], window, base)
    compare("out", out.cpu(), ro)
    compare("lse", lse.cpu(), rl)
    # backward given the oracle's forward outputs (the same O on both sides)
    O = torch.from_numpy(ro).to(torch.bfloat16)
    L = torch.from_numpy(rl).to(torch.float32)
    dO = mi.dout_like(sum(lengths), 4, hq)
    dq, dk, dv, ds = ga.bwd(q, k, v, s, O.to(dev), L.to(dev), dO.to(dev), cu, max(lengths), window, base)
    torch.cuda.synchronize()
    rq, rk, rv, rs = oracle.prefill_bwd(d["q"], d["k"], d["v"], d["sink"], dO, d["cu_seqlens"], window, base,
                                        out_given=O)
    compare("dq", dq.cpu(), rq, grad=True)
    compare("dk", dk.cpu(), rk, grad=True)
    compare("dv", dv.cpu(), rv, grad=True)
    if sink:
        compare_rel("dsink", ds.cpu(), rs)


@pytest.mark.parametrize("hq,hkv,window,base,sink", SHARDS)
def test_shard_decode_full(hq, hkv, window, base, sink):
    ga = _gpu()
    g = torch.Generator().manual_seed(14)
    lens = [5000, 1, 0, 130, 128] if window < 0 else [128, 1, 0, 127, 128]
    B = len(lens)
    r = lambda *sh: torch.randn(*sh, generator=g).to(torch.bfloat16)  # noqa: E731
    cu = mi.cu_from_lengths(lens)
    q, kn, vn = r(B, hq, 192), r(B, hkv, 192), r(B, hkv, 128)
    kc, vc = r(int(cu[-1]), hkv, 192), r(int(cu[-1]), hkv, 128)
    pos = torch.tensor([n + 900 for n in lens], dtype=torch.int32)
    sk = torch.randn(hq, generator=g) if sink else None
    print(f"case shard decode hq={hq} hkv={hkv} lens={lens}", flush=True)
    dev = "cuda"
    out = ga.decode(q.to(dev), kn.to(dev), vn.to(dev), kc.to(dev), vc.to(dev), cu.to(dev), pos.to(dev),
                    None if sk is None else sk.to(dev), max(lens), window, base)
    torch.cuda.synchronize()
    ref, _ = oracle.decode_rows(q, kn, vn, kc, vc, cu, pos, sk, window, base)
    compare("out", out.cpu().reshape(-1, 128), ref)


def test_decode_1m_context_sampled():
    """One sequence with 1,048,576 cached rows (global layer: 64 query heads, 4 KV heads, base 1e7; the cache
    drawn on the device, seed 3): 16 heads against the oracle on the copied cache."""
    ga = _gpu()
    n = 1 << 20
    d = mi.decode_global(batch=1, len_lo=n, len_hi=n, device="cuda")
    print("case decode 1M context", flush=True)
    out = ga.decode(d["q"], d["k_new"], d["v_new"], d["k_cache"], d["v_cache"], d["cu_cache"], d["positions"],
                    None, n, -1, 1e7)
    torch.cuda.synchronize()
    out = out.cpu()
    assert torch.isfinite(out.float()).all()
    heads = np.arange(0, 64, 4)
    ref, _ = oracle.decode_rows(d["q"].cpu(), d["k_new"].cpu(), d["v_new"].cpu(), d["k_cache"].cpu(),
                                d["v_cache"].cpu(), [0, n], d["positions"].cpu(), None, -1, 1e7, rows=heads)
    compare("out 1M", out[0][heads], ref)


def test_decode_few_long_sequences_sampled():
    """Three sequences (200000, 65536 and 3 cached rows; hundreds of splits per sequence): 8 heads each."""
    ga = _gpu()
    lens = [200000, 65536, 3]
    g = torch.Generator(device="cuda").manual_seed(15)
    B, hq, hkv = 3, 64, 4
    r = lambda *sh: torch.randn(*sh, generator=g, device="cuda").to(torch.bfloat16)  # noqa: E731
    cu = mi.cu_from_lengths(lens)
    q, kn, vn = r(B, hq, 192), r(B, hkv, 192), r(B, hkv, 128)
    kc, vc = r(int(cu[-1]), hkv, 192), r(int(cu[-1]), hkv, 128)
    pos = torch.tensor(lens, dtype=torch.int32)
    print("case decode 3 long sequences", flush=True)
    out = ga.decode(q, kn, vn, kc, vc, cu.cuda(), pos.cuda(), None, max(lens), -1, 1e7)
    torch.cuda.synchronize()
    out = out.cpu()
    heads = np.arange(3, 64, 8)
    rows = np.concatenate([b * hq + heads for b in range(B)])
    ref, _ = oracle.decode_rows(q.cpu(), kn.cpu(), vn.cpu(), kc.cpu(), vc.cpu(), cu, pos, None, -1, 1e7, rows=rows)
    compare("out", out.reshape(-1, 128)[rows], ref)
