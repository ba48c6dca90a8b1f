"""The no-allocation paged decode (mimo_attn_decode_paged_noalloc, split partials in the library's scratch
array) against mimo_attn_decode_paged (caller workspace), through the C ABI, on two calls in a row: a batch-64
global-layer step whose usual split plan needs more than the 64 MiB array (so the call takes fewer, longer
splits: equal to the oracle tolerance, max-abs 2e-2 and mean-abs 2e-3), then a smaller sliding-window step
with a sink whose plan fits (bit for bit), which also shows that nothing the first call left in the array
leaks into the second."""
import pytest
import torch

from parity import compare

pytestmark = pytest.mark.gpu


def _case(batch, hkv, window, sink, len_lo, len_hi, seed):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    lens = torch.randint(len_lo, len_hi + 1, (batch,), generator=g, device="cuda").to(torch.int32)
    cu = torch.zeros(batch + 1, dtype=torch.int32, device="cuda")
    cu[1:] = torch.cumsum(lens, 0)
    N = int(cu[-1])
    P = N + 1000
    r = lambda *sh: torch.randn(*sh, generator=g, device="cuda").to(torch.bfloat16)  # noqa: E731
    d = dict(q=r(batch, 64, 192), k_new=r(batch, hkv, 192), v_new=r(batch, hkv, 128), k_pool=r(P, hkv, 192),
             v_pool=r(P, hkv, 128), cu=cu, table=torch.randperm(P, generator=g, device="cuda")[:N].to(torch.int32),
             positions=(lens + 5).contiguous(), sink=torch.randn(64, generator=g, device="cuda") if sink else None,
             max_len=int(lens.max()), window=window)
    return d


def _both(ga, d, base):
    args = (d["q"], d["k_new"], d["v_new"], d["k_pool"], d["v_pool"], d["table"], d["cu"], d["positions"], d["sink"],
            d["max_len"], d["window"], base)
    ref = ga.decode_paged(*args)
    out = torch.full_like(ref, float("nan"))
    ga.decode_paged_noalloc(*args, out=out)
    torch.cuda.synchronize()
    return out.cpu(), ref.cpu()


def test_decode_paged_noalloc_matches_decode_paged():
    import global_gqa_attention_amd as ga

    if not torch.cuda.is_available():
        pytest.fail("a GPU is required for the -m gpu tests")
    print("case noalloc call 1: batch 64 global, caches 20000..32768 rows (capped split plan)", flush=True)
    d = _case(64, 4, -1, False, 20000, 32768, 60)
    out, ref = _both(ga, d, 1e7)
    compare("noalloc vs decode_paged (capped plan)", out.reshape(-1, 128), ref.reshape(-1, 128))
    del d
    torch.cuda.empty_cache()
    print("case noalloc call 2: batch 8 sliding window 128 with sink (usual plan)", flush=True)
    d = _case(8, 8, 128, True, 1, 3000, 61)
    out, ref = _both(ga, d, 1e4)
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))

