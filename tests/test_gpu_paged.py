"""GPU tests of the paged KV cache (page size 1): the append kernel against the oracle's rotation and the
forward's own rotation, decode and multi-token verify over a paged cache against the oracle (bf16 outputs
within max-abs 2e-2, mean-abs 2e-3) and bit for bit against the same cache stored contiguously, and a short
serving loop (prefill chunk, append, decode steps) against the whole-sequence prefill."""
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


def _scatter(kc, vc, extra, seed):
    """The rows of a contiguous cache scattered over a larger pool: (k_pool, v_pool, table) with
    k_pool[table[i]] = kc[i]; unused pool rows hold other values."""
    g = torch.Generator().manual_seed(seed)
    n, hkv = kc.shape[0], kc.shape[1]
    P = n + extra
    perm = torch.randperm(P, generator=g)[:n].to(torch.int32)
    kp = torch.randn(P, hkv, 192, generator=g).to(torch.bfloat16)
    vp = torch.randn(P, hkv, 128, generator=g).to(torch.bfloat16)
    kp[perm.long()] = kc
    vp[perm.long()] = vc
    return kp, vp, perm


def test_cache_append_rotation():
    """The appended keys equal the oracle's rotation within bf16 rounding, equal the forward's rotation of the
    same rows bit for bit (its rotated-q output), values are copied exactly and other pool rows stay."""
    ga = _gpu()
    g = torch.Generator().manual_seed(40)
    n, hkv, P = 300, 2, 1000
    k = torch.randn(n, hkv, 192, generator=g).to(torch.bfloat16)
    v = torch.randn(n, hkv, 128, generator=g).to(torch.bfloat16)
    pos = torch.cat([torch.arange(150), torch.randint(0, 131073, (150,), generator=g)]).to(torch.int32)
    slots = torch.randperm(P, generator=g)[:n].to(torch.int32)
    kp0 = torch.randn(P, hkv, 192, generator=g).to(torch.bfloat16)
    vp0 = torch.randn(P, hkv, 128, generator=g).to(torch.bfloat16)
    kp, vp = kp0.cuda(), vp0.cuda()
    print("case append n=300 hkv=2 pool=1000", flush=True)
    ga.cache_append(k.cuda(), v.cuda(), pos.cuda(), slots.cuda(), kp, vp, 1e7)
    torch.cuda.synchronize()
    kp, vp = kp.cpu(), vp.cpu()
    sl = slots.long()
    assert torch.equal(vp[sl].view(torch.int16), v.view(torch.int16))
    others = torch.ones(P, dtype=torch.bool)
    others[sl] = False
    assert torch.equal(kp[others].view(torch.int16), kp0[others].view(torch.int16))
    assert torch.equal(vp[others].view(torch.int16), vp0[others].view(torch.int16))
    ref = oracle.rope(k.reshape(-1, 192), pos.repeat_interleave(hkv), 1e7).reshape(n, hkv, 192)
    got = kp[sl].double().numpy()
    assert (np.abs(got - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-30).all()
    # the forward's rotation of the same rows at positions 0..149 (one 150-token sequence, these rows given as
    # its queries; the forward's rotated-q output uses the same cos/sin table and arithmetic as for keys)
    x = k[:150, :1].contiguous()
    qr = torch.empty(150, 1, 192, dtype=torch.bfloat16, device="cuda")
    ga.fwd(x.cuda(), x.cuda(), v[:150, :1].contiguous().cuda(), None,
           torch.tensor([0, 150], dtype=torch.int32, device="cuda"), 150, -1, 1e7, q_rot=qr)
    torch.cuda.synchronize()
    assert torch.equal(qr.cpu().view(torch.int16), kp[sl[:150], :1].view(torch.int16))


@pytest.mark.parametrize("lens,hkv,window,sink", [
    ([0, 1, 31, 32, 33, 1000, 2049, 5000], 4, -1, False),
    ([128, 1, 0, 127, 128, 128], 8, 128, True),
    ([3000, 7, 129], 2, 50, True),
])
def test_decode_paged(lens, hkv, window, sink):
    ga = _gpu()
    g = torch.Generator().manual_seed(41)
    B, hq = len(lens), 64
    r = lambda *sh: torch.randn(*sh, generator=g).to(torch.bfloat16)  # noqa: E731
    cu = mi.cu_from_lengths(lens)
    q, kn, vn = r(B, hq, 192), r(B, hkv, 192), r(B, hkv, 128)
    kc, vc = r(int(cu[-1]), hkv, 192), r(int(cu[-1]), hkv, 128)
    pos = torch.tensor([n + 33 for n in lens], dtype=torch.int32)
    sk = torch.randn(hq, generator=g) if sink else None
    kp, vp, table = _scatter(kc, vc, 777, 42)
    print(f"case decode_paged lens={lens} hkv={hkv} window={window}", flush=True)
    dev = "cuda"
    s = None if sk is None else sk.to(dev)
    o_p = ga.decode_paged(q.to(dev), kn.to(dev), vn.to(dev), kp.to(dev), vp.to(dev), table.to(dev), cu.to(dev),
                          pos.to(dev), s, max(lens), window, 1e4)
    o_c = ga.decode(q.to(dev), kn.to(dev), vn.to(dev), kc.to(dev), vc.to(dev), cu.to(dev), pos.to(dev), s, max(lens),
                    window, 1e4)
    torch.cuda.synchronize()
    assert torch.equal(o_p.view(torch.int16), o_c.view(torch.int16))
    ref, _ = oracle.decode_rows(q, kn, vn, kp[table.long()], vp[table.long()], cu, pos, sk, window, 1e4)
    compare("out", o_p.cpu().reshape(-1, 128), ref)


@pytest.mark.parametrize("hkv,window,sink,base", [(4, -1, False, 1e7), (8, 128, True, 1e4)])
def test_prefill_paged_verify(hkv, window, sink, base):
    """Eight draft tokens per sequence over a paged cache (the verify step of speculative decoding): against
    the oracle, and bit for bit against the same cache stored contiguously."""
    ga = _gpu()
    prefixes = [5000, 1, 300, 128, 0, 2047]
    chunks = [8] * len(prefixes)
    d = mi.make_cached(chunks, prefixes, 64, hkv, 43, sink, 128 if window >= 0 else None)
    kp, vp, table = _scatter(d["k_cache"], d["v_cache"], 500, 44)
    print(f"case verify hkv={hkv} window={window}", flush=True)
    dev = "cuda"
    t = lambda x: None if x is None else x.to(dev)  # noqa: E731
    o_p, l_p = ga.prefill_paged(t(d["q"]), t(d["k"]), t(d["v"]), t(kp), t(vp), t(table), t(d["sink"]),
                                t(d["cu_seqlens"]), t(d["cu_cache"]), t(d["positions"]), 8, d["max_position"], window,
                                base)
    o_c, l_c = ga.prefill_cached(t(d["q"]), t(d["k"]), t(d["v"]), t(d["k_cache"]), t(d["v_cache"]), t(d["sink"]),
                                 t(d["cu_seqlens"]), t(d["cu_cache"]), t(d["positions"]), 8, d["max_position"], window,
                                 base)
    torch.cuda.synchronize()
    assert torch.equal(o_p.view(torch.int16), o_c.view(torch.int16)) and torch.equal(l_p, l_c)
    ro, rl = oracle.prefill_cached_rows(d["q"], d["k"], d["v"], d["k_cache"], d["v_cache"], d["cu_seqlens"],
                                        d["cu_cache"], d["positions"], d["sink"], window, base)
    T = o_p.shape[0]
    compare("out", o_p.cpu(), ro.reshape(T, 64, -1))
    compare("lse", l_p.cpu(), rl.reshape(T, 64).T)


@pytest.mark.parametrize("hkv,window,sink,base", [(4, -1, False, 1e7), (8, 128, True, 1e4)])
def test_serving_loop_matches_whole_prefill(hkv, window, sink, base):
    """Two sequences: prefill a first chunk (no cache), append its keys to a pool, prefill a second chunk over
    the paged cache, append, then three decode steps over the paged cache, appending each token.  Every
    output row equals (to the tolerance) the same row of the oracle's prefill of the whole sequences."""
    ga = _gpu()
    L1, L2, steps = [300, 90], [40, 200], 3
    lengths = [a + b + steps for a, b in zip(L1, L2)]
    d = mi.make_layer(lengths, 64, hkv, 45, sink)
    print(f"case serving loop hkv={hkv} window={window}", flush=True)
    ro, rl = oracle.prefill(d["q"], d["k"], d["v"], d["sink"], d["cu_seqlens"], window, base)
    dev = "cuda"
    starts = [0, lengths[0]]
    P = sum(lengths) + 64
    kp = torch.zeros(P, hkv, 192, dtype=torch.bfloat16, device=dev)
    vp = torch.zeros(P, hkv, 128, dtype=torch.bfloat16, device=dev)
    sink_d = None if d["sink"] is None else d["sink"].to(dev)
    g = torch.Generator().manual_seed(46)
    free = torch.randperm(P, generator=g).tolist()
    tables = [[], []]
    cached = [0, 0]

    def append(b, toks):
        rows = [starts[b] + t for t in toks]
        slots = [free.pop() for _ in toks]
        ga.cache_append(d["k"][rows].to(dev), d["v"][rows].to(dev), torch.tensor(toks, dtype=torch.int32, device=dev),
                        torch.tensor(slots, dtype=torch.int32, device=dev), kp, vp, base)
        tables[b] += slots

    def chunk(lo, ln):
        """Prefill tokens lo[b] .. lo[b]+ln[b]-1 of each sequence over the paged cache, then append them."""
        rows = [starts[b] + lo[b] + i for b in range(2) for i in range(ln[b])]
        cuq = mi.cu_from_lengths(ln).to(dev)
        cup = mi.cu_from_lengths([len(t) for t in tables]).to(dev)
        tab = torch.tensor(tables[0] + tables[1], dtype=torch.int32, device=dev)
        out, lse = ga.prefill_paged(d["q"][rows].to(dev), d["k"][rows].to(dev), d["v"][rows].to(dev), kp, vp, tab,
                                    sink_d, cuq, cup, torch.tensor(lo, dtype=torch.int32, device=dev), max(ln),
                                    max(lengths), window, base)
        torch.cuda.synchronize()
        compare(f"chunk at {lo}", out.cpu(), ro[rows])
        for b in range(2):
            append(b, list(range(lo[b], lo[b] + ln[b])))

    chunk([0, 0], L1)
    chunk(L1, L2)
    for s in range(steps):
        p = [L1[b] + L2[b] + s for b in range(2)]
        rows = [starts[b] + p[b] for b in range(2)]
        cup = mi.cu_from_lengths([len(t) for t in tables]).to(dev)
        tab = torch.tensor(tables[0] + tables[1], dtype=torch.int32, device=dev)
        out = ga.decode_paged(d["q"][rows].to(dev), d["k"][rows].to(dev), d["v"][rows].to(dev), kp, vp, tab, cup,
                              torch.tensor(p, dtype=torch.int32, device=dev), sink_d, max(len(t) for t in tables),
                              window, base)
        torch.cuda.synchronize()
        compare(f"decode step {s}", out.cpu(), ro[rows])
        for b in range(2):
            append(b, [p[b]])


@pytest.mark.parametrize("prior,hkv,window,sink,base,nq", [
    ([5000, 0, 300, 128, 1020, 2047], 4, -1, False, 1e7, 8),
    ([5000, 0, 300, 128, 1020, 2047], 8, 128, True, 1e4, 8),
    ([40, 3, 1020], 2, 5, True, 1e4, 8),
    ([700, 1, 0], 4, -1, True, 1e7, 3),
    ([3000, 77, 0, 513], 4, 128, True, 1e4, 6),    # 96 columns: three column blocks and an idle wave
])
def test_verify_paged(prior, hkv, window, sink, base, nq):
    """nq draft tokens per sequence appended to a paged cache, then verified: against the oracle's prefill of
    the drafts over the prior rows (including a split that some drafts cannot see at all)."""
    ga = _gpu()
    hq = 64
    d = mi.make_cached([nq] * len(prior), prior, hq, hkv, 47, sink)
    print(f"case verify prior={prior} hkv={hkv} window={window} nq={nq}", flush=True)
    dev = "cuda"
    B = len(prior)
    Tc = d["k_cache"].shape[0]
    P = Tc + B * nq + 100
    g = torch.Generator().manual_seed(48)
    kp = torch.randn(P, hkv, 192, generator=g).to(torch.bfloat16).to(dev)
    vp = torch.randn(P, hkv, 128, generator=g).to(torch.bfloat16).to(dev)
    perm = torch.randperm(P, generator=g).to(torch.int32)
    cache_slots, draft_slots = perm[:Tc], perm[Tc:Tc + B * nq]
    kp[cache_slots.long()] = d["k_cache"].to(dev)
    vp[cache_slots.long()] = d["v_cache"].to(dev)
    pos = d["positions"]
    draft_pos = torch.cat([pos[b] + torch.arange(nq, dtype=torch.int32) for b in range(B)])
    ga.cache_append(d["k"].to(dev), d["v"].to(dev), draft_pos.to(dev), draft_slots.to(dev), kp, vp, base)
    cc = d["cu_cache"].tolist()
    table = torch.cat([torch.cat([cache_slots[cc[b]:cc[b + 1]], draft_slots[b * nq:(b + 1) * nq]]) for b in range(B)])
    cup = mi.cu_from_lengths([cc[b + 1] - cc[b] + nq for b in range(B)])
    maxlen = max(int(cup[b + 1] - cup[b]) for b in range(B))
    s = None if d["sink"] is None else d["sink"].to(dev)
    out = ga.verify_paged(d["q"].to(dev), kp, vp, table.to(dev), cup.to(dev), pos.to(dev), s, nq, maxlen, window, base)
    torch.cuda.synchronize()
    ro, _ = oracle.prefill_cached_rows(d["q"], d["k"], d["v"], d["k_cache"], d["v_cache"], d["cu_seqlens"],
                                       d["cu_cache"], d["positions"], d["sink"], window, base)
    compare("out", out.cpu(), ro.reshape(B * nq, hq, -1))


def test_verify_one_token_is_decode():
    """A one-token verify (the token's key appended first) gives decode's result within the tolerance."""
    ga = _gpu()
    g = torch.Generator().manual_seed(49)
    lens, hq, hkv = [300, 1, 2000], 64, 4
    B = len(lens)
    r = lambda *sh: torch.randn(*sh, generator=g).to(torch.bfloat16)  # noqa: E731
    cu = mi.cu_from_lengths(lens)
    q, kn, vn = r(B, hq, 192), r(B, hkv, 192), r(B, hkv, 128)
    kc, vc = r(int(cu[-1]), hkv, 192), r(int(cu[-1]), hkv, 128)
    pos = torch.tensor(lens, dtype=torch.int32)
    dev = "cuda"
    o_dec = ga.decode(q.to(dev), kn.to(dev), vn.to(dev), kc.to(dev), vc.to(dev), cu.to(dev), pos.to(dev), None,
                      max(lens), -1, 1e7)
    Tc = int(cu[-1])
    kp = torch.cat([kc, torch.zeros(B, hkv, 192, dtype=torch.bfloat16)]).to(dev)
    vp = torch.cat([vc, torch.zeros(B, hkv, 128, dtype=torch.bfloat16)]).to(dev)
    slots = torch.arange(Tc, Tc + B, dtype=torch.int32)
    ga.cache_append(kn.to(dev), vn.to(dev), pos.to(dev), slots.to(dev), kp, vp, 1e7)
    cl = cu.tolist()
    table = torch.cat([torch.cat([torch.arange(cl[b], cl[b + 1], dtype=torch.int32), slots[b:b + 1]]) for b in range(B)])
    cup = mi.cu_from_lengths([n + 1 for n in lens])
    o_ver = ga.verify_paged(q.to(dev), kp, vp, table.to(dev), cup.to(dev), pos.to(dev), None, 1, max(lens) + 1, -1, 1e7)
    torch.cuda.synchronize()
    compare("verify vs decode", o_ver.cpu(), o_dec.cpu().double(), max_abs=1e-2, mean_abs=1e-3)


def _guarded(x, fill, rows=64):
    """x on the GPU inside one larger allocation with `rows` guard rows of `fill` before and after it:
    (the whole buffer, the view holding x)."""
    buf = torch.full((rows + x.shape[0] + rows, *x.shape[1:]), fill, dtype=x.dtype, device="cuda")
    buf[rows:rows + x.shape[0]] = x.to("cuda")
    return buf, buf[rows:rows + x.shape[0]]


@pytest.mark.parametrize("hkv,window,sink,base", [(4, -1, False, 1e7), (8, 128, True, 1e4)])
def test_prefill_paged_index_arrays_disagree_with_sizes(hkv, window, sink, base):
    """Regression test of the guards for index arrays that do not match the sizes given.  Inputs, pools and
    the table sit inside larger allocations whose guard rows hold NaN (a read past any of them would make the
    outputs non-finite) and the output inside one whose guard rows hold a sentinel (a write past it would
    change them).  (a) A table with more entries than cu_pages covers: the extra entries belong to no sequence,
    so the output equals, bit for bit, the call with the exact table, and the oracle.  (b) cu_pages claiming
    2000 more cache rows for the second sequence than the table holds (the later sequences' keys then start
    past the prepared stream): keys the arrays do not account for are zero-filled and the key range is clamped
    to the stream, so the rows of that call are finite (not checked against the oracle: they are not
    defined), the guard rows of the output are untouched, and the first sequence, whose entries are exact,
    keeps the exact call's rows bit for bit."""
    ga = _gpu()
    prefixes, chunks = [300, 5, 64, 0], [40, 7, 129, 33]
    d = mi.make_cached(chunks, prefixes, 64, hkv, 46, sink, 128 if window >= 0 else None)
    kp, vp, table = _scatter(d["k_cache"], d["v_cache"], 300, 47)
    g = torch.Generator().manual_seed(48)
    extra = torch.randint(0, kp.shape[0], (50,), generator=g).to(torch.int32)
    nan = float("nan")
    _, q = _guarded(d["q"], nan)
    _, k = _guarded(d["k"], nan)
    _, v = _guarded(d["v"], nan)
    _, kpg = _guarded(kp, nan)
    _, vpg = _guarded(vp, nan)
    T = d["q"].shape[0]
    dev = "cuda"
    t = lambda x: None if x is None else x.to(dev)  # noqa: E731
    print(f"case index arrays vs sizes hkv={hkv} window={window}", flush=True)

    def run(tab, cu_pages):
        obuf, out = _guarded(torch.zeros(T, 64, 128, dtype=torch.bfloat16), 7.0)
        o, lse = ga.prefill_paged(q, k, v, kpg, vpg, tab, t(d["sink"]), t(d["cu_seqlens"]), cu_pages,
                                  t(d["positions"]), max(chunks), d["max_position"] + 4000, window, base, out=out)
        torch.cuda.synchronize()
        g_ = obuf.cpu().float()
        assert (g_[:64] == 7.0).all() and (g_[64 + T:] == 7.0).all(), "output guard rows changed"
        return o.cpu(), lse.cpu()

    o_exact, l_exact = run(t(table), t(d["cu_cache"]))
    _, tab_long = _guarded(torch.cat([table, extra]).reshape(-1, 1), 0)
    o_long, l_long = run(tab_long.reshape(-1), t(d["cu_cache"]))
    assert torch.equal(o_long.view(torch.int16), o_exact.view(torch.int16)) and torch.equal(l_long, l_exact)
    ro, rl = oracle.prefill_cached_rows(d["q"], d["k"], d["v"], d["k_cache"], d["v_cache"], d["cu_seqlens"],
                                        d["cu_cache"], d["positions"], d["sink"], window, base)
    compare("out (longer table)", o_long, ro.reshape(T, 64, -1))

    over = d["cu_cache"].clone()
    over[2:] += 2000
    o_over, l_over = run(t(table), t(over))
    assert torch.isfinite(o_over.float()).all() and not torch.isnan(l_over).any()
    n0 = chunks[0]
    assert torch.equal(o_over[:n0].view(torch.int16), o_exact[:n0].view(torch.int16))
