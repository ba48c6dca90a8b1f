"""CPU checks of the C ABI: the library loads without a GPU, exports every declared symbol, and rejects bad
arguments on the host before launching anything (no compute call is made here)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mimo_attn.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(mimo_attn_\w+)\s*\(", src)))


@pytest.fixture(scope="module")
def L():
    import global_gqa_attention_amd as ga

    if not os.path.exists(ga.LIB_PATH):
        pytest.fail("libmimo_attn.so is not built (run __graft_entry__.build())")
    return ga.lib()


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ("mimo_attn_fwd", "mimo_attn_bwd", "mimo_attn_decode", "mimo_attn_fwd_workspace_size",
              "mimo_attn_bwd_workspace_size", "mimo_attn_bwd_workspace_size_fast",
              "mimo_attn_decode_workspace_size", "mimo_attn_status_string", "mimo_attn_last_error",
              "mimo_attn_release", "mimo_attn_prefill_cached", "mimo_attn_prefill_cached_workspace_size",
              "mimo_attn_cache_append", "mimo_attn_decode_paged", "mimo_attn_prefill_paged"):
        assert n in names


def test_library_exports_every_declared_symbol(L):
    for n in declared_functions():
        assert hasattr(L, n), n


def test_status_strings(L):
    for code, name in [(0, b"MIMO_OK"), (1, b"MIMO_ERR_INVALID_ARG"), (2, b"MIMO_ERR_UNSUPPORTED"),
                       (3, b"MIMO_ERR_HIP"), (4, b"MIMO_ERR_WORKSPACE")]:
        assert L.mimo_attn_status_string(code) == name


FAKE = ctypes.c_void_p(0x1000)   # never dereferenced: every case below fails host validation first


def fwd(L, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, sink=None, cu=FAKE, batch=1, T=16, max_seqlen=16, window=128,
             base=1e4, hq=64, hkv=8, out=FAKE, lse=None, q_rot=None, k_rot=None, ws=FAKE, wsb=1 << 30)
    a.update(kw)
    return L.mimo_attn_fwd(a["q"], a["k"], a["v"], a["sink"], a["cu"], a["batch"], a["T"], a["max_seqlen"],
                           a["window"], a["base"], a["hq"], a["hkv"], a["out"], a["lse"], a["q_rot"], a["k_rot"], a["ws"],
                           a["wsb"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(hkv=7), 1), (dict(window=-2), 1), (dict(batch=-1), 1), (dict(T=-5), 1), (dict(q=None), 1),
    (dict(out=None), 1), (dict(base=0.5), 1), (dict(base=float("inf")), 1), (dict(max_seqlen=0), 1),
    (dict(batch=0), 1), (dict(hq=0), 1), (dict(cu=None), 1), (dict(ws=None), 4), (dict(wsb=64), 4),
])
def test_fwd_rejects_bad_arguments(L, kw, code):
    assert fwd(L, **kw) == code
    assert L.mimo_attn_last_error() != b""


def test_empty_batch_is_a_no_op(L):
    assert fwd(L, batch=0, T=0, q=None, k=None, v=None, cu=FAKE, out=None) == 0


def bwd(L, **kw):
    a = dict(sink=None, dsink=None, ws=FAKE, wsb=1 << 30, hkv=8, T=16, window=128)
    a.update(kw)
    return L.mimo_attn_bwd(FAKE, FAKE, FAKE, a["sink"], FAKE, FAKE, FAKE, None, None, FAKE, 1, a["T"], 16, a["window"],
                           1e4, 64, a["hkv"], FAKE, FAKE, FAKE, a["dsink"], a["ws"], a["wsb"], None)


def test_bwd_rejects_bad_arguments(L):
    assert bwd(L, sink=FAKE, dsink=None) == 1          # dsink must come with sink
    assert bwd(L, sink=None, dsink=FAKE) == 1
    assert bwd(L, ws=None) == 4                         # workspace missing
    assert bwd(L, wsb=16) == 4                          # workspace too small
    assert bwd(L, hkv=3) == 1


def test_workspace_sizes(L):
    assert L.mimo_attn_fwd_workspace_size(32768, 64, 8, 128) >= 32768 * 8 * 640
    n = L.mimo_attn_bwd_workspace_size(32768, 64, 8, 128)
    assert n >= 32768 * 64 * 4
    assert L.mimo_attn_decode_workspace_size(64, 131072, 64, -1) > 0
    assert L.mimo_attn_bwd_workspace_size(-1, 64, 8, 128) == 0


def _ds_blocks_per_head(lengths, window):
    """dS blocks of one head as the stored-dS layout lays them out: sequence b has nq query tiles of 32 that
    start at seq_start & ~15; causal rows hold n + 1 blocks, sliding-window rows (window + 62) // 32 + 1."""
    tot, start = 0, 0
    for L_ in lengths:
        nq = (start + L_ - 1 - (start & ~15)) // 32 + 1 if L_ > 0 else 0
        tot += nq * ((window + 62) // 32 + 1) if window >= 0 else nq * (nq + 1) // 2
        start += L_
    return tot


@pytest.mark.parametrize("window", [-1, 128, 0])
def test_fast_bwd_workspace_covers_every_batch(L, window):
    import numpy as np

    rng = np.random.default_rng(5)
    for trial in range(300):
        batch = int(rng.integers(1, 40))
        lengths = [int(x) for x in rng.integers(0, 3000, size=batch)]
        if rng.random() < 0.3:
            lengths[int(rng.integers(batch))] = int(rng.integers(3000, 40000))
        T, maxl = sum(lengths), max(lengths)
        if T == 0:
            continue
        base = L.mimo_attn_bwd_workspace_size(T, 64, 4, window)
        fast = L.mimo_attn_bwd_workspace_size_fast(T, batch, maxl, 64, 4, window)
        need = 64 * _ds_blocks_per_head(lengths, window) * 2048 + (batch + 1) * 8
        assert fast >= base + need, (lengths, window)


def test_fast_bwd_workspace_falls_back_for_other_groups(L):
    # the stored-dS dQ kernel takes query heads four at a time: other group sizes keep the least size
    assert L.mimo_attn_bwd_workspace_size_fast(4096, 2, 4096, 6, 2, -1) == L.mimo_attn_bwd_workspace_size(4096, 6, 2, -1)
    assert L.mimo_attn_bwd_workspace_size_fast(4096, 2, 4096, 64, 4, -1) > L.mimo_attn_bwd_workspace_size(4096, 64, 4, -1)
    assert L.mimo_attn_bwd_workspace_size_fast(-1, 2, 4096, 64, 4, -1) == 0


def test_decode_rejects_bad_arguments(L):
    def dec(**kw):
        a = dict(batch=4, hq=64, hkv=8, window=128, ws=FAKE, wsb=1 << 30, q=FAKE)
        a.update(kw)
        return L.mimo_attn_decode(a["q"], FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, a["batch"], 128, a["window"],
                                  1e4, a["hq"], a["hkv"], FAKE, a["ws"], a["wsb"], None)
    assert dec(hkv=5) == 1
    assert dec(window=-3) == 1
    assert dec(q=None) == 1
    assert dec(ws=None) == 4
    assert dec(batch=0) == 0


def test_prefill_cached_rejects_bad_arguments(L):
    def pc(**kw):
        a = dict(batch=2, T=16, Tc=64, max_seqlen=16, max_position=200, window=128, hq=64, hkv=8, ws=FAKE,
                 wsb=1 << 30, kc=FAKE, cuc=FAKE, pos=FAKE, out=FAKE)
        a.update(kw)
        return L.mimo_attn_prefill_cached(FAKE, FAKE, FAKE, a["kc"], FAKE, None, FAKE, a["cuc"], a["pos"], a["batch"],
                                          a["T"], a["Tc"], a["max_seqlen"], a["max_position"], a["window"], 1e4,
                                          a["hq"], a["hkv"], a["out"], None, a["ws"], a["wsb"], None)
    assert pc(hkv=5) == 1
    assert pc(window=-3) == 1
    assert pc(Tc=-1) == 1
    assert pc(cuc=None) == 1
    assert pc(pos=None) == 1
    assert pc(kc=None) == 1
    assert pc(out=None) == 1
    assert pc(max_position=8) == 1
    assert pc(ws=None) == 4
    assert pc(wsb=16) == 4
    assert pc(T=0) == 0
    assert pc(T=0, Tc=0, batch=0, max_seqlen=0) == 0
    need = L.mimo_attn_prefill_cached_workspace_size(16, 64, 8)
    assert need >= L.mimo_attn_fwd_workspace_size(80, 64, 8, 128)
    assert L.mimo_attn_prefill_cached_workspace_size(-1, 0, 8) == 0


def test_paged_entry_points_reject_bad_arguments(L):
    def app(**kw):
        a = dict(k=FAKE, n=4, hkv=8, pool=100, base=1e4, kp=FAKE)
        a.update(kw)
        return L.mimo_attn_cache_append(a["k"], FAKE, FAKE, FAKE, a["n"], a["hkv"], a["pool"], a["base"], a["kp"], FAKE,
                                        None)
    assert app(n=-1) == 1
    assert app(hkv=0) == 1
    assert app(pool=-1) == 1
    assert app(base=1.0) == 1
    assert app(k=None) == 1
    assert app(kp=None) == 1
    assert app(n=0) == 0

    def dec(**kw):
        a = dict(batch=4, hkv=8, table=FAKE, maxlen=128, ws=FAKE)
        a.update(kw)
        return L.mimo_attn_decode_paged(FAKE, FAKE, FAKE, FAKE, FAKE, a["table"], FAKE, FAKE, None, a["batch"],
                                        a["maxlen"], 128, 1e4, 64, a["hkv"], FAKE, a["ws"], 1 << 30, None)
    assert dec(table=None) == 1
    assert dec(hkv=5) == 1
    assert dec(ws=None) == 4
    assert dec(batch=0) == 0

    def pre(**kw):
        a = dict(table=FAKE, npg=64, T=16, ws=FAKE)
        a.update(kw)
        return L.mimo_attn_prefill_paged(FAKE, FAKE, FAKE, FAKE, FAKE, a["table"], None, FAKE, FAKE, FAKE, 2, a["T"],
                                         a["npg"], 16, 200, 128, 1e4, 64, 8, FAKE, None, a["ws"], 1 << 30, None)
    assert pre(table=None) == 1
    assert pre(ws=None) == 4
    assert pre(T=0) == 0


def test_binding_refuses_cpu_tensors():
    import torch

    import global_gqa_attention_amd as ga

    q = torch.zeros(4, 8, 192, dtype=torch.bfloat16)
    k = torch.zeros(4, 8, 192, dtype=torch.bfloat16)
    v = torch.zeros(4, 8, 128, dtype=torch.bfloat16)
    cu = torch.tensor([0, 4], dtype=torch.int32)
    with pytest.raises(ga.MimoAttnError):
        ga.fwd(q, k, v, None, cu, 4, 128, 1e4)


def test_key_stream_offset_limits(L):
    """Key streams whose transposed copies would need 32-bit copy offsets past 2^32 are refused: the forward
    and cached prefill up to T_pad * 256 bytes per V^T row block, the backward up to T_pad * 384."""
    fwd_max, bwd_max = 16_777_136, 11_184_736          # largest token counts whose padded stream fits
    assert L.mimo_attn_fwd_workspace_size(fwd_max, 1, 1, -1) > 0
    assert L.mimo_attn_fwd_workspace_size(fwd_max + 1, 1, 1, -1) == 0
    assert L.mimo_attn_prefill_cached_workspace_size(fwd_max - 1000, 1000, 1) > 0
    assert L.mimo_attn_prefill_cached_workspace_size(fwd_max - 1000, 1001, 1) == 0
    assert L.mimo_attn_bwd_workspace_size(bwd_max, 1, 1, -1) > 0
    assert L.mimo_attn_bwd_workspace_size(bwd_max + 1, 1, 1, -1) == 0
    assert L.mimo_attn_bwd_workspace_size_fast(bwd_max + 1, 1, bwd_max + 1, 4, 1, -1) == 0
    assert fwd(L, T=fwd_max + 1, max_seqlen=fwd_max + 1, hq=1, hkv=1) == 2
    assert b"32-bit" in L.mimo_attn_last_error()
    assert L.mimo_attn_bwd(FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE, None, None, FAKE, 1, bwd_max + 1, bwd_max + 1, -1,
                           1e4, 1, 1, FAKE, FAKE, FAKE, None, FAKE, 1 << 62, None) == 2
    assert L.mimo_attn_prefill_cached(FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE, 1, 16, fwd_max, 16,
                                      fwd_max + 16, -1, 1e4, 1, 1, FAKE, None, FAKE, 1 << 62, None) == 2
    assert fwd(L, hq=8192, hkv=8) == 2                  # head counts beyond the copy offsets' range


def _fwd_tile_starts(t0, t_last, kofs, kseq, window, T_pad, BN):
    """Every key-tile start the forward kernel issues for one work item, restated from its integer formulas:
    the first tile at kstart, then in each step the tile one (two-stage ring) or two (three-stage ring)
    ahead, clamped to the last tile klast."""
    klo = max(kseq, t0 + kofs - window) if window >= 0 else kseq
    kstart = min(max(klo, 0) & ~15, T_pad - BN)
    khi = min(t_last + kofs, T_pad - BN - 1)
    num = khi - kstart + BN
    nkt = max(int(num / BN), 0)                          # C division truncates toward zero
    klast = kstart + max(nkt - 1, 0) * BN
    starts = [kstart]
    if window < 0:                                       # causal: three-stage ring
        starts.append(min(kstart + BN, klast))
        for it in range(nkt):
            starts.append(min(kstart + (it + 2) * BN, klast))
    else:                                                # sliding window: two-stage ring
        for it in range(0, nkt, 2):
            k0 = kstart + it * BN
            starts += [min(k0 + BN, klast), min(k0 + 2 * BN, klast)]
    computed = [kstart + it * BN for it in range(nkt)]
    return starts, computed, khi


@pytest.mark.parametrize("window,BN,TT", [(-1, 32, 48), (128, 32, 16), (3, 32, 16)])
def test_fwd_key_tiles_stay_inside_the_prepared_stream(window, BN, TT):
    """Cached prefill with cache index arrays that agree with the sizes, claim more rows than given (the key
    offsets run past the stream) or fewer: every tile the forward issues lies inside the T_pad rows of the
    prepared stream, and with agreeing arrays every key a query sees is computed."""
    import numpy as np

    rng = np.random.default_rng(11)
    for trial in range(400):
        batch = int(rng.integers(1, 6))
        lens = rng.integers(0, 300, batch)
        ncache = rng.integers(0, 400, batch)
        T, Tc = int(lens.sum()), int(ncache.sum())
        cu = np.concatenate([[0], np.cumsum(lens)])
        cuc = np.concatenate([[0], np.cumsum(ncache)])
        mode = trial % 3
        if mode == 1:                                    # over-stated: more cache rows than Tc
            cuc = cuc + rng.integers(0, 5000) * np.arange(batch + 1)
        elif mode == 2:                                  # under-stated
            cuc = cuc // 2
        T_pad = (T + Tc + 15) // 16 * 16 + 64
        for b in range(batch):
            s, e = int(cu[b]), int(cu[b + 1])
            kofs, kseq = int(cuc[b + 1]), int(cuc[b]) + s
            for t0 in range(s, e, TT):
                t_last = min(t0 + TT - 1, e - 1)
                starts, computed, khi = _fwd_tile_starts(t0, t_last, kofs, kseq, window, T_pad, BN)
                for k in starts:
                    assert 0 <= k and k + BN <= T_pad, (trial, mode, k, T_pad)
                if mode == 0:
                    need_lo = max(kseq, t0 + kofs - window) if window >= 0 else kseq
                    need_hi = t_last + kofs
                    assert computed and computed[0] <= need_lo and computed[-1] + BN - 1 >= need_hi


def test_decode_paged_noalloc_rejects_partials_beyond_its_scratch(L):
    """One split's partials of batch x n_q_heads rows (520 bytes each) must fit the 64 MiB scratch array:
    129055 rows do, 4096 x 64 do not (rejected on the host, nothing launched)."""
    rc = L.mimo_attn_decode_paged_noalloc(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, 4096, 128, -1, 1e7,
                                          64, 4, FAKE, None)
    assert rc == 2 and b"scratch" in L.mimo_attn_last_error()
    assert L.mimo_attn_decode_paged_noalloc(FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, None, 4, 128, -1, 1e7,
                                            64, 4, FAKE, None) == 1          # no page table
    assert L.mimo_attn_decode_paged_noalloc(None, None, None, None, None, None, None, None, None, 0, 0, -1, 1e7,
                                            64, 4, None, None) == 0          # empty batch: nothing to do


def test_m0_guard_of_the_build():
    """The build rejects device code that touches m0 anywhere but in the copy helper's own sequence."""
    from global_gqa_attention_amd.build import _m0_misuse

    ok = "\ts_mov_b32 m0, s31\n\ts_nop 0\n\tglobal_load_lds_dwordx4 v65, s[12:13]\n\tv_add_u32 v1, v2, v3 ; m0 in a comment\n"
    assert _m0_misuse(ok) == []
    assert _m0_misuse("\ts_mov_b32 m0, -1\n\tds_read_b32 v1, v2\n") == ["s_mov_b32 m0, -1"]
    assert _m0_misuse("\ts_mov_b32 m0, s4\n\ts_nop 0\n\tds_gws_init v1\n") == ["s_mov_b32 m0, s4"]
    assert _m0_misuse("\ts_mov_b32 s5, m0\n") == ["s_mov_b32 s5, m0"]


def test_causal_backward_head_split_rule(L):
    """The causal backward's fp32 dK/dV partials (the only part of its workspace that a sliding-window layer
    does not have) follow the head-split rule: two splits where the 128-key tiles of all KV heads number at
    least 1024, four below that, none for groups under four query heads."""
    def tpad(T):
        return (T + 15) // 16 * 16 + 64

    def al(n):
        return (n + 255) // 256 * 256

    for T, hq, hkv in [(32768, 64, 4), (65536, 64, 4), (16384, 64, 4), (32768, 16, 1), (32768, 16, 2),
                       (4000, 64, 8), (131072, 16, 1), (32768, 12, 4), (32768, 24, 4)]:
        G = hq // hkv
        tiles = -(-T // 128) * hkv
        splits = 1 if G % 2 or G < 4 else (2 if tiles >= 1024 or G % 4 else 4)
        part = L.mimo_attn_bwd_workspace_size(T, hq, hkv, -1) - L.mimo_attn_bwd_workspace_size(T, hq, hkv, 128)
        assert part == (al(splits * tpad(T) * hkv * 1280) if splits > 1 else 0), (T, hq, hkv, splits)
