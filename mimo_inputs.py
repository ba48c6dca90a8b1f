"""Seeded synthetic inputs for the MiMo-V2.6-Flash attention layer.

This module only draws random numbers and builds index arrays; it holds none of the layer's arithmetic.  It
is the one piece shared by the HIP-path tests, the oracle tests and the benchmark, so both sides of every
parity check see the same bytes.

Recipe (every tensor drawn with ``torch.Generator().manual_seed(seed)`` on the CPU unless a function says
otherwise, ``randn`` in fp32, then rounded to bf16 round-to-nearest-even by ``.to(torch.bfloat16)``):

* ``swa_512``  -- one sequence of 512 tokens; 64 Q heads, 8 KV heads, window 128, RoPE base 1e4, fp32
  N(0,1) sink per Q head.  Seed 0.  Draw order: q, k, v, sink.
* ``global_2x4096`` -- two sequences of 4096 tokens; 64 Q heads, 4 KV heads, causal, base 1e7, no sink.
  Seed 1.  Draw order: q, k, v.
* ``thd_32k`` -- 16 lengths drawn by ``randint(1024, 2049)`` (uniform over [1024, 2048] inclusive), then
  one final sequence that pads the batch to 32768 tokens (17 sequences, int32 cu_seqlens).  Seed 2.  Draw
  order: lengths, SWA-layer q, k (8 heads), v, sink, global-layer q, k (4 heads), v.
* ``dout_32k`` -- bf16 N(0,1) upstream gradient [T, 64, 128], seed 4.
* decode (seed 3): batch 64, one token per sequence.  SWA: 128-entry ring cache per sequence holding rotated
  K and unscaled V, positions drawn from [8192, 131072] inclusive; global: cached lengths drawn from
  [8192, 131072] inclusive, position = cached length.  Draw order: positions or lengths, q, k_new, v_new,
  sink (SWA), then the cache (K, then V).  The global cache (about 11 GB) is drawn on the device with a
  device generator seeded the same way when ``device`` is a GPU, since the CPU stream would take minutes;
  its first-kind recipe is then ``torch.Generator(device).manual_seed(seed + 1000)``.
* cached prefill (``make_cached``): new tokens (q, k, v) per sequence plus cache rows standing for the keys
  just before them (random bf16 K treated as already rotated, and V); sequence b's first new token sits at
  position prefix_b, and its cache holds the last min(prefix_b, keep) rows (keep None: the whole prefix).
  Draw order: q, k, v of the new tokens, sink, then the cache (K, then V).  ``chunked_16`` (seed 5): 16
  sequences, prefixes drawn by ``randint(2048, 8193)``, chunks by ``randint(1024, 2049)``, then the tensors
  of the global layer (4 KV heads, whole prefix cached, base 1e7, no sink) and of the SWA layer (8 KV heads,
  the last 128 rows cached, window 128, sink, base 1e4).
"""
from __future__ import annotations

import torch

HQ = 64
DQK = 192
DV = 128


def _gen(seed: int) -> torch.Generator:
    g = torch.Generator()
    g.manual_seed(seed)
    return g


def _randn_bf16(shape, g, device="cpu") -> torch.Tensor:
    return torch.randn(shape, generator=g, dtype=torch.float32).to(torch.bfloat16).to(device)


def cu_from_lengths(lengths) -> torch.Tensor:
    lens = torch.as_tensor(lengths, dtype=torch.int64)
    cu = torch.zeros(len(lens) + 1, dtype=torch.int64)
    cu[1:] = torch.cumsum(lens, 0)
    return cu.to(torch.int32)


def make_layer(lengths, n_q_heads, n_kv_heads, seed, with_sink, device="cpu", g=None):
    """q, k, v (bf16), sink (fp32 or None), cu_seqlens (int32) for the given sequence lengths."""
    g = g if g is not None else _gen(seed)
    cu = cu_from_lengths(lengths)
    T = int(cu[-1])
    q = _randn_bf16((T, n_q_heads, DQK), g, device)
    k = _randn_bf16((T, n_kv_heads, DQK), g, device)
    v = _randn_bf16((T, n_kv_heads, DV), g, device)
    sink = torch.randn((n_q_heads,), generator=g, dtype=torch.float32).to(device) if with_sink else None
    return dict(q=q, k=k, v=v, sink=sink, cu_seqlens=cu.to(device), lengths=[int(x) for x in lengths])


def swa_512(device="cpu"):
    d = make_layer([512], HQ, 8, 0, True, device)
    d.update(window=128, rope_base=1e4)
    return d


def global_2x4096(device="cpu"):
    d = make_layer([4096, 4096], HQ, 4, 1, False, device)
    d.update(window=-1, rope_base=1e7)
    return d


def thd_lengths(seed=2, total=32768, n=16, lo=1024, hi=2048, g=None):
    g = g if g is not None else _gen(seed)
    lens = torch.randint(lo, hi + 1, (n,), generator=g).tolist()
    pad = total - sum(lens)
    if pad < 0:
        raise ValueError("drawn lengths exceed the total")
    return lens + [pad], g


def thd_32k(device="cpu", total=32768):
    """Both layers of the 32768-token THD batch: dict(swa=..., glb=...) sharing cu_seqlens."""
    lens, g = thd_lengths(2, total)
    swa = make_layer(lens, HQ, 8, None, True, device, g=g)
    swa.update(window=128, rope_base=1e4)
    glb = make_layer(lens, HQ, 4, None, False, device, g=g)
    glb.update(window=-1, rope_base=1e7)
    return dict(swa=swa, glb=glb)


def dout_like(T, seed=4, n_q_heads=HQ, device="cpu"):
    return _randn_bf16((T, n_q_heads, DV), _gen(seed), device)


def decode_swa(batch=64, ring=128, n_kv_heads=8, seed=3, device="cpu", pos_lo=8192, pos_hi=131072):
    g = _gen(seed)
    positions = torch.randint(pos_lo, pos_hi + 1, (batch,), generator=g).to(torch.int32)
    q = _randn_bf16((batch, HQ, DQK), g, device)
    k_new = _randn_bf16((batch, n_kv_heads, DQK), g, device)
    v_new = _randn_bf16((batch, n_kv_heads, DV), g, device)
    sink = torch.randn((HQ,), generator=g, dtype=torch.float32).to(device)
    lens = [min(ring, int(p)) for p in positions]
    cu = cu_from_lengths(lens)
    Tc = int(cu[-1])
    k_cache = _randn_bf16((Tc, n_kv_heads, DQK), g, device)
    v_cache = _randn_bf16((Tc, n_kv_heads, DV), g, device)
    return dict(q=q, k_new=k_new, v_new=v_new, k_cache=k_cache, v_cache=v_cache, cu_cache=cu.to(device),
                positions=positions.to(device), sink=sink, window=ring, rope_base=1e4, n_kv_heads=n_kv_heads)


def decode_global(batch=64, n_kv_heads=4, seed=3, device="cpu", len_lo=8192, len_hi=131072):
    g = _gen(seed)
    lens = torch.randint(len_lo, len_hi + 1, (batch,), generator=g).to(torch.int32)
    q = _randn_bf16((batch, HQ, DQK), g, device)
    k_new = _randn_bf16((batch, n_kv_heads, DQK), g, device)
    v_new = _randn_bf16((batch, n_kv_heads, DV), g, device)
    cu = cu_from_lengths(lens.tolist())
    Tc = int(cu[-1])
    dev = torch.device(device)
    if dev.type == "cpu":
        k_cache = _randn_bf16((Tc, n_kv_heads, DQK), g)
        v_cache = _randn_bf16((Tc, n_kv_heads, DV), g)
    else:
        gd = torch.Generator(device=dev)
        gd.manual_seed(seed + 1000)
        k_cache = torch.empty((Tc, n_kv_heads, DQK), dtype=torch.bfloat16, device=dev)
        v_cache = torch.empty((Tc, n_kv_heads, DV), dtype=torch.bfloat16, device=dev)
        # drawn in 256 Mi-element chunks to bound the fp32 temporary
        for t, d in ((k_cache, DQK), (v_cache, DV)):
            flat = t.view(-1)
            step = 1 << 28
            for s in range(0, flat.numel(), step):
                e = min(flat.numel(), s + step)
                flat[s:e] = torch.randn((e - s,), generator=gd, device=dev, dtype=torch.float32).to(torch.bfloat16)
    return dict(q=q, k_new=k_new, v_new=v_new, k_cache=k_cache, v_cache=v_cache, cu_cache=cu.to(device),
                positions=lens.to(device), sink=None, window=-1, rope_base=1e7, n_kv_heads=n_kv_heads)


def make_cached(chunk_lengths, prefixes, n_q_heads, n_kv_heads, seed, with_sink, keep=None, device="cpu", g=None):
    """A prefill chunk over cached prefixes: q, k, v of the new tokens (bf16), sink, cu_seqlens (new tokens),
    k_cache, v_cache (bf16), cu_cache, positions (int32: the first new token's position = the prefix)."""
    g = g if g is not None else _gen(seed)
    d = make_layer(chunk_lengths, n_q_heads, n_kv_heads, None, with_sink, device, g=g)
    rows = [int(p) if keep is None else min(int(p), keep) for p in prefixes]
    cuc = cu_from_lengths(rows)
    Tc = int(cuc[-1])
    d["k_cache"] = _randn_bf16((Tc, n_kv_heads, DQK), g, device)
    d["v_cache"] = _randn_bf16((Tc, n_kv_heads, DV), g, device)
    d["cu_cache"] = cuc.to(device)
    d["positions"] = torch.as_tensor([int(p) for p in prefixes], dtype=torch.int32).to(device)
    d["cache_rows"] = rows
    d["max_position"] = max([int(p) + int(n) for p, n in zip(prefixes, chunk_lengths)] + [1])
    return d


def chunked_16(device="cpu", seed=5):
    """Both layers of a 16-sequence chunked prefill: dict(glb=..., swa=...)."""
    g = _gen(seed)
    prefixes = torch.randint(2048, 8193, (16,), generator=g).tolist()
    chunks = torch.randint(1024, 2049, (16,), generator=g).tolist()
    glb = make_cached(chunks, prefixes, HQ, 4, None, False, None, device, g=g)
    glb.update(window=-1, rope_base=1e7)
    swa = make_cached(chunks, prefixes, HQ, 8, None, True, 128, device, g=g)
    swa.update(window=128, rope_base=1e4)
    return dict(glb=glb, swa=swa)
