"""GPU parity at the serving engine's long sizes (SGLang cookbook page "MiMo-V2.6", section 2 "Configuration
tips", "Context length and memory": chunked prefill of up to 49152 tokens, 65536 prefill tokens per batch):

  * a 49152-token chunk over cached prefixes of up to 70000 rows (global layer with the whole prefix cached,
    sliding-window layer with the last 128 rows), sampled rows against the oracle;
  * a 65536-token THD batch (16 lengths in [1024, 2048] plus a pad sequence of about 41000 tokens, so the
    offsets inside one sequence pass 32768), forward on sampled rows and the backward with the least workspace
    (the stored-dS workspace bound exceeds the card at this size) on sampled dq and dk/dv rows.

The backward's oracle needs forward outputs only on the rows the sampled gradients depend on: dq of row i on
row i, dk/dv of key j on the queries that see j.  Those rows get the oracle's O and LSE; every other row gets
O = 0 and LSE = 1e4, which make its probabilities and D exactly zero, so it adds nothing to any gradient."""
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


@pytest.mark.parametrize("layer", ["glb", "swa"])
def test_prefill_cached_49152_token_chunk(layer):
    ga = _gpu()
    chunks, prefixes = [40000, 8000, 1152], [30000, 70000, 0]
    swa = layer == "swa"
    d = mi.make_cached(chunks, prefixes, 64, 8 if swa else 4, 70, swa, 128 if swa else None)
    window, base = (128, 1e4) if swa else (-1, 1e7)
    T = sum(chunks)
    assert T == 49152
    print(f"case prefill_cached 49152-token chunk {layer}: cache rows {d['cache_rows']}", flush=True)
    dev = "cuda"
    t = lambda x: None if x is None else x.to(dev)  # noqa: E731
    out, lse = ga.prefill_cached(t(d["q"]), t(d["k"]), t(d["v"]), t(d["k_cache"]), t(d["v_cache"]), t(d["sink"]),
                                 t(d["cu_seqlens"]), t(d["cu_cache"]), t(d["positions"]), max(chunks),
                                 d["max_position"], window, base)
    torch.cuda.synchronize()
    out, lse = out.cpu(), lse.cpu()
    assert torch.isfinite(out.float()).all()
    rng = np.random.default_rng(71)
    starts = np.concatenate([[0], np.cumsum(chunks)])
    toks = set(rng.integers(0, T, 120).tolist())
    for b in range(len(chunks)):
        toks.update([int(starts[b]), int(starts[b]) + 1, int(starts[b + 1]) - 1, int(starts[b]) + 129])
    toks = np.array(sorted(toks))
    rows = toks * 64 + rng.integers(0, 64, len(toks))
    ro, rl = oracle.prefill_cached_rows(d["q"], d["k"], d["v"], d["k_cache"], d["v_cache"], d["cu_seqlens"],
                                        d["cu_cache"], d["positions"], d["sink"], window, base, rows=rows)
    compare("out (sampled)", out.reshape(-1, 128)[rows], ro)
    compare("lse (sampled)", lse.T.reshape(-1)[rows], rl)


def _needed_rows(starts, seq_of, qrows, krows, hq, hkv, window):
    """Forward rows (token * hq + head) the sampled gradients depend on."""
    G = hq // hkv
    need = set(int(r) for r in qrows)
    for kr in krows.tolist():
        tok, g = kr // hkv, kr % hkv
        e = int(starts[seq_of[tok] + 1])
        last = e if window < 0 else min(e, tok + window + 1)
        need.update(i * hq + g * G + h for i in range(tok, last) for h in range(G))
    return np.array(sorted(need), dtype=np.int64)


@pytest.mark.parametrize("layer", ["glb", "swa"])
def test_thd_65536_fwd_and_least_workspace_bwd(layer):
    ga = _gpu()
    lens, g = mi.thd_lengths(80, 65536)
    swa = layer == "swa"
    d = mi.make_layer(lens, 64, 8 if swa else 4, None, swa, g=g)
    window, base = (128, 1e4) if swa else (-1, 1e7)
    T, hq, hkv = 65536, 64, d["k"].shape[1]
    assert sum(lens) == T and max(lens) > 32768
    print(f"case thd 65536 {layer}: longest sequence {max(lens)}", flush=True)
    dev = "cuda"
    sink = None if d["sink"] is None else d["sink"].to(dev)
    q, k, v, cu = d["q"].to(dev), d["k"].to(dev), d["v"].to(dev), d["cu_seqlens"].to(dev)
    out, lse = ga.fwd(q, k, v, sink, cu, max(lens), window, base)
    torch.cuda.synchronize()
    out, lse = out.cpu(), lse.cpu()
    rng = np.random.default_rng(81)
    starts = np.concatenate([[0], np.cumsum(lens)])
    seq_of = np.searchsorted(starts, np.arange(T), side="right") - 1
    # forward: first, last and window-edge tokens of every sequence, deep rows of the long one, random rows
    ftok = set(rng.integers(0, T, 150).tolist()) | set(rng.integers(int(starts[-2]) + 32768, T, 20).tolist())
    for b in range(len(lens)):
        ftok.update([int(starts[b]), int(starts[b + 1]) - 1, int(starts[b]) + 128, int(starts[b]) + 129])
    ftok = np.array(sorted(ftok))
    frows = ftok * hq + rng.integers(0, hq, len(ftok))
    ro, rl = oracle.prefill_rows(d["q"], d["k"], d["v"], d["sink"], d["cu_seqlens"], window, base, rows=frows)
    compare("fwd out (sampled)", out.reshape(-1, 128)[frows], ro)
    compare("fwd lse (sampled)", lse.T.reshape(-1)[frows], rl)

    # backward with the least workspace
    dO = mi.dout_like(T, 4)
    qtok = [int(starts[b]) for b in range(len(lens))] + [int(starts[b + 1]) - 1 for b in range(len(lens))]
    qrows = np.array(sorted(set(t * hq + int(rng.integers(0, hq)) for t in qtok)
                            | set(rng.integers(0, T * hq, 120).tolist())
                            | set((rng.integers(int(starts[-2]) + 32768, T, 20) * hq).tolist())), dtype=np.int64)
    ktok = sorted(set(int(starts[b + 1]) - m for b in range(len(lens)) for m in (1, 2, 33, 100)
                      if int(starts[b + 1]) - m >= int(starts[b])))
    if swa:      # every key of a sliding-window layer has few queries: add random ones
        ktok = sorted(set(ktok) | set(rng.integers(0, T, 40).tolist()))
    krows = np.array([t * hkv + int(rng.integers(0, hkv)) for t in ktok], dtype=np.int64)
    need = _needed_rows(starts, seq_of, qrows, krows, hq, hkv, window)
    print(f"  backward: {len(need)} oracle forward rows, {len(qrows)} dq rows, {len(krows)} dk/dv rows", flush=True)
    o, l = oracle.prefill_rows(d["q"], d["k"], d["v"], d["sink"], d["cu_seqlens"], window, base, rows=need)
    O = torch.zeros(T * hq, 128, dtype=torch.bfloat16)
    O[torch.from_numpy(need)] = torch.from_numpy(o).to(torch.bfloat16)
    O = O.reshape(T, hq, 128)
    L = torch.full((T * hq,), 1e4, dtype=torch.float32)
    L[torch.from_numpy(need)] = torch.from_numpy(l).to(torch.float32)
    L = L.reshape(T, hq).T.contiguous()
    ws = torch.empty(ga.bwd_workspace_size(T, hq, hkv, window), dtype=torch.uint8, device=dev)
    dq, dk, dv, ds = ga.bwd(q, k, v, sink, O.to(dev), L.to(dev), dO.to(dev), cu, max(lens), window, base,
                            workspace=ws)
    torch.cuda.synchronize()
    dq, dk, dv = dq.cpu(), dk.cpu(), dv.cpu()
    rq = oracle.bwd_dq_rows(d["q"], d["k"], d["v"], d["sink"], dO, d["cu_seqlens"], window, base, qrows,
                            out_given=O)
    compare("dq (sampled)", dq.reshape(-1, 192)[qrows], rq, grad=True)
    rk, rv = oracle.bwd_dkv_rows(d["q"], d["k"], d["v"], d["sink"], dO, d["cu_seqlens"], window, base, krows,
                                 out_given=O)
    compare("dk (sampled)", dk.reshape(-1, 192)[krows], rk, grad=True)
    compare("dv (sampled)", dv.reshape(-1, 128)[krows], rv, grad=True)
    if swa:
        # dsink sums over every row of a head: the rows without oracle outputs contribute exactly zero on
        # both sides (their LSE of 1e4 makes exp(sink - LSE) zero), so the given-outputs reading still holds
        G = hq // hkv
        g0 = int(krows[0] % hkv)
        heads = [g0 * G, g0 * G + G - 1]     # heads whose rows after the first sampled key have oracle outputs
        rs = oracle.bwd_dsink_heads(d["q"], d["k"], d["v"], d["sink"], dO, d["cu_seqlens"], window, base, heads,
                                    out_given=O)
        compare_rel("dsink (2 heads)", ds.cpu()[heads], rs)
