"""GPU backward parity against the fp64 oracle.

The backward is given the forward outputs; both sides receive the same O (the oracle's forward rounded to
bf16) and LSE (rounded to fp32), so D = rowsum(dO * O) uses the same O on both sides.  dq/dk/dv: max-abs
2e-2 on the unrounded value plus the bf16 rounding of it (parity.grad_bound), mean-abs 2e-3; dsink: 1e-2
relative per head.  Elements beyond the strict 2e-2 are counted per compare and summarised at session end.
Both backward paths run: "fast" (a workspace that keeps the dS blocks, which the dQ kernel reads back) and
"least" (the least workspace: dQ recomputes S and dP).
"""
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


def _given_outputs(d, rows=None):
    """Oracle forward (all rows) rounded to the forward's output types: O bf16 [T,hq,128], LSE fp32 [hq,T]."""
    o, l = oracle.prefill(d["q"], d["k"], d["v"], d["sink"], d["cu_seqlens"], d["window"], d["rope_base"])
    return torch.from_numpy(o).to(torch.bfloat16), torch.from_numpy(l).to(torch.float32)


def _run_bwd(ga, d, O, L, dO, path="fast", q_rot=None, k_rot=None):
    dev = "cuda"
    sink = None if d["sink"] is None else d["sink"].to(dev)
    T, hq, hkv = d["q"].shape[0], d["q"].shape[1], d["k"].shape[1]
    maxl = max(d["lengths"] + [1])
    if path == "fast":
        n = ga.bwd_workspace_size(T, hq, hkv, d["window"], len(d["lengths"]), maxl)
    else:
        n = ga.bwd_workspace_size(T, hq, hkv, d["window"])
    ws = torch.empty(max(n, 1), dtype=torch.uint8, device=dev)
    g = ga.bwd(d["q"].to(dev), d["k"].to(dev), d["v"].to(dev), sink, O.to(dev), L.to(dev), dO.to(dev),
               d["cu_seqlens"].to(dev), maxl, d["window"], d["rope_base"], workspace=ws, q_rot=q_rot,
               k_rot=k_rot)
    torch.cuda.synchronize()
    return [None if x is None else x.cpu() for x in g]


@pytest.mark.parametrize("lengths,hq,hkv,window,base,sink", [
    ([512], 64, 8, 128, 1e4, True),
    ([1, 5, 63, 64, 65, 129, 200, 0, 300], 64, 8, 128, 1e4, True),
    ([1, 5, 63, 64, 65, 129, 200, 0, 300], 64, 4, -1, 1e7, False),
    ([17, 130, 1], 64, 4, -1, 1e7, True),
    ([70, 33, 257], 16, 8, 0, 1e4, True),
    ([100, 29], 12, 4, 40, 1e4, True),
    ([100, 29], 8, 1, -1, 1e4, False),
    ([33, 1, 31, 47, 16, 17], 32, 8, 3, 1e4, True),
    ([129, 64, 250], 64, 4, 128, 1e4, True),    # 16 heads per KV head on a sliding-window layer
    ([300, 77], 64, 2, -1, 1e7, False),         # 32 heads per KV head on a causal layer
    ([200, 131, 67], 16, 2, 63, 1e4, True),     # windows near 64: the two halves of a key tile see
    ([190, 300], 16, 2, 65, 1e4, True),         # query ranges 64 apart, so their tile spans just touch
])
@pytest.mark.parametrize("path", ["fast", "least"])
def test_bwd_small_full(lengths, hq, hkv, window, base, sink, path):
    ga = _gpu()
    d = mi.make_layer(lengths, hq, hkv, 9, sink)
    d.update(window=window, rope_base=base)
    print(f"case lengths={lengths} hq={hq} hkv={hkv} window={window} sink={sink} path={path}", flush=True)
    O, L = _given_outputs(d)
    dO = mi.dout_like(sum(lengths), 4, hq)
    dq, dk, dv, ds = _run_bwd(ga, d, O, L, dO, path)
    rq, rk, rv, rs = oracle.prefill_bwd(d["q"], d["k"], d["v"], d["sink"], dO, d["cu_seqlens"], window, base,
                                        out_given=O)
    compare("dq", dq, rq, grad=True)
    compare("dk", dk, rk, grad=True)
    compare("dv", dv, rv, grad=True)
    if sink:
        compare_rel("dsink", ds, rs)
    else:
        assert ds is None


@pytest.mark.parametrize("window,sink", [(128, True), (-1, False)])
def test_bwd_deterministic_and_paths_agree(window, sink):
    """Each path is bitwise repeatable; dk, dv and dsink come from the same kernels on both paths (the fast
    one only also keeps dS), so they agree bitwise; dq agrees to fp32 summation order."""
    ga = _gpu()
    d = mi.make_layer([700, 333, 95], 64, 8 if window >= 0 else 4, 10, sink)
    d.update(window=window, rope_base=1e4)
    O, L = _given_outputs(d)
    dO = mi.dout_like(1128, 4)
    print(f"case paths window={window}", flush=True)
    a = _run_bwd(ga, d, O, L, dO, "fast")
    b = _run_bwd(ga, d, O, L, dO, "fast")
    c = _run_bwd(ga, d, O, L, dO, "least")
    for x, y in zip(a, b):
        assert (x is None and y is None) or torch.equal(x, y)
    for x, y in zip(a[1:], c[1:]):
        assert (x is None and y is None) or torch.equal(x, y)
    diff = (a[0].float() - c[0].float()).abs()
    assert float(diff.max()) <= 2e-2 and float(diff.mean()) <= 1e-4, (float(diff.max()), float(diff.mean()))


def _sampled_bwd(ga, d, dO, nq, nk, heads, seed, path="fast", check_forward=False):
    """Full-size backward: the oracle computes the forward rows it needs, and then sampled dq rows, dk/dv rows
    near the ends of sequences (few queries see them under causal attention), and dsink for a few heads.
    check_forward: the oracle's forward is computed on every row anyway, so the GPU forward of the same
    batch is compared with it on every row too."""
    rng = np.random.default_rng(seed)
    T, hq, hkv = d["q"].shape[0], d["q"].shape[1], d["k"].shape[1]
    starts = np.concatenate([[0], np.cumsum(d["lengths"])])
    # the given forward outputs on every row (the GPU needs them all): oracle rows in chunks
    O = torch.empty(T, hq, 128, dtype=torch.bfloat16)
    L = torch.empty(hq, T, dtype=torch.float32)
    o, l = oracle.prefill_rows(d["q"], d["k"], d["v"], d["sink"], d["cu_seqlens"], d["window"], d["rope_base"])
    O[:] = torch.from_numpy(o.reshape(T, hq, 128)).to(torch.bfloat16)
    L[:] = torch.from_numpy(l.reshape(T, hq).T.copy()).to(torch.float32)
    if check_forward:
        dev = "cuda"
        sink = None if d["sink"] is None else d["sink"].to(dev)
        go, gl = ga.fwd(d["q"].to(dev), d["k"].to(dev), d["v"].to(dev), sink, d["cu_seqlens"].to(dev),
                        max(d["lengths"]), d["window"], d["rope_base"])
        torch.cuda.synchronize()
        compare("fwd out (every row)", go.cpu().reshape(-1, 128), o)
        compare("fwd lse (every row)", gl.cpu().T.reshape(-1), l)
        del go, gl
    dq, dk, dv, ds = _run_bwd(ga, d, O, L, dO, path)
    qrows = rng.integers(0, T * hq, nq)
    rq = oracle.bwd_dq_rows(d["q"], d["k"], d["v"], d["sink"], dO, d["cu_seqlens"], d["window"], d["rope_base"],
                            qrows, out_given=O)
    compare("dq (sampled)", dq.reshape(-1, 192)[qrows], rq, grad=True)
    toks = []
    for b in range(len(d["lengths"])):
        if d["lengths"][b]:
            end = starts[b + 1]
            toks += [end - 1, end - 2, max(starts[b], end - 50)] + rng.integers(starts[b], end, 1).tolist()
    toks = np.array(sorted(set(toks)))[:nk]
    krows = toks * hkv + rng.integers(0, hkv, len(toks))
    rk, rv = oracle.bwd_dkv_rows(d["q"], d["k"], d["v"], d["sink"], dO, d["cu_seqlens"], d["window"],
                                 d["rope_base"], krows, out_given=O)
    compare("dk (sampled)", dk.reshape(-1, 192)[krows], rk, grad=True)
    compare("dv (sampled)", dv.reshape(-1, 128)[krows], rv, grad=True)
    if d["sink"] is not None:
        rs = oracle.bwd_dsink_heads(d["q"], d["k"], d["v"], d["sink"], dO, d["cu_seqlens"], d["window"],
                                    d["rope_base"], heads, out_given=O)
        compare_rel("dsink (sampled heads)", ds[heads], rs)


def test_bwd_thd_32k_swa_sampled():
    """SWA layer of the 32768-token THD batch with dO ~ N(0,1) seed 4: the forward on every row, the backward
    on sampled rows, 4 full dsink heads."""
    ga = _gpu()
    d = mi.thd_32k()["swa"]
    dO = mi.dout_like(32768, 4)
    print("case thd_32k swa fwd (every row) + bwd", flush=True)
    _sampled_bwd(ga, d, dO, 400, 60, [0, 17, 40, 63], 3, check_forward=True)


@pytest.mark.parametrize("path", ["fast", "least"])
def test_bwd_thd_32k_global_sampled(path):
    """Global layer of the 32768-token THD batch, the launch the benchmark times, checked on sampled rows.

    The oracle's forward over all 2.1 M (token, head) rows is too slow for a test, and none is needed: dq of
    row i depends on the forward outputs of row i only (through D_i and LSE_i), and dk/dv of key j on those
    of the queries that see j, which under causal attention are the tokens from j to the end of its
    sequence.  The oracle computes O and LSE exactly on every row the sampled gradients depend on; every
    other row gets O = 0 and LSE = 1e4, which make its probabilities and D exactly zero, so it adds nothing
    to any gradient (and no inf or NaN) whatever its true value."""
    ga = _gpu()
    d = mi.thd_32k()["glb"]
    dO = mi.dout_like(32768, 4)
    T, hq, hkv = d["q"].shape[0], d["q"].shape[1], d["k"].shape[1]
    G = hq // hkv
    starts = np.concatenate([[0], np.cumsum(d["lengths"])])
    rng = np.random.default_rng(7)
    # sampled dq rows: first and last token of every sequence, and random rows
    qtok = [int(starts[b]) for b in range(len(d["lengths"]))] + [int(starts[b + 1]) - 1 for b in range(len(d["lengths"]))]
    qrows = np.array(sorted(set(t * hq + int(rng.integers(0, hq)) for t in qtok)
                            | set(rng.integers(0, T * hq, 160).tolist())), dtype=np.int64)
    # sampled key rows: 1, 2, 33 and 100 tokens before the end of every sequence (ragged against the tiles)
    ktok = sorted(set(int(starts[b + 1]) - m for b in range(len(d["lengths"])) for m in (1, 2, 33, 100)
                      if int(starts[b + 1]) - m >= int(starts[b])))
    krows = np.array([t * hkv + int(rng.integers(0, hkv)) for t in ktok], dtype=np.int64)
    need = set(qrows.tolist())
    seq_of = np.searchsorted(starts, np.arange(T), side="right") - 1
    for kr in krows.tolist():
        t, g = kr // hkv, kr % hkv
        e = int(starts[seq_of[t] + 1])
        need.update(i * hq + g * G + h for i in range(t, e) for h in range(G))
    need = np.array(sorted(need), dtype=np.int64)
    print(f"case thd_32k glb bwd path={path}: {len(need)} oracle forward rows, {len(qrows)} dq rows, "
          f"{len(krows)} dk/dv rows", flush=True)
    o, l = oracle.prefill_rows(d["q"], d["k"], d["v"], d["sink"], d["cu_seqlens"], d["window"], d["rope_base"],
                               rows=need)
    O = torch.zeros(T * hq, 128, dtype=torch.bfloat16)
    O[torch.from_numpy(need)] = torch.from_numpy(o).to(torch.bfloat16)
    O = O.reshape(T, hq, 128)
    L = torch.full((T * hq,), 1e4, dtype=torch.float32)
    L[torch.from_numpy(need)] = torch.from_numpy(l).to(torch.float32)
    L = L.reshape(T, hq).T.contiguous()
    dq, dk, dv, _ = _run_bwd(ga, d, O, L, dO, path)
    rq = oracle.bwd_dq_rows(d["q"], d["k"], d["v"], d["sink"], dO, d["cu_seqlens"], d["window"], d["rope_base"],
                            qrows, out_given=O)
    compare("dq (sampled)", dq.reshape(-1, 192)[qrows], rq, grad=True)
    rk, rv = oracle.bwd_dkv_rows(d["q"], d["k"], d["v"], d["sink"], dO, d["cu_seqlens"], d["window"],
                                 d["rope_base"], krows, out_given=O)
    compare("dk (sampled)", dk.reshape(-1, 192)[krows], rk, grad=True)
    compare("dv (sampled)", dv.reshape(-1, 128)[krows], rv, grad=True)


@pytest.mark.parametrize("path", ["fast", "least"])
def test_bwd_global_small_batch_sampled(path):
    """Global layer on a 2 x 2048 batch (the oracle's full forward stays fast): sampled rows."""
    ga = _gpu()
    d = mi.make_layer([2048, 1999], 64, 4, 11, False)
    d.update(window=-1, rope_base=1e7)
    dO = mi.dout_like(4047, 4)
    print(f"case global 2048+1999 bwd path={path}", flush=True)
    _sampled_bwd(ga, d, dO, 300, 40, [], 4, path)


@pytest.mark.parametrize("lengths,hkv,window", [([33, 1, 31, 47, 16, 17], 8, 3), ([700, 333, 95], 4, -1)])
@pytest.mark.parametrize("path", ["fast", "least"])
def test_bwd_with_forward_q_rot(lengths, hkv, window, path):
    """Handing the backward the forward's rotated q gives bitwise the gradients of the backward's own
    rotation pass (the same table and rounding), including the last query tile, which reads past the T rows
    of the caller's buffer (clamped)."""
    ga = _gpu()
    d = mi.make_layer(lengths, 64, hkv, 12, window >= 0)
    d.update(window=window, rope_base=1e4)
    print(f"case q_rot bwd lengths={lengths} path={path}", flush=True)
    dev = "cuda"
    qr = torch.empty(d["q"].shape, dtype=torch.bfloat16, device=dev)
    sink = None if d["sink"] is None else d["sink"].to(dev)
    O, L = ga.fwd(d["q"].to(dev), d["k"].to(dev), d["v"].to(dev), sink, d["cu_seqlens"].to(dev), max(lengths),
                  window, 1e4, q_rot=qr)
    O, L = O.cpu(), L.cpu()
    dO = mi.dout_like(sum(lengths), 4)
    a = _run_bwd(ga, d, O, L, dO, path)
    b = _run_bwd(ga, d, O, L, dO, path, q_rot=qr)
    for x, y in zip(a, b):
        assert (x is None and y is None) or torch.equal(x, y)


@pytest.mark.parametrize("lengths,hkv,window", [([33, 1, 31, 47, 16, 17], 8, 3), ([700, 333, 95], 4, -1),
                                                ([129, 64, 250], 8, 128)])
@pytest.mark.parametrize("path", ["fast", "least"])
def test_bwd_with_forward_k_rot(lengths, hkv, window, path):
    """Handing the backward the forward's rotated k (with q_rot too) gives bitwise the gradients of the
    backward's own rotation passes, including the key tiles of the dQ kernel that reach past the T rows of
    the caller's buffer (clamped); the least-workspace path ignores it.  The k_rot output itself is RoPE
    applied at each key's position in its own sequence (the oracle's fp64 rotation, to one bf16 rounding)."""
    ga = _gpu()
    d = mi.make_layer(lengths, 64, hkv, 13, window >= 0)
    d.update(window=window, rope_base=1e4)
    print(f"case k_rot bwd lengths={lengths} path={path}", flush=True)
    dev = "cuda"
    qr = torch.empty(d["q"].shape, dtype=torch.bfloat16, device=dev)
    kr = torch.full(d["k"].shape, float("nan"), dtype=torch.bfloat16, device=dev)
    sink = None if d["sink"] is None else d["sink"].to(dev)
    O, L = ga.fwd(d["q"].to(dev), d["k"].to(dev), d["v"].to(dev), sink, d["cu_seqlens"].to(dev), max(lengths),
                  window, 1e4, q_rot=qr, k_rot=kr)
    O, L = O.cpu(), L.cpu()
    T = sum(lengths)
    pos = np.concatenate([np.arange(n) for n in lengths]).astype(np.int32)
    ref = oracle.rope(d["k"].reshape(T * hkv, 192), np.repeat(pos, hkv), 1e4)
    got = kr.cpu().float().numpy().reshape(T * hkv, 192)
    assert np.isfinite(got).all()
    assert (np.abs(got - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-6).all()
    dO = mi.dout_like(T, 4)
    a = _run_bwd(ga, d, O, L, dO, path, q_rot=qr)
    b = _run_bwd(ga, d, O, L, dO, path, q_rot=qr, k_rot=kr)
    c = _run_bwd(ga, d, O, L, dO, path, k_rot=kr)          # k handed over, q rotated by the backward
    for x, y, z in zip(a, b, c):
        assert (x is None and y is None and z is None) or (torch.equal(x, y) and torch.equal(x, z))


@pytest.mark.parametrize("window,hkv,sink", [(128, 4, True), (-1, 4, False)])
@pytest.mark.parametrize("path", ["fast", "least"])
def test_bwd_many_sequences(window, hkv, sink, path):
    """More than 64 sequences (work items are located 64 sequences at a time): 100 ragged sequences."""
    ga = _gpu()
    rng = np.random.default_rng(22)
    lengths = [int(x) for x in rng.integers(0, 41, 100)]
    d = mi.make_layer(lengths, 16, hkv, 14, sink)
    d.update(window=window, rope_base=1e4)
    print(f"case bwd many sequences window={window} path={path}", flush=True)
    O, L = _given_outputs(d)
    dO = mi.dout_like(sum(lengths), 4, 16)
    dq, dk, dv, ds = _run_bwd(ga, d, O, L, dO, path)
    rq, rk, rv, rs = oracle.prefill_bwd(d["q"], d["k"], d["v"], d["sink"], dO, d["cu_seqlens"], window, 1e4,
                                        out_given=O)
    compare("dq", dq, rq, grad=True)
    compare("dk", dk, rk, grad=True)
    compare("dv", dv, rv, grad=True)
    if sink:
        compare_rel("dsink", ds, rs)
