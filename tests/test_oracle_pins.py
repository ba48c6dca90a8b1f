"""Pins for the fp64 oracle: every check compares it with something other than itself.

Pins used (none of them re-types the oracle's formulas):
  * closed forms with all scores equal (q = 0): output and LSE depend only on the number of visible keys and
    the sink, which pins the 129-key window, the sink's place in the denominator and the 0.707 V scale;
  * brute force on tiny inputs: perturb one V (or K) row and record which outputs move -- the set must be the
    window the pages state (the query plus 128 previous keys inside its own sequence);
  * library routine: torch's scaled_dot_product_attention in fp64 (with explicit masks, repeated KV heads and
    the sink as an extra zero-valued key carrying an additive logit), after rotating Q/K with an independent
    complex-number form of rotate-half RoPE;
  * special cases the pages fix: sink = -inf equals no sink; window >= L-1 equals causal; GQA equals
    repeated KV heads; only dims 0..63 rotate; zero-length sequences change nothing;
  * calculus: central finite differences of sum(O * dO) in fp64 for dq, dk, dv and dsink;
  * decode equals the matching prefill row, and is invariant to the order of the cache rows.
Sources: miles PR "feat(models): add MiMo-V2.6-Flash-RL support" (PR body / commit messages), miles docs
"MiMo-V2.6-Flash" sections 1, 5.1 and 5.4, Megatron-Bridge "mimo_v2_flash_bridge" module summary.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from mimo_inputs import cu_from_lengths

DQK, DV, ROT = 192, 128, 64


def f64_layer(lengths, hq, hkv, seed, sink=True, scale=1.0):
    g = torch.Generator().manual_seed(seed)
    T = sum(lengths)
    q = torch.randn(T, hq, DQK, generator=g, dtype=torch.float64) * scale
    k = torch.randn(T, hkv, DQK, generator=g, dtype=torch.float64) * scale
    v = torch.randn(T, hkv, DV, generator=g, dtype=torch.float64)
    s = torch.randn(hq, generator=g, dtype=torch.float64) if sink else None
    return q, k, v, s, cu_from_lengths(lengths)


def positions_of(lengths):
    return np.concatenate([np.arange(n) for n in lengths]) if lengths else np.zeros(0, np.int64)


def window_sets(lengths, window):
    """W(i) for every token, from the pages' statement: own sequence, causal, at most `window` back."""
    out, start = [], 0
    for n in lengths:
        for p in range(n):
            lo = 0 if window < 0 else max(0, p - window)
            out.append(set(range(start + lo, start + p + 1)))
        start += n
    return out


# --------------------------------------------------------------------------------------------------------
# independent RoPE (complex multiplication) and the library attention routine
# --------------------------------------------------------------------------------------------------------
def rope_complex(x, pos, base):
    """Rotate-half RoPE written as multiplication of z = x[:32] + i x[32:64] by exp(i p base^(-d/32))."""
    x = np.asarray(x, np.float64).copy()
    z = x[..., :32] + 1j * x[..., 32:64]
    inv = base ** (-np.arange(32) / 32.0)
    ang = np.asarray(pos, np.float64)[:, None] * inv[None, :]
    shape = [x.shape[0]] + [1] * (x.ndim - 2) + [32]
    z = z * np.exp(1j * ang).reshape(shape)
    x[..., :32] = z.real
    x[..., 32:64] = z.imag
    return x


def sdpa_reference(q, k, v, sink, lengths, window, base):
    """Layer output via torch.nn.functional.scaled_dot_product_attention (fp64 CPU), per sequence."""
    hq, hkv = q.shape[1], k.shape[1]
    G = hq // hkv
    pos = positions_of(lengths)
    qr = torch.from_numpy(rope_complex(q.numpy(), pos, base))
    kr = torch.from_numpy(rope_complex(k.numpy(), pos, base))
    outs, start = [], 0
    for n in lengths:
        if n == 0:
            continue
        Q = qr[start:start + n].permute(1, 0, 2)                                   # [hq, n, 192]
        K = kr[start:start + n].repeat_interleave(G, dim=1).permute(1, 0, 2)       # [hq, n, 192]
        V = v[start:start + n].repeat_interleave(G, dim=1).permute(1, 0, 2) * 0.707
        i = torch.arange(n)[:, None]
        j = torch.arange(n)[None, :]
        ok = (j <= i) & ((j >= i - window) if window >= 0 else torch.ones_like(j <= i))
        bias = torch.where(ok, 0.0, -math.inf).to(torch.float64).expand(hq, n, n)
        if sink is not None:
            # the sink as one more key: q.k = 0 plus an additive logit sink_h, and a zero value
            K = torch.cat([K, torch.zeros(hq, 1, DQK, dtype=torch.float64)], 1)
            V = torch.cat([V, torch.zeros(hq, 1, DV, dtype=torch.float64)], 1)
            col = sink.to(torch.float64).view(hq, 1, 1).expand(hq, n, 1)
            bias = torch.cat([bias, col], 2)
        o = torch.nn.functional.scaled_dot_product_attention(Q, K, V, attn_mask=bias, scale=1 / math.sqrt(DQK))
        outs.append(o.permute(1, 0, 2))
        start += n
    return torch.cat(outs, 0).numpy() if outs else np.zeros((0, hq, DV))


def run(q, k, v, s, cu, window, base):
    return oracle.prefill(q, k, v, s, cu, window, base, nthreads=2)


# --------------------------------------------------------------------------------------------------------
# closed forms
# --------------------------------------------------------------------------------------------------------
@pytest.mark.parametrize("window", [128, 0, 5, -1])
def test_closed_form_equal_scores(window):
    """q = 0 makes every score 0: O = 0.707 n / (n + e^sink), LSE = ln(n + e^sink), n = visible keys."""
    lengths = [300, 7, 1]
    T, hq, hkv = sum(lengths), 4, 2
    q = torch.zeros(T, hq, DQK, dtype=torch.bfloat16)
    k = torch.randn(T, hkv, DQK).to(torch.bfloat16)
    v = torch.ones(T, hkv, DV, dtype=torch.bfloat16)
    sink = torch.tensor([0.3, -1.0, 2.0, -5.0])
    out, lse = run(q, k, v, sink, cu_from_lengths(lengths), window, 1e4)
    pos = positions_of(lengths)
    n = pos + 1 if window < 0 else np.minimum(pos + 1, window + 1)
    es = np.exp(sink.double().numpy())
    exp_o = 0.707 * n[:, None] / (n[:, None] + es[None, :])
    np.testing.assert_allclose(out, np.broadcast_to(exp_o[:, :, None], out.shape), rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse.T, np.log(n[:, None] + es[None, :]), rtol=0, atol=1e-12)
    if window == 128:
        assert n.max() == 129  # query + 128 previous keys


def test_closed_form_mean_of_window():
    """q = 0, no sink, v_j = position of j: O_i = 0.707 * mean of the positions in W(i)."""
    lengths = [260, 3]
    T = sum(lengths)
    pos = positions_of(lengths)
    q = torch.zeros(T, 1, DQK, dtype=torch.float64)
    k = torch.randn(T, 1, DQK, dtype=torch.float64)
    v = torch.from_numpy(np.repeat(pos.astype(np.float64)[:, None, None], DV, axis=2))
    out, _ = run(q, k, v, None, cu_from_lengths(lengths), 128, 1e4)
    lo = np.maximum(pos - 128, 0)
    exp = 0.707 * (lo + pos) / 2.0
    np.testing.assert_allclose(out[:, 0, :], np.repeat(exp[:, None], DV, 1), rtol=0, atol=1e-12)


# --------------------------------------------------------------------------------------------------------
# brute force: which keys does each query see?
# --------------------------------------------------------------------------------------------------------
@pytest.mark.parametrize("lengths,window", [([260], 128), ([40, 1, 25], 6), ([30, 12], -1), ([9], 0)])
def test_window_brute_force(lengths, window):
    q, k, v, s, cu = f64_layer(lengths, 1, 1, 7)
    T = sum(lengths)
    base, _ = run(q, k, v, s, cu, window, 1e4)
    seen = [set() for _ in range(T)]
    for j in range(T):
        v2 = v.clone()
        v2[j] += 1.0
        o2, _ = run(q, k, v2, s, cu, window, 1e4)
        moved = np.nonzero(np.abs(o2 - base).max(axis=(1, 2)) > 0)[0]
        for i in moved:
            seen[i].add(j)
    assert seen == window_sets(lengths, window)
    if window == 128:
        assert max(len(x) for x in seen) == 129


def test_key_perturbation_matches_window():
    lengths = [150]
    q, k, v, s, cu = f64_layer(lengths, 1, 1, 8)
    base, _ = run(q, k, v, s, cu, 128, 1e4)
    for j in (0, 21, 75, 149):
        k2 = k.clone()
        k2[j] += 0.5
        o2, _ = run(q, k2, v, s, cu, 128, 1e4)
        moved = set(np.nonzero(np.abs(o2 - base).max(axis=(1, 2)) > 0)[0].tolist())
        assert moved == set(range(j, min(150, j + 129)))


# --------------------------------------------------------------------------------------------------------
# library routine
# --------------------------------------------------------------------------------------------------------
@pytest.mark.parametrize("window,with_sink,base", [(128, True, 1e4), (-1, False, 1e7), (3, True, 1e7),
                                                   (-1, True, 1e4)])
def test_matches_torch_sdpa(window, with_sink, base):
    lengths = [200, 0, 37, 1]
    q, k, v, s, cu = f64_layer(lengths, 8, 2, 11, with_sink)
    out, lse = run(q, k, v, s, cu, window, base)
    ref = sdpa_reference(q, k, v, s, lengths, window, base)
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)


def test_rope_free_matches_sdpa_any_base():
    """Q/K zero on dims 0..63: RoPE has nothing to rotate, so the base must not matter."""
    lengths = [64, 20]
    q, k, v, s, cu = f64_layer(lengths, 4, 4, 12)
    q[..., :ROT] = 0
    k[..., :ROT] = 0
    o1, _ = run(q, k, v, s, cu, 128, 1e4)
    o2, _ = run(q, k, v, s, cu, 128, 1e7)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_allclose(o1, sdpa_reference(q, k, v, s, lengths, 128, 1.0), rtol=0, atol=1e-12)


# --------------------------------------------------------------------------------------------------------
# special cases fixed by the pages
# --------------------------------------------------------------------------------------------------------
def test_sink_minus_inf_is_no_sink():
    q, k, v, s, cu = f64_layer([50, 30], 4, 2, 13)
    o1, l1 = run(q, k, v, torch.full((4,), -math.inf, dtype=torch.float64), cu, 128, 1e4)
    o2, l2 = run(q, k, v, None, cu, 128, 1e4)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)


def test_large_sink_absorbs_everything():
    q, k, v, s, cu = f64_layer([20], 2, 1, 14)
    o, _ = run(q, k, v, torch.tensor([60.0, 60.0], dtype=torch.float64), cu, 128, 1e4)
    assert np.abs(o).max() < 1e-20


@pytest.mark.parametrize("extra", [0, 1, 50])
def test_window_covering_sequence_is_causal(extra):
    lengths = [70, 33]
    q, k, v, s, cu = f64_layer(lengths, 4, 2, 15)
    o1, l1 = run(q, k, v, s, cu, max(lengths) - 1 + extra, 1e4)
    o2, l2 = run(q, k, v, s, cu, -1, 1e4)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)


@pytest.mark.parametrize("hq,hkv", [(8, 2), (8, 1), (6, 3)])
def test_gqa_equals_repeated_kv(hq, hkv):
    lengths = [40, 25]
    q, k, v, s, cu = f64_layer(lengths, hq, hkv, 16)
    G = hq // hkv
    o1, l1 = run(q, k, v, s, cu, 5, 1e4)
    o2, l2 = run(q, k.repeat_interleave(G, 1), v.repeat_interleave(G, 1), s, cu, 5, 1e4)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)


def test_thd_is_concatenation_and_empty_sequences_are_noops():
    lengths = [33, 0, 17, 0, 0, 50]
    q, k, v, s, cu = f64_layer(lengths, 4, 2, 17)
    o, l = run(q, k, v, s, cu, 128, 1e7)
    start = 0
    for n in lengths:
        if n:
            sl = slice(start, start + n)
            o1, l1 = run(q[sl], k[sl], v[sl], s, cu_from_lengths([n]), 128, 1e7)
            np.testing.assert_array_equal(o[sl], o1)
            np.testing.assert_array_equal(l[:, sl], l1)
        start += n


# --------------------------------------------------------------------------------------------------------
# RoPE
# --------------------------------------------------------------------------------------------------------
def test_rope_properties():
    g = torch.Generator().manual_seed(18)
    x = torch.randn(200, DQK, generator=g, dtype=torch.float64)
    pos = np.random.default_rng(0).integers(0, 131072, 200)
    for base in (1e4, 1e7):
        r = oracle.rope(x, pos, base)
        np.testing.assert_array_equal(r[:, ROT:], x.numpy()[:, ROT:])             # dims 64..191 untouched
        np.testing.assert_allclose(np.linalg.norm(r, axis=1), np.linalg.norm(x.numpy(), axis=1), rtol=1e-13)
        np.testing.assert_array_equal(oracle.rope(x, np.zeros(200, np.int64), base), x.numpy())  # p = 0
        np.testing.assert_allclose(r, rope_complex(x.numpy(), pos, base), rtol=0, atol=1e-9)


def test_rope_relative_position():
    """Scores depend on positions only through their difference."""
    g = torch.Generator().manual_seed(19)
    q = torch.randn(50, DQK, generator=g, dtype=torch.float64)
    k = torch.randn(50, DQK, generator=g, dtype=torch.float64)
    rng = np.random.default_rng(1)
    pq = rng.integers(0, 4096, 50)
    pk = rng.integers(0, 4096, 50)
    shift = 100003
    for base in (1e4, 1e7):
        a = (oracle.rope(q, pq, base) * oracle.rope(k, pk, base)).sum(1)
        b = (oracle.rope(q, pq + shift, base) * oracle.rope(k, pk + shift, base)).sum(1)
        np.testing.assert_allclose(a, b, rtol=0, atol=1e-8)
        c = (oracle.rope(q, pq - pk + 5000, base) * oracle.rope(k, np.full(50, 5000), base)).sum(1)
        np.testing.assert_allclose(a, c, rtol=0, atol=1e-8)


def test_rope_bf16_input_decodes_exactly():
    x = torch.randn(10, DQK).to(torch.bfloat16)
    r1 = oracle.rope(x, np.arange(10), 1e4)
    r2 = oracle.rope(x.double(), np.arange(10), 1e4)
    np.testing.assert_array_equal(r1, r2)


# --------------------------------------------------------------------------------------------------------
# backward: central finite differences in fp64
# --------------------------------------------------------------------------------------------------------
def loss(q, k, v, s, cu, dO, window, base):
    o, _ = oracle.prefill(q, k, v, s, cu, window, base, nthreads=1)
    return float((o * dO).sum())


def fd(fn, x, idx, h=1e-6):
    x0 = x[idx].item()
    x[idx] = x0 + h
    lp = fn()
    x[idx] = x0 - h
    lm = fn()
    x[idx] = x0
    return (lp - lm) / (2 * h)


@pytest.mark.parametrize("window,with_sink,base", [(3, True, 1e4), (-1, False, 1e7), (-1, True, 10.0)])
def test_backward_finite_differences(window, with_sink, base):
    lengths = [9, 6]
    q, k, v, s, cu = f64_layer(lengths, 4, 2, 20, with_sink)
    T = sum(lengths)
    dO = np.random.default_rng(2).standard_normal((T, 4, DV))
    dq, dk, dv, ds = oracle.prefill_bwd(q, k, v, s, torch.from_numpy(dO), cu, window, base, nthreads=1)
    f = lambda: loss(q, k, v, s, cu, dO, window, base)  # noqa: E731
    rng = np.random.default_rng(3)
    checks = []
    # every rotated dim of a few rows, plus random elements elsewhere
    for t in (0, 5, 9, 14):
        for d in list(range(0, ROT, 3)) + [64, 100, 191]:
            checks.append(("q", (t, int(rng.integers(4)), d)))
            checks.append(("k", (t, int(rng.integers(2)), d)))
    for _ in range(40):
        checks.append(("v", (int(rng.integers(T)), int(rng.integers(2)), int(rng.integers(DV)))))
        checks.append(("q", (int(rng.integers(T)), int(rng.integers(4)), int(rng.integers(DQK)))))
        checks.append(("k", (int(rng.integers(T)), int(rng.integers(2)), int(rng.integers(DQK)))))
    tens = dict(q=(q, dq), k=(k, dk), v=(v, dv))
    for name, idx in checks:
        x, g = tens[name]
        num = fd(f, x, idx)
        assert abs(num - g[idx]) < 1e-7 * max(1.0, abs(num)), (name, idx, num, g[idx])
    if with_sink:
        for h in range(4):
            num = fd(f, s, (h,))
            assert abs(num - ds[h]) < 1e-7 * max(1.0, abs(num)), (h, num, ds[h])
    # directional derivative over all inputs at once
    u = {n: torch.from_numpy(rng.standard_normal(t[0].shape)) for n, t in tens.items()}
    eps = 1e-6
    def shifted(sign):  # noqa: E306
        return loss(q + sign * eps * u["q"], k + sign * eps * u["k"], v + sign * eps * u["v"], s, cu, dO, window, base)
    num = (shifted(1) - shifted(-1)) / (2 * eps)
    ana = sum(float((tens[n][1] * u[n].numpy()).sum()) for n in tens)
    assert abs(num - ana) < 1e-7 * max(1.0, abs(num))


def test_backward_given_exact_o_equals_exact_mode():
    lengths = [20, 11]
    q, k, v, s, cu = f64_layer(lengths, 4, 2, 21)
    dO = torch.randn(sum(lengths), 4, DV, dtype=torch.float64)
    o, _ = oracle.prefill(q, k, v, s, cu, 4, 1e4)
    a = oracle.prefill_bwd(q, k, v, s, dO, cu, 4, 1e4)
    b = oracle.prefill_bwd(q, k, v, s, dO, cu, 4, 1e4, out_given=torch.from_numpy(o))
    for x, y in zip(a, b):
        np.testing.assert_allclose(x, y, rtol=0, atol=1e-12)


def test_backward_dk_sums_to_zero_without_sink():
    """No sink, RoPE-free: every row of dS sums to zero, so the dk of a sequence and KV head sum to zero."""
    lengths = [30, 17]
    q, k, v, _, cu = f64_layer(lengths, 4, 2, 22, sink=False)
    q[..., :ROT] = 0
    k[..., :ROT] = 0
    dO = torch.randn(sum(lengths), 4, DV, dtype=torch.float64)
    _, dk, _, _ = oracle.prefill_bwd(q, k, v, None, dO, cu, 6, 1e4)
    np.testing.assert_allclose(dk[:30].sum(0), 0, atol=1e-12)
    np.testing.assert_allclose(dk[30:].sum(0), 0, atol=1e-12)


def test_sampled_backward_entry_points_agree_with_full():
    lengths = [40, 23]
    for window, with_sink in ((128, True), (-1, False), (5, True)):
        q, k, v, s, cu = f64_layer(lengths, 4, 2, 23, with_sink)
        q, k, v = q.to(torch.bfloat16), k.to(torch.bfloat16), v.to(torch.bfloat16)
        T = sum(lengths)
        dO = torch.randn(T, 4, DV).to(torch.bfloat16)
        og = oracle.prefill(q, k, v, s, cu, window, 1e4)[0]
        og = torch.from_numpy(og).to(torch.bfloat16)
        dq, dk, dv, ds = oracle.prefill_bwd(q, k, v, s, dO, cu, window, 1e4, out_given=og)
        rows = np.array([0, 5, 77, 4 * 40 + 3, 4 * T - 1])
        np.testing.assert_allclose(oracle.bwd_dq_rows(q, k, v, s, dO, cu, window, 1e4, rows, og),
                                   dq.reshape(-1, DQK)[rows], rtol=0, atol=1e-12)
        krows = np.array([0, 1, 2 * 39 + 1, 2 * 40, 2 * T - 1])
        a, b = oracle.bwd_dkv_rows(q, k, v, s, dO, cu, window, 1e4, krows, og)
        np.testing.assert_allclose(a, dk.reshape(-1, DQK)[krows], rtol=0, atol=1e-12)
        np.testing.assert_allclose(b, dv.reshape(-1, DV)[krows], rtol=0, atol=1e-12)
        if with_sink:
            np.testing.assert_allclose(oracle.bwd_dsink_heads(q, k, v, s, dO, cu, window, 1e4, [0, 3], og),
                                       ds[[0, 3]], rtol=1e-12, atol=1e-12)


# --------------------------------------------------------------------------------------------------------
# decode
# --------------------------------------------------------------------------------------------------------
@pytest.mark.parametrize("window,base,with_sink", [(128, 1e4, True), (-1, 1e7, False), (7, 1e4, True)])
def test_decode_equals_prefill_row(window, base, with_sink):
    lengths = [300, 140, 5, 1]
    q, k, v, s, cu = f64_layer(lengths, 8, 2, 24, with_sink)
    o_pre, l_pre = oracle.prefill(q, k, v, s, cu, window, base)
    B = len(lengths)
    starts = np.concatenate([[0], np.cumsum(lengths)])
    qd, kn, vn, kc, vc, cc, pos = [], [], [], [], [], [0], []
    for b, n in enumerate(lengths):
        t = starts[b] + n - 1
        qd.append(q[t]); kn.append(k[t]); vn.append(v[t])
        rows = np.arange(starts[b], t)
        kc.append(torch.from_numpy(rope_complex(k[rows].numpy(), np.arange(n - 1), base)))
        vc.append(v[rows])
        cc.append(cc[-1] + n - 1)
        pos.append(n - 1)
    out, lse = oracle.decode_rows(torch.stack(qd), torch.stack(kn), torch.stack(vn), torch.cat(kc), torch.cat(vc),
                                  np.array(cc), np.array(pos), s, window, base)
    last = starts[1:] - 1
    np.testing.assert_allclose(out.reshape(B, 8, DV), o_pre[last], rtol=0, atol=1e-10)
    np.testing.assert_allclose(lse.reshape(B, 8), l_pre[:, last].T, rtol=0, atol=1e-10)


def test_decode_cache_order_irrelevant_when_all_rows_visible():
    g = torch.Generator().manual_seed(25)
    B, hq, hkv, n = 3, 4, 2, 50
    q = torch.randn(B, hq, DQK, generator=g, dtype=torch.float64)
    kn = torch.randn(B, hkv, DQK, generator=g, dtype=torch.float64)
    vn = torch.randn(B, hkv, DV, generator=g, dtype=torch.float64)
    kc = torch.randn(B * n, hkv, DQK, generator=g, dtype=torch.float64)
    vc = torch.randn(B * n, hkv, DV, generator=g, dtype=torch.float64)
    cc = np.arange(B + 1) * n
    pos = np.array([50, 9000, 131072])
    sink = torch.randn(hq, generator=g, dtype=torch.float64)
    for window in (-1, n, n + 10):
        a, _ = oracle.decode_rows(q, kn, vn, kc, vc, cc, pos, sink, window, 1e4)
        perm = torch.cat([torch.randperm(n, generator=g) + b * n for b in range(B)])
        b_, _ = oracle.decode_rows(q, kn, vn, kc[perm], vc[perm], cc, pos, sink, window, 1e4)
        np.testing.assert_allclose(a, b_, rtol=0, atol=1e-12)


def test_decode_window_takes_last_rows():
    g = torch.Generator().manual_seed(26)
    q = torch.randn(1, 2, DQK, generator=g, dtype=torch.float64)
    kn = torch.randn(1, 1, DQK, generator=g, dtype=torch.float64)
    vn = torch.randn(1, 1, DV, generator=g, dtype=torch.float64)
    kc = torch.randn(20, 1, DQK, generator=g, dtype=torch.float64)
    vc = torch.randn(20, 1, DV, generator=g, dtype=torch.float64)
    a, _ = oracle.decode_rows(q, kn, vn, kc, vc, [0, 20], [100], None, 6, 1e4)
    b, _ = oracle.decode_rows(q, kn, vn, kc[14:], vc[14:], [0, 6], [100], None, -1, 1e4)
    np.testing.assert_array_equal(a, b)


# --------------------------------------------------------------------------------------------------------
# cached prefill (a chunk of new tokens over a cached prefix)
# --------------------------------------------------------------------------------------------------------
def split_for_cache(q, k, v, lengths, splits, base, keep=None):
    """The second parts of the sequences as a chunk over a cache that holds the first parts' rotated K
    (independent complex RoPE) and V; keep: cache only the last `keep` rows of each first part."""
    starts = np.concatenate([[0], np.cumsum(lengths)])
    qc, kn, vn, kc, vc, cuq, cuc, pos, rows = [], [], [], [], [], [0], [0], [], []
    for b, (n, s) in enumerate(zip(lengths, splits)):
        first = np.arange(starts[b], starts[b] + s)
        second = np.arange(starts[b] + s, starts[b] + n)
        c = first if keep is None else first[max(0, s - keep):]
        kc.append(torch.from_numpy(rope_complex(k[c].numpy(), c - starts[b], base)))
        vc.append(v[c])
        qc.append(q[second]); kn.append(k[second]); vn.append(v[second])
        cuq.append(cuq[-1] + len(second)); cuc.append(cuc[-1] + len(c)); pos.append(s)
        rows.extend(second.tolist())
    return (torch.cat(qc), torch.cat(kn), torch.cat(vn), torch.cat(kc), torch.cat(vc), np.array(cuq),
            np.array(cuc), np.array(pos), np.array(rows))


@pytest.mark.parametrize("window,base,with_sink,keep", [(128, 1e4, True, None), (7, 1e4, True, 7),
                                                        (-1, 1e7, False, None), (0, 1e4, True, 0)])
def test_cached_prefill_continues_a_prefill(window, base, with_sink, keep):
    """Prefill of the later tokens over a cache of the earlier ones equals the same rows of the whole
    prefill (the cache may drop rows outside the window)."""
    lengths, splits = [300, 140, 5, 1, 33], [170, 0, 5, 0, 32]
    q, k, v, s, cu = f64_layer(lengths, 8, 2, 31, with_sink)
    o_pre, l_pre = oracle.prefill(q, k, v, s, cu, window, base, nthreads=2)
    qc, kn, vn, kc, vc, cuq, cuc, pos, rows = split_for_cache(q, k, v, lengths, splits, base, keep)
    out, lse = oracle.prefill_cached_rows(qc, kn, vn, kc, vc, cuq, cuc, pos, s, window, base, nthreads=2)
    np.testing.assert_allclose(out.reshape(-1, 8, DV), o_pre[rows], rtol=0, atol=1e-10)
    np.testing.assert_allclose(lse.reshape(-1, 8), l_pre[:, rows].T, rtol=0, atol=1e-10)


def test_cached_prefill_without_cache_is_prefill():
    lengths = [40, 0, 17]
    q, k, v, s, cu = f64_layer(lengths, 4, 2, 32)
    for window in (5, -1):
        o_pre, l_pre = oracle.prefill(q, k, v, s, cu, window, 1e4)
        empty = torch.zeros(0, 2, DQK, dtype=torch.float64)
        out, lse = oracle.prefill_cached_rows(q, k, v, empty, torch.zeros(0, 2, DV, dtype=torch.float64), cu,
                                              np.zeros(4, np.int32), np.zeros(3, np.int32), s, window, 1e4)
        np.testing.assert_allclose(out.reshape(-1, 4, DV), o_pre, rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse.reshape(-1, 4), l_pre.T, rtol=0, atol=1e-12)


@pytest.mark.parametrize("window", [-1, 6, 50])
def test_cached_prefill_chunk_of_one_is_decode(window):
    g = torch.Generator().manual_seed(33)
    B, hq, hkv, n = 3, 4, 2, 20
    q = torch.randn(B, hq, DQK, generator=g, dtype=torch.float64)
    kn = torch.randn(B, hkv, DQK, generator=g, dtype=torch.float64)
    vn = torch.randn(B, hkv, DV, generator=g, dtype=torch.float64)
    kc = torch.randn(B * n, hkv, DQK, generator=g, dtype=torch.float64)
    vc = torch.randn(B * n, hkv, DV, generator=g, dtype=torch.float64)
    cc = np.arange(B + 1) * n
    pos = np.array([20, 900, 131072])
    sink = torch.randn(hq, generator=g, dtype=torch.float64)
    a, la = oracle.decode_rows(q, kn, vn, kc, vc, cc, pos, sink, window, 1e4)
    b, lb = oracle.prefill_cached_rows(q, kn, vn, kc, vc, np.arange(B + 1), cc, pos, sink, window, 1e4)
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-12)
    np.testing.assert_allclose(la, lb, rtol=0, atol=1e-12)


def test_cached_prefill_rejects_cache_longer_than_position():
    q, k, v, s, cu = f64_layer([4], 2, 1, 34)
    kc = torch.zeros(5, 1, DQK, dtype=torch.float64)
    vc = torch.zeros(5, 1, DV, dtype=torch.float64)
    with pytest.raises(ValueError):
        oracle.prefill_cached_rows(q, k, v, kc, vc, cu, np.array([0, 5]), np.array([4]), s, -1, 1e4)


def test_oracle_rejects_bad_arguments():
    q, k, v, s, cu = f64_layer([10], 4, 3, 27)
    with pytest.raises(ValueError):
        oracle.prefill(q, k, v, s, cu, 3, 1e4)          # 4 % 3 != 0
    q, k, v, s, cu = f64_layer([10], 4, 2, 27)
    with pytest.raises(ValueError):
        oracle.prefill(q, k, v, s, cu, -2, 1e4)         # window < -1
    with pytest.raises(ValueError):
        oracle.prefill(q, k, v, s, np.array([0, 11], np.int32), 3, 1e4)   # cu[-1] != T


def test_golden_window_closed_form():
    """tests/golden/window_closed_form.json: values that follow from the 129-key window and the 0.707 scale."""
    import json
    import os

    fx = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "window_closed_form.json")))
    L = max(r["position"] for r in fx["rows"]) + 1
    hq = len(fx["sinks"])
    q = torch.zeros(L, hq, DQK, dtype=torch.bfloat16)
    k = torch.randn(L, 1, DQK).to(torch.bfloat16)
    v = torch.ones(L, 1, DV, dtype=torch.bfloat16)
    out, lse = oracle.prefill(q, k, v, torch.tensor(fx["sinks"]), cu_from_lengths([L]), fx["window"], 1e4)
    for r in fx["rows"]:
        p = r["position"]
        np.testing.assert_allclose(out[p, :, 0], r["out"], rtol=0, atol=1e-13)
        np.testing.assert_allclose(lse[:, p], r["lse"], rtol=0, atol=1e-12)
