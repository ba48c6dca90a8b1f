"""The sliding-window dK/dV stage walk (attn_bwd.hip, bwd_dkdv_kernel with a window): the two halves of a
128-key tile (keys kb0 .. kb0 + 63 and the rest) each walk only the 32-query tiles that their keys see, one
tile of the same head per stage, so a head takes max(n_0, n_1) stages instead of nq.  Restated here from the
kernel's formulas and checked against the plain walk (every query tile of every head, the kernel's per-wave
visibility test): every 32-key block of the tile is given exactly the (query tile, head) steps it sees, each
once; every tile a half loads lies on the tile grid between q_lo and q_top; no GPU is used.
"""
import numpy as np
import pytest

NKB, MQ = 128, 32


def visible(q0, kw0, kb_last, window):
    """The kernel's per-wave test: does the 32-key block at kw0 see any query of the tile at q0?"""
    return not (q0 + MQ - 1 < kw0 or kw0 > kb_last or q0 > kw0 + 31 + window)


def geometry(seq_start, seq_end, tile, window):
    kb0 = seq_start + tile * NKB
    kb_last = min(kb0 + NKB - 1, seq_end - 1)
    q_lo = kb0 & ~15
    q_hi = min(seq_end - 1, kb_last + window)
    nq = (q_hi - q_lo + MQ) // MQ
    q_top = q_lo + (nq - 1) * MQ
    return kb0, kb_last, q_lo, q_top, nq


def half_range(kg0, kb_last, q_top, nq, window):
    """(first tile index counted from the top, tile count) of the half whose keys start at kg0."""
    if kg0 > kb_last:
        return 0, 0
    kg1 = min(kg0 + 63, kb_last)
    lo = max(0, (q_top - kg1 - window + MQ - 1) >> 5)
    hi = min(nq - 1, (q_top + MQ - 1 - kg0) >> 5)
    return lo, max(0, hi - lo + 1)


def skewed_steps(seq_start, seq_end, tile, window, heads):
    """{kq: [(q0, h), ...]} in stage order, and the tiles each half loads, from the kernel's stage walk."""
    kb0, kb_last, q_lo, q_top, nq = geometry(seq_start, seq_end, tile, window)
    rng = [half_range(kb0, kb_last, q_top, nq, window), half_range(kb0 + 64, kb_last, q_top, nq, window)]
    nS = max(rng[0][1], rng[1][1])
    assert 1 <= nS <= nq
    steps = {kq: [] for kq in range(4)}
    loads = {0: [], 1: []}
    for h in heads:
        for j in range(nS):
            for g in (0, 1):
                lo, n = rng[g]
                if j >= n:
                    continue
                q0 = q_top - MQ * (lo + min(j, n - 1))
                loads[g].append((q0, h))
                for kq in (2 * g, 2 * g + 1):
                    if visible(q0, kb0 + 32 * kq, kb_last, window):
                        steps[kq].append((q0, h))
    return steps, loads, (q_lo, q_top, nq, nS)


def plain_steps(seq_start, seq_end, tile, window, heads):
    kb0, kb_last, q_lo, q_top, nq = geometry(seq_start, seq_end, tile, window)
    steps = {kq: [] for kq in range(4)}
    for h in heads:
        for j in range(nq):
            q0 = q_top - MQ * j
            for kq in range(4):
                if visible(q0, kb0 + 32 * kq, kb_last, window):
                    steps[kq].append((q0, h))
    return steps


@pytest.mark.parametrize("window", [0, 3, 20, 40, 50, 63, 64, 65, 128, 300])
def test_window_walk_covers_the_plain_walk(window):
    rng = np.random.default_rng(77 + window)
    heads = [3, 4, 5]
    saved = total = 0
    for _ in range(40):
        seq_start = int(rng.integers(0, 5000))
        seq_end = seq_start + int(rng.integers(1, 900))
        for tile in range((seq_end - seq_start + NKB - 1) // NKB):
            new, loads, (q_lo, q_top, nq, nS) = skewed_steps(seq_start, seq_end, tile, window, heads)
            old = plain_steps(seq_start, seq_end, tile, window, heads)
            for kq in range(4):
                assert len(set(new[kq])) == len(new[kq])                       # each step once
                assert sorted(new[kq]) == sorted(old[kq]), (seq_start, seq_end, tile, kq)
            for g in (0, 1):
                for q0, _ in loads[g]:
                    assert q_lo <= q0 <= q_top and (q0 - q_lo) % MQ == 0
            saved += nq - nS
            total += nq
    assert total > 0 and saved >= 0


def test_full_tiles_of_a_128_key_window_take_six_or_seven_stages():
    for seq_start in range(0, 32):
        _, _, (q_lo, q_top, nq, nS) = skewed_steps(seq_start, seq_start + 4096, 5, 128, [0])
        assert nq in (8, 9) and nS == nq - 2
