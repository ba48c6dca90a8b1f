"""The stored-dS block index that the causal dK/dV kernel's score waves carry from one step to the next (one
update per step, attn_bwd.hip: blk_next) equals the closed form of the block layout at every step of every
key block: ragged sequence starts, several KV heads and head splits.  (With a window the kernel evaluates the
closed form at each step.)

The layout (attn_bwd.hip, "Stored-dS layout"): query tiles of sequence b start at S16 = seq_start & ~15, key
blocks at seq_start; row n holds the key blocks k_lo(n) .. k_hi(n); block (slot, head) sits at
slot * hq + head with slot = ds_index[b] + rows before n + (k - k_lo(n)).  The walk below restates the
kernel's causal step order (query tiles from the last one down, the workgroup's heads inner) and its update
rules; no GPU is used.
"""
import numpy as np
import pytest

NKB, MQ = 128, 32


def row_width(window):
    return (window + 62) // 32 + 1


def rows_before(n, window):
    return n * row_width(window) if window >= 0 else n * (n + 1) // 2


def k_lo(q0, seq_start, window):
    return max(0, q0 - window - seq_start) // 32 if window >= 0 else 0


def split_counts(G):
    """The head-split counts the causal kernel can choose for a group of G query heads (attn_bwd.hip:
    dkv_splits; which one depends on the number of key tiles)."""
    if G % 2 or G < 4:
        return [1]
    return [2, 4] if G % 4 == 0 else [2]


def walk(seq_start, seq_end, tile, kq, window, hq, hkv, kvh, split, ds_seq, splits):
    """Every step of one score wave: assert the carried index equals the closed form; returns the count."""
    G = hq // hkv
    GS = G // splits
    kb0 = seq_start + tile * NKB
    kb_last = min(kb0 + NKB - 1, seq_end - 1)
    q_lo = kb0 & ~15
    q_hi = min(seq_end - 1, kb_last + window) if window >= 0 else seq_end - 1
    nq = (q_hi - q_lo + MQ) // MQ
    nsteps = nq * GS
    s16 = seq_start & ~15
    kap = 4 * tile + kq
    q_top = q_lo + (nq - 1) * MQ
    first = (q_top, kvh * G + split * GS)

    def advance(p):
        q0, h = p[0], p[1] + 1
        if h == first[1] + GS:
            q0, h = q0 - MQ, first[1]
        return (q0, h)

    def closed(p):
        q0, h = p
        n = (q0 - s16) >> 5
        return (ds_seq + rows_before(n, window) + (kap - k_lo(q0, seq_start, window))) * hq + h

    blk_top = closed(first)

    def blk_next(b, p, np_):
        if np_[0] == p[0]:
            return b + 1
        return b - ((p[0] - s16) >> 5) * hq - (GS - 1)

    pc, pn = first, (advance(first) if nsteps > 1 else first)
    bc = bn = blk_top
    if nsteps > 1:
        bn = blk_next(blk_top, first, pn)
    for st in range(nsteps):
        assert bc == closed(pc), (seq_start, seq_end, tile, kq, window, st, pc)
        # the kernel's stage end: block indices first (from the old pn), then the positions
        bc = bn
        if st + 2 <= nsteps - 1:
            bn = blk_next(bn, pn, advance(pn))
        pc = pn
        if st + 2 <= nsteps - 1:
            pn = advance(pn)
    return nsteps


@pytest.mark.parametrize("hq,hkv", [(64, 8), (64, 4), (16, 2), (12, 4)])
def test_carried_block_index_matches_layout(hq, hkv):
    window = -1
    rng = np.random.default_rng(999 + 7 * hq + hkv)
    G = hq // hkv
    steps = 0
    for _ in range(6):
        seq_start = int(rng.integers(0, 5000))
        seq_end = seq_start + int(rng.integers(1, 700))
        ds_seq = int(rng.integers(0, 1 << 20))
        ntiles = (seq_end - seq_start + NKB - 1) // NKB
        for tile in range(ntiles):
            for kq in range(4):
                kvh = int(rng.integers(0, hkv))
                for sp in split_counts(G):
                    split = int(rng.integers(0, sp))
                    steps += walk(seq_start, seq_end, tile, kq, window, hq, hkv, kvh, split, ds_seq, sp)
    assert steps > 0
