"""The benchmark's work count (CPU): the attended (query, key) pairs that the
effective TFLOP/s figure divides by, checked against a brute-force count of
the pairs the method attends (the causal part of a query's own block plus
every key of its selected historical blocks, Eq. 9 / Alg. 1 of the SAS
paper), for fixed-length and variable-length batches."""
import numpy as np
import torch

import bench
import oracle


def brute_pairs(sel, block, gs, lens=None):
    """Loop over every (batch, query head, query row, key) and test the
    definition directly.  sel: [B, Hs, C, C] bool (row i selects block m)."""
    B, Hs, C, _ = sel.shape
    n = C * block
    total = 0
    for b in range(B):
        nb = n if lens is None else max(0, min(n, int(lens[b])))
        for s in range(Hs):
            for _h in range(gs):   # the query heads of score head s
                for r in range(nb):
                    i = r // block
                    for key in range(nb):
                        m = key // block
                        if (m == i and key <= r) or (m < i and sel[b, s, i, m]):
                            total += 1
    return total


def _selection(B, Hs, C, K, seed, lens=None, block=None):
    g = torch.Generator().manual_seed(seed)
    scores = torch.randn(B, Hs, C, C, generator=g).numpy()   # float32, as the kernels take
    _, _, sel = oracle.gate_threshold(scores, K, seq_lens=lens, block=block)
    return sel


def test_count_pairs_matches_brute_force():
    B, Hs, C, block, K, gs = 2, 3, 6, 4, 2, 2
    sel = _selection(B, Hs, C, K, seed=3)
    cnt = torch.from_numpy(sel.sum(-1).astype(np.int32))
    got = bench.count_pairs(cnt, cap=C, block=block, group=gs)
    assert got == brute_pairs(sel, block, gs)


def test_count_pairs_respects_the_capacity():
    B, Hs, C, block, K, gs = 1, 2, 8, 4, 5, 3
    sel = _selection(B, Hs, C, K, seed=4)
    cap = 2   # rows with more selected blocks keep their first cap (ascending)
    kept = np.zeros_like(sel)
    for b in range(B):
        for s in range(Hs):
            for i in range(C):
                idx = np.nonzero(sel[b, s, i])[0][:cap]
                kept[b, s, i, idx] = True
    cnt = torch.from_numpy(sel.sum(-1).astype(np.int32))
    assert bench.count_pairs(cnt, cap=cap, block=block, group=gs) == brute_pairs(kept, block, gs)


def test_unit_pairs_matches_brute_force_with_ragged_lengths():
    B, Hs, C, block, K, gs = 3, 2, 6, 4, 2, 2
    lens = np.array([24, 9, 1])   # full, a ragged block, a single token
    sel = _selection(B, Hs, C, K, seed=5, lens=lens, block=block)
    cnt = sel.sum(-1)
    units = [(b, s, i) for b in range(B) for s in range(Hs) for i in range(C)]
    got = bench.unit_pairs(units, cnt, block, gs, lens)
    assert got == brute_pairs(sel, block, gs, lens)
