"""CPU oracle for SAS sparse decode (one new query token per sequence).

TEST INFRASTRUCTURE ONLY.  Only the test-suite and the benchmark's CPU-baseline
leg may import this module.  The product path (the HIP library and its Python
binding) never calls it, and this module imports nothing from the product path.

Source: "SAS: Simple Attention Sparsification via End-to-End Optimization of
Context Ranking" (arXiv 2609.13141):

  * Sec. 4.3, Alg. 2 (SAS inference step): the selector scores the cached
    blocks, I = Top-K(s, K), S = B0 u U_{m in I} B_m and
    o = softmax(q K_S^T) V_S -- no gates at inference.
  * Sec. 5.1, "Inference implementation": prefill is dense, decode is block
    sparse; at each step the Top-K blocks are chosen per query group (grouped
    query attention with per-group selection), only those KV blocks are
    gathered from the paged KV cache, and decoding is batched.
  * Sec. 6.3 / Fig. 7: the decode step is selector scoring, Top-K selection
    and the attention over the selected blocks.

Readings where the pages leave a step open (also listed in the design notes):
  * the newest token's K/V are in the cache; a sequence holding n tokens has
    its query at position n - 1, whose block c = (n - 1) // b is the current
    block B0 (kept, whether full or partial); the historical blocks are the
    complete blocks m < c, and K counts historical blocks only (as in
    training); K >= c keeps every historical block, K = 0 keeps none;
  * the selection is per (sequence, kv head) and shared by the G query heads
    of the group; Top-K is the threshold tau = K-th largest fp32 score, with
    every score >= tau kept (ties at tau all kept), as in the training path;
  * sm_scale = 1/sqrt(D) multiplies q.k (the training convention; Alg. 2
    writes the product without the factor, as Eq. 1 does);
  * the paged cache holds pages of one block (b tokens, all kv heads):
    pool [P, Hkv, b, D]; block_table[s, m] is the page of logical block m of
    sequence s.  The selector scores are an input [B, Hkv, Cmax] (the selector
    network needs trained weights and is not part of the path).

Everything is float64 numpy; inputs are upcast from the exact values the GPU
sees.  Pins: tests/test_decode_oracle.py (torch.topk for the selection; torch
scaled-dot-product attention over a contiguous cache for the attention, with
the paged pool built from it by an independent scatter; closed forms).
"""

from __future__ import annotations

import math

import numpy as np


def current_block(n: int, block: int) -> int:
    """Index of the block holding the query token (position n - 1)."""
    return (int(n) - 1) // block


def decode_select(scores: np.ndarray, seq_lens, block: int, budget_k: int):
    """Top-K as a threshold over the historical blocks of each (sequence, kv head).

    scores: fp32 [B, Hkv, Cmax]; only entries m < c_b are read.
    Returns (tau float32 [B, Hkv], sel bool [B, Hkv, Cmax]).
    """
    scores = np.asarray(scores)
    assert scores.dtype == np.float32 and scores.ndim == 3
    bsz, hkv, cmax = scores.shape
    tau = np.empty((bsz, hkv), dtype=np.float32)
    sel = np.zeros((bsz, hkv, cmax), dtype=bool)
    for b in range(bsz):
        c = current_block(seq_lens[b], block)
        for h in range(hkv):
            hist = scores[b, h, :c]
            if budget_k >= c:
                t = np.float32(-np.inf)
            elif budget_k == 0:
                t = np.float32(np.inf)
            else:
                # the K-th largest historical score
                t = np.float32(np.sort(hist)[c - budget_k])
            tau[b, h] = t
            sel[b, h, :c] = hist >= t
    return tau, sel


def attended_positions(n: int, block: int, sel_row: np.ndarray) -> np.ndarray:
    """Logical token positions the query of a sequence of n tokens attends:
    the tokens of its current block up to n - 1 and every token of each
    selected historical block (ascending)."""
    c = current_block(n, block)
    blocks = [int(m) for m in np.nonzero(sel_row)[0] if m < c]
    pos = [np.arange(m * block, (m + 1) * block) for m in blocks]
    pos.append(np.arange(c * block, n))
    return np.concatenate(pos)


def decode_attn(q, k_pool, v_pool, block_table, seq_lens, sel, block: int,
                sm_scale: float | None = None):
    """o = softmax(sm_scale q K_S^T) V_S for every (sequence, query head).

    q: [B, Hq, D]; k_pool, v_pool: [P, Hkv, block, D]; block_table: int [B, Cmax];
    seq_lens: [B]; sel: bool [B, Hkv, Cmax].
    Returns (o float64 [B, Hq, D], lse float64 [B, Hq], natural log).
    """
    q = np.asarray(q, dtype=np.float64)
    kp = np.asarray(k_pool, dtype=np.float64)
    vp = np.asarray(v_pool, dtype=np.float64)
    bt = np.asarray(block_table)
    bsz, hq, d = q.shape
    hkv = kp.shape[1]
    g = hq // hkv
    scale = 1.0 / math.sqrt(d) if sm_scale is None or sm_scale <= 0 else float(sm_scale)
    o = np.zeros((bsz, hq, d))
    lse = np.zeros((bsz, hq))
    for b in range(bsz):
        n = int(seq_lens[b])
        for hk in range(hkv):
            pos = attended_positions(n, block, sel[b, hk])
            pages = bt[b, pos // block]
            rows = pos % block
            keys = kp[pages, hk, rows]      # [L, D]
            vals = vp[pages, hk, rows]
            for hh in range(hk * g, (hk + 1) * g):
                z = scale * (keys @ q[b, hh])
                mx = np.max(z)
                e = np.exp(z - mx)
                s = np.sum(e)
                o[b, hh] = (e / s) @ vals
                lse[b, hh] = mx + np.log(s)
    return o, lse
