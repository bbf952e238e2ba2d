"""CPU oracle for SAS gated block-sparse attention (forward and backward).

TEST INFRASTRUCTURE ONLY.  Only the test-suite, the package's smoke check and
the CPU-baseline leg of the benchmark may import this module.  The product path
(the HIP library and its Python binding) never calls it, and this module imports
nothing from the product path.

Source: "SAS: Simple Attention Sparsification via End-to-End Optimization of
Context Ranking" (arXiv 2609.13141), cited below by section / equation /
algorithm:

  * Sec. 3 (Eq. 2-3): n context tokens are cut into C = n/b contiguous blocks;
    a query attends to the union of its selected blocks.
  * Sec. 4.1 (Eq. 4): the query's own block B0 is always kept with unit gate
    g0 = 1 (zero additive bias); the historical blocks get gates g = phi(s).
  * Sec. 4.2.2 (Eq. 6): with phi = softmax, log g_m = s_m - LSE(s) over the
    historical blocks only.
  * Sec. 4.3 (Eq. 9, Alg. 1): I = Top-K(g, K); S = B0 u U_{m in I} B_m;
    o = softmax(q K_S^T + log g_S) V_S.
  * Sec. 4.3 "Kernel Design" and App. E: Top-K is realised as a per-query
    threshold on the gate (a block is active when it reaches the threshold);
    the current block is causal and unbiased; sm_scale multiplies q.k only.
  * App. E (backward): Delta = rowsum(O * dO), P recomputed from LSE,
    dS = P * (dO V^T - Delta); the block log-gate gradient is the sum of dS over
    the tokens of each selected block.
  * App. D.3: softmax backward to the selector scores,
    ds_m = g_m (dg_m - sum_l g_l dg_l), with dg_l = 0 for unselected blocks
    under the sparse scope (Eq. 8).
  * Sec. 4.2.2 (Eq. 5) / App. D.1: closed form of the inner-gate gradient,
    dg_m = sum_{i in B_m} (p_i / g_m) dO^T (v_i - o).
  * Sec. 4.1 "Components of learnable ranking" and Tab. 1 (the ablated
    variants, kept as switches): gate position outer, o = softmax(q K^T)
    (g . V), with dg_m = sum_{i in B_m} p_i dO^T v_i (Eq. 5 outer); gate
    activation sigmoid (log g = log sigmoid(s)) or raw logits (log g = s),
    beside the default softmax (Eq. 6); the current block keeps g0 = 1 in
    every variant.
  * Sec. 4.1 "Ranking preservation", Eq. 7, Tab. 1 row 8: hard Top-K gates
    with the straight-through estimator, g_hat = stopgrad(g_hard - g) + g:
    the forward attends the selected blocks with unit gates; the gate
    gradient of a dropped block is the attention mass its tokens would get
    under the selected set's normaliser (Eq. 7), so every historical block
    receives dg (see ``ste_gate_grad``).

Readings where the pages leave a step open (each also listed in the design
notes of the repository):
  * gates, threshold and selection are per (batch, kv head, query block,
    context block) and are shared by the G query heads of a KV group and by
    the b queries of a query block; a shared gate's gradient is the sum over
    its uses;
  * K counts historical blocks only; the current block is extra; for query
    block i <= K every historical block is selected; K = 0 selects none;
  * the threshold is applied to the fp32 selector score s itself (log g is a
    monotone shift of s), selection is s >= tau, so ties at tau are all kept;
  * query head h reads kv head floor(h / G);
  * sm_scale defaults to 1/sqrt(D) and never scales log g;
  * variable-length batches (the packed varlen sequences of the pages'
    training kernel, held here in a padded [B, H, N, D] layout): sequence b
    has n_b valid tokens and C_b = ceil(n_b / b) blocks, the last one possibly
    ragged; query rows t >= n_b are padding (no output, no gradient), gate
    rows i >= C_b select nothing; the valid rows of a ragged last block attend
    their block causally, so padding keys are never attended.

Everything is float64 numpy; inputs are upcast from the exact values the GPU
sees.  Two forms are provided: a brute-force dense evaluation per query head
(``dense_*``, tiny sizes) and a per-query-block evaluation (``forward`` /
``backward``), which evaluates the same definition one query block at a time
because the attended set is fixed per query block.

Parity pins: every function here is checked in ``tests/test_oracle.py``
against closed forms, library routines and finite differences (no function is
"parity unpinned").
"""

from __future__ import annotations

import math

import numpy as np

NEG_INF = -np.inf


# ---------------------------------------------------------------------------
# Gate activation and Top-K selection (Eq. 4, Eq. 6, Alg. 1, App. E threshold)
# ---------------------------------------------------------------------------

def _logsumexp(x: np.ndarray) -> float:
    mx = np.max(x)
    return float(mx + np.log(np.sum(np.exp(x - mx))))


def kth_largest_threshold(hist_f32: np.ndarray, k: int) -> np.float32:
    """Threshold tau that realises Top-K over one row of historical scores.

    App. E encodes the Top-K set as "selected iff the gate reaches tau".  With
    tau equal to the K-th largest historical value the selected set is exactly
    the K largest (plus any exact ties at tau).  If K >= number of historical
    blocks every block is kept (tau = -inf); K = 0 keeps none (tau = +inf).
    The comparison is made on the fp32 score values themselves.
    """
    n = hist_f32.shape[0]
    if k >= n:
        return np.float32(-np.inf)
    if k == 0:
        return np.float32(np.inf)
    # np.partition: the element at index n-k is the k-th largest.
    return np.float32(np.partition(hist_f32, n - k)[n - k])


def log_activation(hist64: np.ndarray, act: str) -> np.ndarray:
    """log g of one row's historical scores under gate activation ``act``:
    softmax (Eq. 6: s - LSE(s)), sigmoid (log sigmoid(s), Tab. 1 row 5) or
    raw logits (s itself, Tab. 1 row 6)."""
    if act == "softmax":
        return hist64 - _logsumexp(hist64)
    if act == "sigmoid":
        # log sigmoid(s) = -log(1 + exp(-s)), evaluated without overflow
        return -np.logaddexp(0.0, -hist64)
    if act == "raw":
        return hist64.copy()
    raise ValueError(act)


def n_blocks_of(n: int, block: int) -> int:
    """Blocks of a sequence of n tokens (the last one may be ragged)."""
    return (int(n) + block - 1) // block


def gate_threshold(scores: np.ndarray, budget_k: int, act: str = "softmax", seq_lens=None,
                   block: int | None = None):
    """Gates, thresholds and selected sets for every query block.

    scores: fp32 [B, Hkv, C, C]; only entries m < i of row i are read (the
    historical blocks of query block i, Sec. 4.1).  ``act``: gate activation.

    Returns (log_gate, tau, sel):
      log_gate float64 [B, Hkv, C, C]: log phi(s)_m for m < i (Eq. 6 for the
               softmax), 0 on the diagonal (g0 = 1, Eq. 4), -inf above it;
      tau      float32 [B, Hkv, C]: score-space threshold of each row;
      sel      bool    [B, Hkv, C, C]: m < i and s_{i,m} >= tau_i.
    With ``seq_lens`` (and ``block``) a row i >= C_b of sequence b holds no
    query and selects nothing (tau = +inf); its gates are still written.
    """
    scores = np.asarray(scores)
    assert scores.dtype == np.float32 and scores.ndim == 4
    bsz, hkv, c, c2 = scores.shape
    assert c == c2
    log_gate = np.full((bsz, hkv, c, c), NEG_INF, dtype=np.float64)
    tau = np.empty((bsz, hkv, c), dtype=np.float32)
    sel = np.zeros((bsz, hkv, c, c), dtype=bool)
    for b in range(bsz):
        for h in range(hkv):
            for i in range(c):
                hist = scores[b, h, i, :i]
                if i > 0:
                    log_gate[b, h, i, :i] = log_activation(hist.astype(np.float64), act)
                log_gate[b, h, i, i] = 0.0
                if seq_lens is not None and i >= n_blocks_of(seq_lens[b], block):
                    tau[b, h, i] = np.float32(np.inf)
                    continue
                t = kth_largest_threshold(hist, budget_k)
                tau[b, h, i] = t
                sel[b, h, i, :i] = hist >= t
    return log_gate, tau, sel


# ---------------------------------------------------------------------------
# Attended set of one query block (Eq. 9 with the App. E current-block rule)
# ---------------------------------------------------------------------------

def _attended_keys(i: int, block: int, sel_row: np.ndarray, log_gate_row: np.ndarray):
    """Key token indices, per-key additive bias and per-key block id for block i.

    Keys are the current block (bias 0, causal inside it) followed by every
    selected historical block m (bias log g_m).  The order of keys does not
    change the softmax.
    """
    own = np.arange(i * block, (i + 1) * block)
    blocks = [i] + [int(m) for m in np.nonzero(sel_row)[0]]
    keys = np.concatenate([np.arange(m * block, (m + 1) * block) for m in blocks])
    bias = np.concatenate([np.zeros(block)] +
                          [np.full(block, log_gate_row[m]) for m in blocks[1:]])
    kblk = np.repeat(np.array(blocks), block)
    # causal mask inside the current block: key position must not exceed query
    qpos = own[:, None]
    mask = np.ones((block, keys.shape[0]), dtype=bool)
    mask[:, :block] = keys[None, :block] <= qpos
    return keys, bias, kblk, mask


def _f64(x) -> np.ndarray:
    """Exact upcast of a slice (inputs are bf16/fp32 values held in any float array)."""
    return np.asarray(x, dtype=np.float64)


def _softmax_rows(z: np.ndarray):
    mx = np.max(z, axis=1, keepdims=True)
    e = np.exp(z - mx)
    s = np.sum(e, axis=1, keepdims=True)
    return e / s, (mx + np.log(s))[:, 0]


def default_scale(head_dim: int, sm_scale: float | None) -> float:
    if sm_scale is None or sm_scale <= 0:
        return 1.0 / math.sqrt(head_dim)
    return float(sm_scale)


def _valid_rows(b: int, i: int, block: int, seq_lens) -> int:
    """Valid query rows of block i of sequence b (0 .. block)."""
    if seq_lens is None:
        return block
    return int(min(block, max(0, int(seq_lens[b]) - i * block)))


def forward(q, k, v, log_gate, sel, block: int, sm_scale: float | None = None,
            query_blocks=None, gate_pos: str = "inner", seq_lens=None):
    """Eq. 9 output and natural-log LSE, one query block at a time.

    q: [B, Hq, N, D]; k, v: [B, Hkv, N, D]; log_gate/sel: [B, Hs, C, C] with
    Hs score heads: Hs = Hkv (one gate / selection per query group, the
    default) or Hs = Hq (per query head); score head s covers query heads
    s Gs .. s Gs + Gs - 1 (Gs = Hq / Hs), which read kv head s Gs / G.
    ``query_blocks``: optional iterable of (b, s, i) to evaluate (others
    are left 0), so large shapes can be sampled.
    ``gate_pos``: "inner" adds log g to the logits (Eq. 9); "outer" leaves the
    logits ungated and multiplies the value rows of each block by its gate,
    o = softmax(q K^T) (g . V) (Sec. 4.1, Tab. 1 row 3); lse is then the
    ungated one.
    ``seq_lens``: valid tokens per sequence (padding rows get o = 0, lse = 0).
    Returns (o [B, Hq, N, D], lse [B, Hq, N]) in float64.
    """
    bsz, hq, n, d = q.shape
    g = hq // k.shape[1]
    hs = log_gate.shape[1]
    gs = hq // hs
    scale = default_scale(d, sm_scale)
    c = n // block
    o = np.zeros(q.shape)          # calloc: untouched pages cost nothing
    lse = np.zeros((bsz, hq, n))
    units = query_blocks if query_blocks is not None else \
        [(b, h, i) for b in range(bsz) for h in range(hs) for i in range(c)]
    for (b, sh, i) in units:
        nv = _valid_rows(b, i, block, seq_lens)
        if nv == 0:
            continue
        keys, bias, _, mask = _attended_keys(i, block, sel[b, sh, i], log_gate[b, sh, i])
        mask = mask[:nv]
        kvh = (sh * gs) // g
        kk = _f64(k[b, kvh, keys])
        vv = _f64(v[b, kvh, keys])
        if seq_lens is not None:   # padding keys are never attended; keep them out of the sums
            pad = keys >= int(seq_lens[b])
            kk[pad] = 0.0
            vv[pad] = 0.0
        if gate_pos == "outer":
            vv = vv * np.exp(bias)[:, None]
            bias = np.zeros_like(bias)
        rows = slice(i * block, i * block + nv)
        for hh in range(sh * gs, (sh + 1) * gs):
            z = scale * (_f64(q[b, hh, rows]) @ kk.T) + bias[None, :]
            z = np.where(mask, z, NEG_INF)
            p, l = _softmax_rows(z)
            o[b, hh, rows] = p @ vv
            lse[b, hh, rows] = l
    return o, lse


def backward(q, k, v, do, log_gate, sel, block: int, sm_scale: float | None = None,
             query_blocks=None, gate_pos: str = "inner", seq_lens=None, term_mass: bool = False):
    """Gradients of Eq. 9 w.r.t. q, k, v and the block log gates.

    Follows the recomputation view of App. E: P from the attended logits,
    dP = dO V^T, Delta = rowsum(P * dP) (= dO . o), dS = P * (dP - Delta);
    dQ = sm_scale dS K, dK = sm_scale dS^T Q, dV = P^T dO, summed over the G
    query heads that read the same kv head; dLogG[i, m] = sum of dS over the
    query tokens of block i (all query heads of the score head) and the key
    tokens of selected historical block m.  Zero for unselected m, the
    diagonal and the upper triangle.  Score heads as in ``forward``.

    ``gate_pos`` = "outer": the value rows are scaled by their block's gate,
    so dP = dO (g . V)^T, dV = g . (P^T dO), and dLogG[i, m] = g_m dg_m =
    sum over the block of P * dP (Eq. 5 outer: dg_m = sum_i p_i dO^T v_i).

    If ``query_blocks`` is given, only those query blocks contribute (their dQ
    and dLogG rows are exact; dK/dV hold only their contributions).
    ``seq_lens``: padding query rows contribute nothing and get dQ = 0.
    Returns (dq, dk, dv, dlog_gate) in float64.

    ``term_mass``: also return the sums of the absolute values of the terms
    that dK and dV add up (sm_scale |dS|^T |Q| and |g| P^T |dO|), the scale
    of the rounding error of a sum whose terms are rounded (the tests bound
    the error of the bf16 products with it); (dq, dk, dv, dlog_gate,
    dk_mass, dv_mass).
    """
    bsz, hq, n, d = q.shape
    g = hq // k.shape[1]
    hs = log_gate.shape[1]
    gs = hq // hs
    scale = default_scale(d, sm_scale)
    c = n // block
    dq = np.zeros(q.shape)
    dk = np.zeros(k.shape)
    dv = np.zeros(v.shape)
    dlg = np.zeros((bsz, hs, c, c))
    dk_mass = np.zeros(k.shape) if term_mass else None
    dv_mass = np.zeros(v.shape) if term_mass else None
    units = query_blocks if query_blocks is not None else \
        [(b, h, i) for b in range(bsz) for h in range(hs) for i in range(c)]
    for (b, sh, i) in units:
        nv = _valid_rows(b, i, block, seq_lens)
        if nv == 0:
            continue
        keys, bias, kblk, mask = _attended_keys(i, block, sel[b, sh, i], log_gate[b, sh, i])
        mask = mask[:nv]
        hk = (sh * gs) // g
        kk = _f64(k[b, hk, keys])
        vv = _f64(v[b, hk, keys])
        if seq_lens is not None:
            pad = keys >= int(seq_lens[b])
            kk[pad] = 0.0
            vv[pad] = 0.0
        gkey = np.ones(keys.shape[0])
        if gate_pos == "outer":
            gkey = np.exp(bias)
            vv = vv * gkey[:, None]
            bias = np.zeros_like(bias)
        rows = slice(i * block, i * block + nv)
        ds_sum = np.zeros(keys.shape[0])
        for hh in range(sh * gs, (sh + 1) * gs):
            qq = _f64(q[b, hh, rows])
            dd = _f64(do[b, hh, rows])
            z = scale * (qq @ kk.T) + bias[None, :]
            z = np.where(mask, z, NEG_INF)
            p, _ = _softmax_rows(z)
            dp = dd @ vv.T
            delta = np.sum(p * dp, axis=1, keepdims=True)
            ds = p * (dp - delta)
            dq[b, hh, rows] = scale * (ds @ kk)
            # the attended keys of a query block are distinct, so the indexed
            # add accumulates each key row once
            dk[b, hk, keys] += scale * (ds.T @ qq)
            dv[b, hk, keys] += gkey[:, None] * (p.T @ dd)
            if term_mass:
                dk_mass[b, hk, keys] += scale * (np.abs(ds).T @ np.abs(qq))
                dv_mass[b, hk, keys] += np.abs(gkey)[:, None] * (p.T @ np.abs(dd))
            ds_sum += (p * dp).sum(axis=0) if gate_pos == "outer" else ds.sum(axis=0)
        for m in np.unique(kblk):
            if m != i:
                dlg[b, sh, i, m] = ds_sum[kblk == m].sum()
    if term_mass:
        return dq, dk, dv, dlg, dk_mass, dv_mass
    return dq, dk, dv, dlg


def backward_kv_block(q, k, v, do, log_gate, sel, block: int, b: int, hk: int, j: int,
                      sm_scale: float | None = None, gate_pos: str = "inner", seq_lens=None,
                      term_mass: bool = False):
    """dK and dV of one key block j of one (batch, kv head), exactly.

    Sums the contributions of every query block that attends block j: the
    diagonal block i = j and every i > j with j in I_i (Eq. 9 gradient).
    ``seq_lens`` as in ``backward`` (padding rows contribute nothing).
    Returns (dk_j [block, D], dv_j [block, D]), and with ``term_mass`` also
    the block's term masses as in ``backward``.
    """
    c = q.shape[2] // block
    g = q.shape[1] // k.shape[1]
    gs = q.shape[1] // sel.shape[1]
    heads = range(hk * g // gs, (hk + 1) * g // gs)   # score heads of kv head hk
    users = [(b, sh, i) for sh in heads for i in range(j, c) if i == j or sel[b, sh, i, j]]
    out = backward(q, k, v, do, log_gate, sel, block, sm_scale, query_blocks=users,
                   gate_pos=gate_pos, seq_lens=seq_lens, term_mass=term_mass)
    rows = slice(j * block, (j + 1) * block)
    if term_mass:
        return out[1][b, hk, rows], out[2][b, hk, rows], out[4][b, hk, rows], out[5][b, hk, rows]
    return out[1][b, hk, rows], out[2][b, hk, rows]


def ste_gate_grad(q, k, v, do, log_gate, sel, block: int, sm_scale: float | None = None,
                  seq_lens=None, rows=None):
    """Gate gradients of the hard Top-K gates with the straight-through estimator
    (Sec. 4.1 "Ranking preservation", Eq. 7, Tab. 1 row 8).

    Forward: g_hat = 1 on selected blocks and 0 on dropped ones, so the output
    is the selected-set attention with zero bias.  With p_i = g_hat_b(i) e^z_i /
    sum_j g_hat_b(j) e^z_j, dL/dg_hat_m = sum_{i in B_m} (dp_i/dg_hat_m ...) =
    sum_{t, u in B_m} e^{z_tu - lse_t} (dO_t . v_u - Delta_t), where lse_t is
    the selected set's log normaliser (Eq. 7: the weight a dropped block's
    token would get under it); for a selected block this is the block's dS sum.
    The STE passes dL/dg = dL/dg_hat.
    Returns dg float64 [B, Hs, C, C] (score heads as in ``forward``) for every
    historical block m < i (0 for m >= i).  ``rows``: optional iterable of
    gate rows (b, s, i) to evaluate (the others stay 0), so that large shapes
    can be sampled.
    """
    bsz, hq, n, d = q.shape
    g = hq // k.shape[1]
    hs = log_gate.shape[1]
    gs = hq // hs
    scale = default_scale(d, sm_scale)
    c = n // block
    zero = np.where(np.isfinite(log_gate), 0.0, log_gate)
    if rows is None:
        rows = [(b, sh, i) for b in range(bsz) for sh in range(hs) for i in range(1, c)]
    rows = sorted(set((int(b), int(sh), int(i)) for (b, sh, i) in rows))
    o, lse = forward(q, k, v, zero, sel, block, sm_scale, query_blocks=rows, seq_lens=seq_lens)
    dg = np.zeros((bsz, hs, c, c))
    for (b, sh, i) in rows:
        hk = (sh * gs) // g
        nv = _valid_rows(b, i, block, seq_lens)
        if i < 1 or nv == 0:
            continue
        qrows = slice(i * block, i * block + nv)
        for m in range(i):
            cols = slice(m * block, (m + 1) * block)
            kk = _f64(k[b, hk, cols])
            vv = _f64(v[b, hk, cols])
            tot = 0.0
            for hh in range(sh * gs, (sh + 1) * gs):
                dd = _f64(do[b, hh, qrows])
                z = scale * (_f64(q[b, hh, qrows]) @ kk.T)
                pw = np.exp(z - lse[b, hh, qrows][:, None])
                delta = np.sum(dd * o[b, hh, qrows], axis=1, keepdims=True)
                tot += float(np.sum(pw * (dd @ vv.T - delta)))
            dg[b, sh, i, m] = tot
    return dg


def dscores_from_dg(dg, log_gate):
    """Softmax backward (App. D.3) from gate gradients given for every
    historical block (full scope): ds_m = g_m (dg_m - sum_l g_l dg_l)."""
    bsz, hkv, c, _ = dg.shape
    out = np.zeros((bsz, hkv, c, c))
    for b in range(bsz):
        for h in range(hkv):
            for i in range(1, c):
                gate = np.exp(log_gate[b, h, i, :i])
                out[b, h, i, :i] = gate * (dg[b, h, i, :i] - np.sum(gate * dg[b, h, i, :i]))
    return out


def dscores(dlog_gate, log_gate, sel, act: str = "softmax"):
    """Selector-score gradient from the block log-gate gradient (App. D.3).

    dg_m = dLogG_m / g_m on selected blocks and 0 on unselected ones (sparse
    scope, Eq. 8); for the softmax gate ds_m = g_m (dg_m - sum_l g_l dg_l)
    over the historical blocks m < i.  For the sigmoid gate each block's
    gate depends on its own score only: ds_m = g_m (1 - g_m) dg_m; for raw
    logits log g = s, so ds_m = dLogG_m.  Zero for m >= i.  No gradient flows
    through the Top-K selection itself (it is piecewise constant in s, Sec. 3).
    """
    bsz, hkv, c, _ = dlog_gate.shape
    out = np.zeros((bsz, hkv, c, c))
    for b in range(bsz):
        for h in range(hkv):
            for i in range(1, c):
                gate = np.exp(log_gate[b, h, i, :i])
                s = sel[b, h, i, :i]
                dg = np.zeros(i)
                dg[s] = dlog_gate[b, h, i, :i][s] / gate[s]
                if act == "softmax":
                    out[b, h, i, :i] = gate * (dg - np.sum(gate * dg))
                elif act == "sigmoid":
                    out[b, h, i, :i] = gate * (1.0 - gate) * dg
                elif act == "raw":
                    out[b, h, i, :i] = gate * dg
                else:
                    raise ValueError(act)
    return out


# ---------------------------------------------------------------------------
# Brute-force dense form (tiny sizes): the full N x N logit matrix per head
# ---------------------------------------------------------------------------

def dense_bias(log_gate, sel, n: int, block: int, b: int, hk: int) -> np.ndarray:
    """Additive N x N bias of Eq. 9 for one (batch, kv head).

    bias[t, u] = 0 if u is in t's own block and u <= t (causal, unit gate);
    log g_{blk t, blk u} if blk u is a selected historical block of blk t;
    -inf otherwise.
    """
    bias = np.full((n, n), NEG_INF)
    for t in range(n):
        bt = t // block
        for u in range(n):
            bu = u // block
            if bu == bt and u <= t:
                bias[t, u] = 0.0
            elif bu < bt and sel[b, hk, bt, bu]:
                bias[t, u] = log_gate[b, hk, bt, bu]
    return bias


def dense_forward(q, k, v, log_gate, sel, block: int, sm_scale: float | None = None):
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    bsz, hq, n, d = q.shape
    g = hq // k.shape[1]
    scale = default_scale(d, sm_scale)
    o = np.zeros_like(q)
    lse = np.zeros((bsz, hq, n))
    for b in range(bsz):
        for hh in range(hq):
            hk = hh // g
            z = scale * (q[b, hh] @ k[b, hk].T) + dense_bias(log_gate, sel, n, block, b, hk)
            p, l = _softmax_rows(z)
            o[b, hh] = p @ v[b, hk]
            lse[b, hh] = l
    return o, lse


def dense_backward(q, k, v, do, log_gate, sel, block: int, sm_scale: float | None = None):
    """Softmax-Jacobian gradients on the full matrix (App. E backward, dense)."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    do = np.asarray(do, np.float64)
    bsz, hq, n, d = q.shape
    hkv = k.shape[1]
    g = hq // hkv
    c = n // block
    scale = default_scale(d, sm_scale)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    dlg = np.zeros((bsz, hkv, c, c))
    for b in range(bsz):
        for hh in range(hq):
            hk = hh // g
            z = scale * (q[b, hh] @ k[b, hk].T) + dense_bias(log_gate, sel, n, block, b, hk)
            p, _ = _softmax_rows(z)
            dp = do[b, hh] @ v[b, hk].T
            ds = p * (dp - np.sum(p * dp, axis=1, keepdims=True))
            dq[b, hh] = scale * ds @ k[b, hk]
            dk[b, hk] += scale * ds.T @ q[b, hh]
            dv[b, hk] += p.T @ do[b, hh]
            blk_sum = ds.reshape(c, block, c, block).sum(axis=(1, 3))
            for i in range(c):
                for m in range(i):
                    if sel[b, hk, i, m]:
                        dlg[b, hk, i, m] += blk_sum[i, m]
    return dq, dk, dv, dlg
