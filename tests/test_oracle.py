"""Pins of the CPU oracle against what the SAS pages and mathematics fix.

Each test checks the oracle against something other than itself: a library
routine (torch SDPA, torch.topk, torch autograd), a closed form printed on the
pages (Eq. 5, Eq. 6, Eq. 8, App. D.3), central finite differences, an
invariant the pages state, or a hand-worked example.  The planted-mistake tests
at the end show that plausible slips in the oracle fail these pins.
"""

import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import sas_oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------------------
# helpers
# ---------------------------------------------------------------------------

def rand_problem(seed, B=1, Hq=2, Hkv=1, N=32, D=8, block=4, K=2, std=1.0, score_std=1.5):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, Hq, N, D)) * std
    k = rng.standard_normal((B, Hkv, N, D)) * std
    v = rng.standard_normal((B, Hkv, N, D))
    do = rng.standard_normal((B, Hq, N, D))
    c = N // block
    scores = (rng.standard_normal((B, Hkv, c, c)) * score_std).astype(np.float32)
    lg, tau, sel = oracle.gate_threshold(scores, K)
    return dict(q=q, k=k, v=v, do=do, scores=scores, lg=lg, tau=tau, sel=sel, block=block, K=K)


def sdpa64(q, k, v, mask=None, causal=False, scale=None):
    """torch scaled_dot_product_attention on the CPU in float64 (GQA by repeat)."""
    qt = torch.from_numpy(q)
    g = q.shape[1] // k.shape[1]
    kt = torch.from_numpy(k).repeat_interleave(g, dim=1)
    vt = torch.from_numpy(v).repeat_interleave(g, dim=1)
    m = None if mask is None else torch.from_numpy(mask)
    out = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=m,
                                                           is_causal=causal, scale=scale)
    return out.numpy()


def torch_dense_model(p, logg_leaf=True, scores_leaf=False):
    """Eq. 9 written with torch ops for autograd (selection held fixed)."""
    B, Hq, N, D = p["q"].shape
    Hkv = p["k"].shape[1]
    G = Hq // Hkv
    blk = p["block"]
    C = N // blk
    scale = 1.0 / math.sqrt(D)
    q = torch.tensor(p["q"], requires_grad=True)
    k = torch.tensor(p["k"], requires_grad=True)
    v = torch.tensor(p["v"], requires_grad=True)
    sel = torch.from_numpy(p["sel"])
    if scores_leaf:
        s = torch.tensor(p["scores"].astype(np.float64), requires_grad=True)
        tri = torch.tril(torch.ones(C, C, dtype=torch.bool), diagonal=-1)
        s_m = torch.where(tri, s, torch.tensor(-1e30, dtype=torch.float64))
        lse = torch.logsumexp(s_m, dim=-1, keepdim=True)
        lg = torch.where(tri, s - lse, torch.zeros_like(s))
        leaf = s
    else:
        lg = torch.tensor(np.where(np.isfinite(p["lg"]), p["lg"], 0.0), requires_grad=logg_leaf)
        leaf = lg
    tok = torch.arange(N)
    tb = tok // blk
    same = tb[:, None] == tb[None, :]
    causal = tok[None, :] <= tok[:, None]
    outs = []
    for b in range(B):
        for h in range(Hq):
            hk = h // G
            bias_blk = lg[b, hk][tb][:, tb]            # log g of (query block, key block)
            selm = sel[b, hk][tb][:, tb]
            bias = torch.where(same & causal, torch.zeros_like(bias_blk),
                               torch.where(selm, bias_blk,
                                           torch.full_like(bias_blk, -math.inf)))
            z = scale * q[b, h] @ k[b, hk].T + bias
            pr = torch.softmax(z, dim=-1)
            outs.append(pr @ v[b, hk])
    o = torch.stack(outs).reshape(B, Hq, N, D)
    loss = (o * torch.from_numpy(p["do"])).sum()
    loss.backward()
    return o.detach().numpy(), q.grad.numpy(), k.grad.numpy(), v.grad.numpy(), leaf.grad.numpy()


def loss_of(p, q=None, k=None, v=None, lg=None):
    o, _ = oracle.forward(p["q"] if q is None else q, p["k"] if k is None else k,
                          p["v"] if v is None else v, p["lg"] if lg is None else lg,
                          p["sel"], p["block"])
    return float(np.sum(o * p["do"]))


# ---------------------------------------------------------------------------
# P2: gates (Eq. 4, Eq. 6)
# ---------------------------------------------------------------------------

def test_gates_sum_to_one_over_historical_blocks():
    p = rand_problem(0, N=64, block=4)
    lg = p["lg"]
    C = lg.shape[-1]
    for i in range(1, C):
        assert abs(np.exp(lg[0, 0, i, :i]).sum() - 1.0) < 1e-12
        assert lg[0, 0, i, i] == 0.0                      # g0 = 1 (current block)
        assert np.all(np.isneginf(lg[0, 0, i, i + 1:]))
    assert lg[0, 0, 1, 0] == 0.0                          # one historical block -> g = 1


def test_gates_shift_invariant():
    rng = np.random.default_rng(3)
    # multiples of 2^-8 in [-4, 4): adding 16 is exact in fp32
    s = (np.round(rng.uniform(-4, 4, (1, 2, 12, 12)) * 256) / 256).astype(np.float32)
    lg1, tau1, sel1 = oracle.gate_threshold(s, 3)
    lg2, tau2, sel2 = oracle.gate_threshold(s + np.float32(16.0), 3)
    fin = np.isfinite(lg1)
    np.testing.assert_allclose(lg1[fin], lg2[fin], atol=1e-12)
    assert np.array_equal(sel1, sel2)


def test_uniform_scores_give_minus_log_i():
    s = np.zeros((1, 1, 10, 10), np.float32)
    lg, _, _ = oracle.gate_threshold(s, 20)
    for i in range(1, 10):
        np.testing.assert_allclose(lg[0, 0, i, :i], -math.log(i), atol=1e-14)


# ---------------------------------------------------------------------------
# P3: Top-K selection as a threshold (Eq. 3, App. E)
# ---------------------------------------------------------------------------

def test_selection_matches_torch_topk():
    rng = np.random.default_rng(5)
    s = rng.standard_normal((2, 3, 40, 40)).astype(np.float32)
    for K in (0, 1, 3, 7, 39, 50):
        _, _, sel = oracle.gate_threshold(s, K)
        for b in range(2):
            for h in range(3):
                for i in range(40):
                    got = set(np.nonzero(sel[b, h, i])[0].tolist())
                    kk = min(K, i)
                    if kk == 0:
                        want = set()
                    else:
                        want = set(torch.topk(torch.from_numpy(s[b, h, i, :i]), kk).indices.tolist())
                    assert got == want, (K, b, h, i)
                    assert len(got) == min(K, i)
                    assert all(m < i for m in got)


def test_selection_monotone_in_budget():
    rng = np.random.default_rng(6)
    s = rng.standard_normal((1, 2, 30, 30)).astype(np.float32)
    prev = None
    for K in (0, 2, 4, 8, 16, 32):
        _, _, sel = oracle.gate_threshold(s, K)
        if prev is not None:
            assert np.all(sel[prev]), "a block selected at a smaller K was dropped"
        prev = sel


def test_selection_ties_are_all_kept():
    s = np.zeros((1, 1, 5, 5), np.float32)
    s[0, 0, 4, :4] = [1.0, 2.0, 2.0, 3.0]
    _, tau, sel = oracle.gate_threshold(s, 2)
    assert tau[0, 0, 4] == np.float32(2.0)
    assert np.nonzero(sel[0, 0, 4])[0].tolist() == [1, 2, 3]    # >= tau keeps both ties
    _, tau, sel = oracle.gate_threshold(s, 1)
    assert np.nonzero(sel[0, 0, 4])[0].tolist() == [3]
    _, tau, sel = oracle.gate_threshold(s, 0)
    assert not sel.any() and tau[0, 0, 4] == np.inf


# ---------------------------------------------------------------------------
# P1 / P4: forward (Eq. 9) against library attention
# ---------------------------------------------------------------------------

def test_zero_gates_all_selected_is_dense_causal_attention():
    p = rand_problem(1, B=2, Hq=4, Hkv=2, N=48, D=16, block=8)
    C = 48 // 8
    lg = np.zeros((2, 2, C, C))
    sel = np.tril(np.ones((C, C), bool), -1)[None, None].repeat(2, 0).repeat(2, 1)
    o, lse = oracle.forward(p["q"], p["k"], p["v"], lg, sel, 8)
    ref = sdpa64(p["q"], p["k"], p["v"], causal=True)
    np.testing.assert_allclose(o, ref, atol=1e-12, rtol=1e-12)


def test_budget_zero_is_block_local_causal_attention():
    p = rand_problem(2, B=1, Hq=2, Hkv=2, N=40, D=8, block=8, K=0)
    o, _ = oracle.forward(p["q"], p["k"], p["v"], p["lg"], p["sel"], 8)
    tok = np.arange(40)
    mask = (tok[None, :] <= tok[:, None]) & (tok[None, :] // 8 == tok[:, None] // 8)
    ref = sdpa64(p["q"], p["k"], p["v"], mask=mask)
    np.testing.assert_allclose(o, ref, atol=1e-12)


def test_forward_matches_sdpa_with_gate_bias_mask():
    p = rand_problem(4, B=1, Hq=3, Hkv=1, N=36, D=8, block=6, K=2)
    o, lse = oracle.forward(p["q"], p["k"], p["v"], p["lg"], p["sel"], 6)
    tok = np.arange(36)
    tb = tok // 6
    lg = p["lg"][0, 0][tb][:, tb]
    sl = p["sel"][0, 0][tb][:, tb]
    mask = np.where((tb[None, :] == tb[:, None]) & (tok[None, :] <= tok[:, None]), 0.0,
                    np.where(sl, lg, -np.inf))
    ref = sdpa64(p["q"], p["k"], p["v"], mask=mask[None, None])
    np.testing.assert_allclose(o, ref, atol=1e-12)
    # LSE agrees with the same bias through torch.logsumexp
    z = p["q"][0] @ p["k"][0, 0].T / math.sqrt(8) + mask[None]
    np.testing.assert_allclose(lse[0], torch.logsumexp(torch.from_numpy(z), -1).numpy(), atol=1e-12)


def test_dense_and_blockwise_forms_agree():
    p = rand_problem(7, B=2, Hq=4, Hkv=2, N=32, D=8, block=4, K=3)
    o1, l1 = oracle.dense_forward(p["q"], p["k"], p["v"], p["lg"], p["sel"], 4)
    o2, l2 = oracle.forward(p["q"], p["k"], p["v"], p["lg"], p["sel"], 4)
    np.testing.assert_allclose(o1, o2, atol=1e-12)
    np.testing.assert_allclose(l1, l2, atol=1e-12)
    g1 = oracle.dense_backward(p["q"], p["k"], p["v"], p["do"], p["lg"], p["sel"], 4)
    g2 = oracle.backward(p["q"], p["k"], p["v"], p["do"], p["lg"], p["sel"], 4)
    for a, b in zip(g1, g2):
        np.testing.assert_allclose(a, b, atol=1e-11)


def test_gqa_equals_repeated_kv_heads():
    p = rand_problem(8, B=1, Hq=4, Hkv=1, N=24, D=8, block=4, K=2)
    o4, _ = oracle.forward(p["q"], p["k"], p["v"], p["lg"], p["sel"], 4)
    k4 = np.repeat(p["k"], 4, axis=1)
    v4 = np.repeat(p["v"], 4, axis=1)
    lg4 = np.repeat(p["lg"], 4, axis=1)
    sel4 = np.repeat(p["sel"], 4, axis=1)
    o1, _ = oracle.forward(p["q"], k4, v4, lg4, sel4, 4)
    np.testing.assert_allclose(o4, o1, atol=1e-13)


def test_multiplicative_gate_form_and_bounded_weights():
    # exp(z + log g) = g exp(z): output = sum g e^z v / sum g e^z over the attended set
    p = rand_problem(9, B=1, Hq=1, Hkv=1, N=24, D=8, block=4, K=2)
    o, lse = oracle.forward(p["q"], p["k"], p["v"], p["lg"], p["sel"], 4)
    q, k, v, lg, sel = p["q"][0, 0], p["k"][0, 0], p["v"][0, 0], p["lg"][0, 0], p["sel"][0, 0]
    for t in range(24):
        bt = t // 4
        num = np.zeros(8)
        den = 0.0
        for u in range(24):
            bu = u // 4
            if bu == bt and u <= t:
                w = 1.0
            elif bu < bt and sel[bt, bu]:
                w = math.exp(lg[bt, bu])
            else:
                continue
            e = w * math.exp(q[t] @ k[u] / math.sqrt(8))
            assert e / math.exp(lse[0, 0, t]) <= 1.0 + 1e-12       # bounded weight
            num += e * v[u]
            den += e
        np.testing.assert_allclose(o[0, 0, t], num / den, atol=1e-12)
        assert abs(lse[0, 0, t] - math.log(den)) < 1e-12


def test_current_block_always_participates():
    # a huge own-block key makes the output equal to its value even at K = 0
    p = rand_problem(10, N=16, block=4, K=0, Hq=1)
    q = p["q"].copy()
    k = p["k"].copy()
    v = p["v"].copy()
    q[0, 0, 13] = 10.0
    k[0, 0, 12] = 10.0
    o, _ = oracle.forward(q, k, v, p["lg"], p["sel"], 4)
    np.testing.assert_allclose(o[0, 0, 13], v[0, 0, 12], atol=1e-10)


# ---------------------------------------------------------------------------
# P5 / P6 / P7: gradients
# ---------------------------------------------------------------------------

def test_backward_matches_torch_autograd():
    p = rand_problem(11, B=1, Hq=4, Hkv=2, N=32, D=8, block=4, K=3)
    o_t, dq_t, dk_t, dv_t, dlg_t = torch_dense_model(p)
    dq, dk, dv, dlg = oracle.backward(p["q"], p["k"], p["v"], p["do"], p["lg"], p["sel"], 4)
    o, _ = oracle.forward(p["q"], p["k"], p["v"], p["lg"], p["sel"], 4)
    np.testing.assert_allclose(o, o_t, atol=1e-12)
    np.testing.assert_allclose(dq, dq_t, atol=1e-11)
    np.testing.assert_allclose(dk, dk_t, atol=1e-11)
    np.testing.assert_allclose(dv, dv_t, atol=1e-11)
    np.testing.assert_allclose(dlg, dlg_t, atol=1e-11)
    assert np.all(dlg[~p["sel"]] == 0.0)


def test_backward_term_masses_match_dense_autograd_terms():
    """The absolute term sums behind dK and dV (the scale of their rounding
    error): scale |dS|^T |Q| and P^T |dO| over the attending query rows of
    every query head of the kv group, with P and dS = dL/dz taken from torch
    autograd over the dense masked logits z; they bound |dK| and |dV|."""
    p = rand_problem(23, B=1, Hq=4, Hkv=2, N=32, D=8, block=4, K=2)
    dq, dk, dv, dlg, dkm, dvm = oracle.backward(p["q"], p["k"], p["v"], p["do"], p["lg"],
                                                p["sel"], 4, term_mass=True)
    dq0, dk0, dv0, dlg0 = oracle.backward(p["q"], p["k"], p["v"], p["do"], p["lg"], p["sel"], 4)
    for x, y in ((dq, dq0), (dk, dk0), (dv, dv0), (dlg, dlg0)):
        np.testing.assert_array_equal(x, y)
    B, Hq, N, D = p["q"].shape
    G = Hq // p["k"].shape[1]
    scale = 1.0 / math.sqrt(D)
    tb = torch.arange(N) // 4
    causal = torch.arange(N)[None, :] <= torch.arange(N)[:, None]
    lg = torch.from_numpy(np.where(np.isfinite(p["lg"]), p["lg"], 0.0))
    sel = torch.from_numpy(p["sel"])
    ref_k = np.zeros_like(dkm)
    ref_v = np.zeros_like(dvm)
    for h in range(Hq):
        hk = h // G
        same = tb[:, None] == tb[None, :]
        bias = torch.where(same & causal, torch.zeros(N, N, dtype=torch.float64),
                           torch.where(sel[0, hk][tb][:, tb], lg[0, hk][tb][:, tb],
                                       torch.full((N, N), -math.inf, dtype=torch.float64)))
        q = torch.from_numpy(p["q"][0, h])
        z = (scale * q @ torch.from_numpy(p["k"][0, hk]).T + bias).requires_grad_(True)
        pr = torch.softmax(z, dim=-1)
        do = torch.from_numpy(p["do"][0, h])
        (pr @ torch.from_numpy(p["v"][0, hk]) * do).sum().backward()
        ref_k[0, hk] += scale * (z.grad.abs().T @ q.abs()).numpy()
        ref_v[0, hk] += (pr.detach().T @ do.abs()).numpy()
    np.testing.assert_allclose(dkm, ref_k, atol=1e-11)
    np.testing.assert_allclose(dvm, ref_v, atol=1e-11)
    assert np.all(np.abs(dk) <= dkm + 1e-12) and np.all(np.abs(dv) <= dvm + 1e-12)
    assert np.any(dkm > np.abs(dk) + 1e-6) and np.any(dvm > np.abs(dv) + 1e-6)


def test_backward_kv_block_equals_full_backward():
    p = rand_problem(17, B=2, Hq=4, Hkv=2, N=32, D=8, block=4, K=2)
    _, dk, dv, _ = oracle.backward(p["q"], p["k"], p["v"], p["do"], p["lg"], p["sel"], 4)
    for (b, h, j) in [(0, 0, 0), (1, 1, 3), (0, 1, 7)]:
        dkj, dvj = oracle.backward_kv_block(p["q"], p["k"], p["v"], p["do"], p["lg"], p["sel"],
                                            4, b, h, j)
        np.testing.assert_allclose(dkj, dk[b, h, 4 * j:4 * j + 4], atol=1e-12)
        np.testing.assert_allclose(dvj, dv[b, h, 4 * j:4 * j + 4], atol=1e-12)


def test_backward_central_differences():
    p = rand_problem(12, B=1, Hq=2, Hkv=1, N=32, D=8, block=4, K=2)
    dq, dk, dv, dlg = oracle.backward(p["q"], p["k"], p["v"], p["do"], p["lg"], p["sel"], 4)
    rng = np.random.default_rng(0)
    h = 1e-6
    for name, grad in (("q", dq), ("k", dk), ("v", dv)):
        for _ in range(6):
            idx = tuple(rng.integers(0, s) for s in p[name].shape)
            xp = p[name].copy()
            xm = p[name].copy()
            xp[idx] += h
            xm[idx] -= h
            fd = (loss_of(p, **{name: xp}) - loss_of(p, **{name: xm})) / (2 * h)
            assert abs(fd - grad[idx]) <= 1e-7 * max(1.0, abs(fd)), (name, idx, fd, grad[idx])
    sel_idx = np.argwhere(p["sel"])
    for idx in sel_idx[:8]:
        idx = tuple(idx)
        lp = p["lg"].copy()
        lm = p["lg"].copy()
        lp[idx] += h
        lm[idx] -= h
        fd = (loss_of(p, lg=lp) - loss_of(p, lg=lm)) / (2 * h)
        assert abs(fd - dlg[idx]) <= 1e-7 * max(1.0, abs(fd))


def test_dlogg_equals_eq5_closed_form():
    # dLogG_m = g_m dg_m = sum_{k in B_m} p_k dO . (v_k - o)   (Eq. 5, App. D.1)
    p = rand_problem(13, B=1, Hq=2, Hkv=1, N=32, D=8, block=4, K=3)
    o, lse = oracle.forward(p["q"], p["k"], p["v"], p["lg"], p["sel"], 4)
    _, _, _, dlg = oracle.backward(p["q"], p["k"], p["v"], p["do"], p["lg"], p["sel"], 4)
    q, k, v, do = p["q"][0], p["k"][0, 0], p["v"][0, 0], p["do"][0]
    C = 8
    for i in range(C):
        for m in range(i):
            want = 0.0
            if p["sel"][0, 0, i, m]:
                for h in range(2):
                    for t in range(4 * i, 4 * i + 4):
                        for u in range(4 * m, 4 * m + 4):
                            z = q[h, t] @ k[u] / math.sqrt(8) + p["lg"][0, 0, i, m]
                            pr = math.exp(z - lse[0, h, t])
                            want += pr * (do[h, t] @ (v[u] - o[0, h, t]))
            assert abs(dlg[0, 0, i, m] - want) < 1e-12


def test_dlogg_row_identity_and_zero_pattern():
    # every query's dS sums to zero, so sum_m dLogG[i, m] = -(sum of dS over own-block keys)
    p = rand_problem(14, B=1, Hq=2, Hkv=1, N=32, D=8, block=4, K=2)
    _, _, _, dlg = oracle.backward(p["q"], p["k"], p["v"], p["do"], p["lg"], p["sel"], 4)
    assert np.all(dlg[~p["sel"]] == 0.0)
    q, k, v, do = p["q"][0], p["k"][0, 0], p["v"][0, 0], p["do"][0]
    o, lse = oracle.forward(p["q"], p["k"], p["v"], p["lg"], p["sel"], 4)
    for i in range(8):
        own = 0.0
        for h in range(2):
            for t in range(4 * i, 4 * i + 4):
                for u in range(4 * i, t + 1):
                    pr = math.exp(q[h, t] @ k[u] / math.sqrt(8) - lse[0, h, t])
                    own += pr * (do[h, t] @ v[u] - do[h, t] @ o[0, h, t])
        assert abs(dlg[0, 0, i].sum() + own) < 1e-11


def test_dscores_matches_autograd_through_scores_and_invariants():
    p = rand_problem(15, B=1, Hq=2, Hkv=2, N=40, D=8, block=4, K=3)
    _, _, _, dlg = oracle.backward(p["q"], p["k"], p["v"], p["do"], p["lg"], p["sel"], 4)
    ds = oracle.dscores(dlg, p["lg"], p["sel"])
    *_, ds_t = torch_dense_model(p, scores_leaf=True)
    C = 10
    tri = np.tril(np.ones((C, C), bool), -1)
    np.testing.assert_allclose(ds[..., tri], ds_t[..., tri], atol=1e-11)
    assert np.all(ds[..., ~tri] == 0.0)
    for b in range(1):
        for h in range(2):
            for i in range(1, C):
                assert abs(ds[b, h, i, :i].sum()) < 1e-12           # shift invariance
                g = np.exp(p["lg"][b, h, i, :i])
                s = p["sel"][b, h, i, :i]
                tot = dlg[b, h, i, :i][s].sum()
                # Eq. 8 sparse scope: unselected m get -g_m * sum_{l in I} g_l dg_l
                np.testing.assert_allclose(ds[b, h, i, :i][~s], -g[~s] * tot, atol=1e-13)


def test_dscores_central_differences_on_scores():
    p = rand_problem(16, B=1, Hq=2, Hkv=1, N=32, D=8, block=4, K=2)
    _, _, _, dlg = oracle.backward(p["q"], p["k"], p["v"], p["do"], p["lg"], p["sel"], 4)
    ds = oracle.dscores(dlg, p["lg"], p["sel"])
    h = 1e-6

    def loss_s(s):
        lg, _, sel = oracle.gate_threshold(s.astype(np.float32), 2)
        assert np.array_equal(sel, p["sel"]), "selection flipped"
        # gates from the float64 scores (fp32 rounding would swamp h)
        lg = lg.copy()
        for i in range(1, 8):
            x = s[0, 0, i, :i]
            lg[0, 0, i, :i] = x - (x.max() + np.log(np.exp(x - x.max()).sum()))
        return loss_of(p, lg=lg)

    base = p["scores"].astype(np.float64)
    checked = 0
    for i in range(3, 8):
        row = np.sort(base[0, 0, i, :i])[::-1]
        if row[1] - row[2] < 100 * h:        # K-th vs (K+1)-th gap too small
            continue
        for m in range(i):
            sp = base.copy()
            sm = base.copy()
            sp[0, 0, i, m] += h
            sm[0, 0, i, m] -= h
            fd = (loss_s(sp) - loss_s(sm)) / (2 * h)
            assert abs(fd - ds[0, 0, i, m]) <= 1e-7 * max(1.0, abs(fd))
            checked += 1
    assert checked > 10


# ---------------------------------------------------------------------------
# hand-worked example (tests/golden/hand_example_q0.txt)
# ---------------------------------------------------------------------------

def _read_golden(name):
    vals = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, idx, val = line.split()
            vals[(key, idx)] = float(val)
    return vals


def test_hand_worked_example():
    gold = _read_golden("hand_example_q0.txt")
    N, D, blk = 6, 2, 2
    t = np.arange(N, dtype=np.float64)
    q = np.zeros((1, 1, N, D))
    k = np.stack([t, np.zeros(N)], -1)[None, None]
    v = np.stack([t, np.ones(N)], -1)[None, None]
    do = np.stack([np.ones(N), np.zeros(N)], -1)[None, None]
    s = np.zeros((1, 1, 3, 3), np.float32)
    s[0, 0, 1, 0] = 0.5
    s[0, 0, 2, 0] = 0.0
    s[0, 0, 2, 1] = np.float32(math.log(3.0))
    lg, tau, sel = oracle.gate_threshold(s, 1)
    assert sel[0, 0, 1].tolist() == [True, False, False]
    assert sel[0, 0, 2].tolist() == [False, True, False]
    o, lse = oracle.forward(q, k, v, lg, sel, blk)
    dq, dk, dv, dlg = oracle.backward(q, k, v, do, lg, sel, blk)
    dsc = oracle.dscores(dlg, lg, sel)
    tol = 2e-7     # ln 3 is rounded to fp32 in the scores
    for ti in range(N):
        assert abs(o[0, 0, ti, 0] - gold[("o_x", str(ti))]) < tol
        assert abs(o[0, 0, ti, 1] - 1.0) < 1e-12
        assert abs(lse[0, 0, ti] - gold[("lse", str(ti))]) < tol
        assert abs(dv[0, 0, ti, 0] - gold[("dv_x", str(ti))]) < tol
        assert abs(dv[0, 0, ti, 1]) < 1e-12
    assert np.all(np.abs(dk) < 1e-12)
    assert abs(dlg[0, 0, 1, 0] - gold[("dlogg_1_0", "-")]) < tol
    assert abs(dlg[0, 0, 2, 1] - gold[("dlogg_2_1", "-")]) < tol
    assert dlg[0, 0, 2, 0] == gold[("dlogg_2_0", "-")]
    assert abs(dsc[0, 0, 2, 0] - gold[("dscore_2_0", "-")]) < tol
    assert abs(dsc[0, 0, 2, 1] - gold[("dscore_2_1", "-")]) < tol
    assert abs(dsc[0, 0, 1, 0] - gold[("dscore_1_0", "-")]) < 1e-12
    assert abs(dq[0, 0, 4, 0] - gold[("dq4_x", "-")]) < tol


# ---------------------------------------------------------------------------
# planted mistakes: each plausible slip must break at least one pin above
# ---------------------------------------------------------------------------

def test_planted_mistake_scaling_the_gate_is_caught(monkeypatch):
    orig = sas_oracle._attended_keys

    def scaled(i, block, sel_row, lg_row):
        keys, bias, kblk, mask = orig(i, block, sel_row, lg_row)
        return keys, bias / math.sqrt(8), kblk, mask       # sm_scale wrongly applied to log g

    monkeypatch.setattr(sas_oracle, "_attended_keys", scaled)
    with pytest.raises(AssertionError):
        test_forward_matches_sdpa_with_gate_bias_mask()


def test_planted_mistake_dscores_sign_is_caught(monkeypatch):
    orig = sas_oracle.dscores
    monkeypatch.setattr(oracle, "dscores", lambda a, b, c: -orig(a, b, c))
    with pytest.raises(AssertionError):
        test_hand_worked_example()


def test_planted_mistake_noncausal_current_block_is_caught(monkeypatch):
    orig = sas_oracle._attended_keys

    def noncausal(i, block, sel_row, lg_row):
        keys, bias, kblk, mask = orig(i, block, sel_row, lg_row)
        return keys, bias, kblk, np.ones_like(mask)

    monkeypatch.setattr(sas_oracle, "_attended_keys", noncausal)
    with pytest.raises(AssertionError):
        test_budget_zero_is_block_local_causal_attention()


def test_planted_mistake_gates_normalised_over_selected_only_is_caught(monkeypatch):
    orig = sas_oracle.gate_threshold

    def sel_norm(scores, k):
        lg, tau, sel = orig(scores, k)
        lg = lg.copy()
        for b, h, i in np.ndindex(*lg.shape[:3]):
            s = sel[b, h, i]
            if s.any():
                x = scores[b, h, i][s].astype(np.float64)
                lg[b, h, i][s] = x - (x.max() + np.log(np.exp(x - x.max()).sum()))
        return lg, tau, sel

    monkeypatch.setattr(oracle, "gate_threshold", sel_norm)
    with pytest.raises(AssertionError):
        test_gates_sum_to_one_over_historical_blocks()
