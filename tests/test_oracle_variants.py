"""Pins of the oracle's gate variants (Sec. 4.1 "Components of learnable
ranking", Tab. 1): gate position (inner / outer) and gate activation
(softmax / sigmoid / raw logits), against torch autograd through the same
formulas written with torch ops, torch's logsigmoid, the outer-gate closed
form of Eq. 5, and special cases.  All CPU.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from oracle import sas_oracle


def rand_problem(seed, B=1, Hq=2, Hkv=1, N=32, D=8, block=4, K=2, act="softmax"):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, Hq, N, D))
    k = rng.standard_normal((B, Hkv, N, D))
    v = rng.standard_normal((B, Hkv, N, D))
    do = rng.standard_normal((B, Hq, N, D))
    c = N // block
    scores = (rng.standard_normal((B, Hkv, c, c)) * 1.5).astype(np.float32)
    lg, tau, sel = oracle.gate_threshold(scores, K, act=act)
    return dict(q=q, k=k, v=v, do=do, scores=scores, lg=lg, sel=sel, block=block, K=K, act=act)


def torch_model(p, gate_pos):
    """Loss sum(o * dO) of the gated block-sparse attention written with torch
    ops; the selector scores are the leaf (selection held fixed)."""
    B, Hq, N, D = p["q"].shape
    Hkv = p["k"].shape[1]
    G = Hq // Hkv
    blk = p["block"]
    C = N // blk
    scale = 1.0 / math.sqrt(D)
    q = torch.tensor(p["q"], requires_grad=True)
    k = torch.tensor(p["k"], requires_grad=True)
    v = torch.tensor(p["v"], requires_grad=True)
    s = torch.tensor(p["scores"].astype(np.float64), requires_grad=True)
    tri = torch.tril(torch.ones(C, C, dtype=torch.bool), diagonal=-1)
    if p["act"] == "softmax":
        s_m = torch.where(tri, s, torch.tensor(-1e30, dtype=torch.float64))
        lg_hist = s - torch.logsumexp(s_m, dim=-1, keepdim=True)
    elif p["act"] == "sigmoid":
        lg_hist = torch.nn.functional.logsigmoid(s)
    else:
        lg_hist = s
    lg = torch.where(tri, lg_hist, torch.zeros_like(s))
    sel = torch.from_numpy(p["sel"])
    tok = torch.arange(N)
    tb = tok // blk
    same = tb[:, None] == tb[None, :]
    causal = tok[None, :] <= tok[:, None]
    outs = []
    for b in range(B):
        for h in range(Hq):
            hk = h // G
            lgb = lg[b, hk][tb][:, tb]                    # log g of (query block, key block)
            keep = (same & causal) | sel[b, hk][tb][:, tb]
            z = scale * q[b, h] @ k[b, hk].T
            if gate_pos == "inner":
                z = z + torch.where(same, torch.zeros_like(lgb), lgb)
                z = torch.where(keep, z, torch.tensor(-math.inf, dtype=torch.float64))
                outs.append(torch.softmax(z, -1) @ v[b, hk])
            else:
                z = torch.where(keep, z, torch.tensor(-math.inf, dtype=torch.float64))
                pr = torch.softmax(z, -1)
                gk = torch.where(same, torch.zeros_like(lgb), lgb).exp()   # per (query, key)
                outs.append((pr * gk) @ v[b, hk])
    o = torch.stack(outs).reshape(B, Hq, N, D)
    loss = (o * torch.from_numpy(p["do"])).sum()
    loss.backward()
    return (o.detach().numpy(), q.grad.numpy(), k.grad.numpy(), v.grad.numpy(), s.grad.numpy())


def test_sigmoid_and_raw_log_gates_and_shared_selection():
    p = rand_problem(1)
    s = p["scores"]
    C = s.shape[-1]
    tri = np.tril(np.ones((C, C), bool), -1)
    lg_sig, tau_sig, sel_sig = oracle.gate_threshold(s, 2, act="sigmoid")
    lg_raw, tau_raw, sel_raw = oracle.gate_threshold(s, 2, act="raw")
    want = torch.nn.functional.logsigmoid(torch.from_numpy(s.astype(np.float64))).numpy()
    np.testing.assert_allclose(lg_sig[..., tri], want[..., tri], rtol=1e-14, atol=1e-14)
    np.testing.assert_array_equal(lg_raw[..., tri], s.astype(np.float64)[..., tri])
    # the selection is made on s itself, so it does not depend on the activation
    np.testing.assert_array_equal(sel_sig, p["sel"])
    np.testing.assert_array_equal(sel_raw, p["sel"])
    np.testing.assert_array_equal(tau_sig, tau_raw)
    for lg in (lg_sig, lg_raw):
        assert np.all(np.diagonal(lg, axis1=-2, axis2=-1) == 0.0)    # g0 = 1 (Eq. 4)
        assert np.all(np.isneginf(lg[..., np.triu(np.ones((C, C), bool), 1)]))


@pytest.mark.parametrize("act", ["softmax", "sigmoid", "raw"])
@pytest.mark.parametrize("gate_pos", ["inner", "outer"])
def test_variant_matches_torch_autograd(act, gate_pos):
    p = rand_problem(2 + len(act) + len(gate_pos), B=1, Hq=4, Hkv=2, N=40, D=8, block=4, K=3,
                     act=act)
    o, lse = oracle.forward(p["q"], p["k"], p["v"], p["lg"], p["sel"], 4, gate_pos=gate_pos)
    dq, dk, dv, dlg = oracle.backward(p["q"], p["k"], p["v"], p["do"], p["lg"], p["sel"], 4,
                                      gate_pos=gate_pos)
    ds = oracle.dscores(dlg, p["lg"], p["sel"], act=act)
    o_t, dq_t, dk_t, dv_t, ds_t = torch_model(p, gate_pos)
    np.testing.assert_allclose(o, o_t, rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(dq, dq_t, rtol=1e-10, atol=1e-10)
    np.testing.assert_allclose(dk, dk_t, rtol=1e-10, atol=1e-10)
    np.testing.assert_allclose(dv, dv_t, rtol=1e-10, atol=1e-10)
    C = 10
    tri = np.tril(np.ones((C, C), bool), -1)
    np.testing.assert_allclose(ds[..., tri], ds_t[..., tri], rtol=1e-10, atol=1e-10)
    assert np.all(ds[..., ~tri] == 0.0)
    # dLogG is zero off the selection in every variant (sparse scope)
    assert np.all(dlg[~p["sel"]] == 0.0)


def test_outer_gate_gradient_is_eq5_closed_form():
    """Eq. 5 (outer): dg_m = sum_{i in B_m} p_i dO^T v_i with the ungated
    probabilities p; dLogG = g_m dg_m."""
    p = rand_problem(7, B=1, Hq=2, Hkv=1, N=32, D=8, block=4, K=2)
    _, _, _, dlg = oracle.backward(p["q"], p["k"], p["v"], p["do"], p["lg"], p["sel"], 4,
                                   gate_pos="outer")
    q, k, v, do, sel, lg = p["q"], p["k"], p["v"], p["do"], p["sel"], p["lg"]
    blk, scale = 4, 1.0 / math.sqrt(8)
    for i in range(1, 8):
        for m in range(i):
            if not sel[0, 0, i, m]:
                continue
            want = 0.0
            for h in range(2):
                for t in range(i * blk, (i + 1) * blk):
                    keys = [u for u in range(t + 1) if u // blk == i or sel[0, 0, i, u // blk]]
                    z = np.array([scale * q[0, h, t] @ k[0, 0, u] for u in keys])
                    pr = np.exp(z - z.max())
                    pr /= pr.sum()
                    for pu, u in zip(pr, keys):
                        if u // blk == m:
                            want += pu * (do[0, h, t] @ v[0, 0, u])
            want *= math.exp(lg[0, 0, i, m])
            assert abs(dlg[0, 0, i, m] - want) < 1e-11 * max(1.0, abs(want))


def test_outer_with_unit_gates_is_inner_with_zero_bias():
    p = rand_problem(8, B=1, Hq=2, Hkv=1, N=32, D=8, block=4, K=2)
    zero = np.where(np.isfinite(p["lg"]), 0.0, p["lg"])
    o_in, lse_in = oracle.forward(p["q"], p["k"], p["v"], zero, p["sel"], 4)
    o_out, lse_out = oracle.forward(p["q"], p["k"], p["v"], zero, p["sel"], 4, gate_pos="outer")
    np.testing.assert_allclose(o_out, o_in, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(lse_out, lse_in, rtol=1e-13, atol=1e-13)


def test_planted_mistake_outer_dlogg_from_ds_is_caught(monkeypatch):
    """Summing dS (the inner rule) for the outer gate must fail the torch pin."""
    p = rand_problem(9, B=1, Hq=2, Hkv=1, N=32, D=8, block=4, K=2)
    real = sas_oracle.backward

    def wrong(*a, **kw):
        kw["gate_pos"] = "inner" if kw.get("gate_pos") == "outer" else kw.get("gate_pos", "inner")
        dq, dk, dv, dlg = real(*a, **kw)
        return dq, dk, dv, dlg
    _, _, _, dlg_bad = wrong(p["q"], p["k"], p["v"], p["do"], p["lg"], p["sel"], 4,
                             gate_pos="outer")
    ds_bad = oracle.dscores(dlg_bad, p["lg"], p["sel"])
    *_, ds_t = torch_model(p, "outer")
    tri = np.tril(np.ones((8, 8), bool), -1)
    assert np.max(np.abs(ds_bad[..., tri] - ds_t[..., tri])) > 1e-3


# ---------------------------------------------------------------------------
# hard Top-K gates with the straight-through estimator (Eq. 7, Tab. 1 row 8)
# ---------------------------------------------------------------------------

def torch_ste_model(p):
    """Multiplicative-gate form p_i = g_hat e^z_i / sum_j g_hat e^z_j with
    g_hat = (g_hard - g).detach() + g and g = softmax(s) over the historical
    blocks (the current block keeps 1); scores are the leaf."""
    B, Hq, N, D = p["q"].shape
    Hkv = p["k"].shape[1]
    G = Hq // Hkv
    blk = p["block"]
    C = N // blk
    scale = 1.0 / math.sqrt(D)
    q = torch.tensor(p["q"], requires_grad=True)
    k = torch.tensor(p["k"], requires_grad=True)
    v = torch.tensor(p["v"], requires_grad=True)
    s = torch.tensor(p["scores"].astype(np.float64), requires_grad=True)
    tri = torch.tril(torch.ones(C, C, dtype=torch.bool), diagonal=-1)
    s_m = torch.where(tri, s, torch.tensor(-1e30, dtype=torch.float64))
    g = torch.where(tri, torch.softmax(s_m, dim=-1), torch.zeros_like(s))
    hard = torch.from_numpy(p["sel"]).to(torch.float64)
    ghat = (hard - g).detach() + g
    ghat = ghat + torch.eye(C, dtype=torch.float64)          # current block: 1
    tok = torch.arange(N)
    tb = tok // blk
    causal = tok[None, :] <= tok[:, None]
    outs = []
    for b in range(B):
        for h in range(Hq):
            hk = h // G
            w = ghat[b, hk][tb][:, tb]
            z = scale * q[b, h] @ k[b, hk].T
            z = torch.where(causal, z, torch.tensor(-math.inf, dtype=torch.float64))
            e = torch.exp(z - z.max(dim=-1, keepdim=True).values) * w
            outs.append((e / e.sum(-1, keepdim=True)) @ v[b, hk])
    o = torch.stack(outs).reshape(B, Hq, N, D)
    (o * torch.from_numpy(p["do"])).sum().backward()
    return o.detach().numpy(), q.grad.numpy(), k.grad.numpy(), v.grad.numpy(), s.grad.numpy()


def test_ste_hard_gates_match_torch_autograd():
    p = rand_problem(31, B=1, Hq=4, Hkv=2, N=40, D=8, block=4, K=3)
    zero = np.where(np.isfinite(p["lg"]), 0.0, p["lg"])
    o, _ = oracle.forward(p["q"], p["k"], p["v"], zero, p["sel"], 4)
    dq, dk, dv, dlg_sel = oracle.backward(p["q"], p["k"], p["v"], p["do"], zero, p["sel"], 4)
    dg = sas_oracle.ste_gate_grad(p["q"], p["k"], p["v"], p["do"], p["lg"], p["sel"], 4)
    ds = sas_oracle.dscores_from_dg(dg, p["lg"])
    o_t, dq_t, dk_t, dv_t, ds_t = torch_ste_model(p)
    np.testing.assert_allclose(o, o_t, rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(dq, dq_t, rtol=1e-10, atol=1e-10)
    np.testing.assert_allclose(dk, dk_t, rtol=1e-10, atol=1e-10)
    np.testing.assert_allclose(dv, dv_t, rtol=1e-10, atol=1e-10)
    C = 10
    tri = np.tril(np.ones((C, C), bool), -1)
    np.testing.assert_allclose(ds[..., tri], ds_t[..., tri], rtol=1e-9, atol=1e-10)
    # on selected blocks the STE gradient is the block's dS sum (unit gates)
    np.testing.assert_allclose(dg[p["sel"]], dlg_sel[p["sel"]], rtol=1e-11, atol=1e-12)
    # dropped blocks get a gradient of their own (Eq. 7), unlike the sparse scope
    assert np.count_nonzero(np.abs(dg[tri[None, None] & ~p["sel"]]) > 1e-9) > 10


def test_ste_gate_grad_sampled_rows_equal_full():
    """Sampled gate rows of the straight-through gate gradient equal those
    rows of the full evaluation, and every other row stays 0."""
    p = rand_problem(33, B=2, Hq=4, Hkv=2, N=40, D=8, block=4, K=3)
    full = sas_oracle.ste_gate_grad(p["q"], p["k"], p["v"], p["do"], p["lg"], p["sel"], 4)
    rows = [(0, 0, 9), (1, 1, 4), (1, 0, 1), (0, 1, 0)]
    part = sas_oracle.ste_gate_grad(p["q"], p["k"], p["v"], p["do"], p["lg"], p["sel"], 4,
                                    rows=rows)
    mask = np.zeros(full.shape[:3], bool)
    for (b, h, i) in rows:
        mask[b, h, i] = True
    np.testing.assert_allclose(part[mask], full[mask], rtol=1e-13, atol=1e-14)
    assert np.all(part[~mask] == 0.0)
    assert np.count_nonzero(part[mask]) > 5
