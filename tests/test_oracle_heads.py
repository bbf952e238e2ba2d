"""Pins of the oracle's per-query-head gates (score heads Hs = Hq; the pages'
training kernel takes a log gate per query position and attention head, while
the serving path selects per query group): torch autograd with a per-head
bias, the reduction to per-group gates when every head of a group carries the
same scores, and G = 1.  All CPU.
"""

import math

import numpy as np
import torch

import oracle


def problem(seed, B=1, Hq=4, Hkv=2, N=40, D=8, block=4, K=3, per_head=True):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, Hq, N, D))
    k = rng.standard_normal((B, Hkv, N, D))
    v = rng.standard_normal((B, Hkv, N, D))
    do = rng.standard_normal((B, Hq, N, D))
    c = N // block
    hs = Hq if per_head else Hkv
    scores = (rng.standard_normal((B, hs, c, c)) * 1.5).astype(np.float32)
    lg, _, sel = oracle.gate_threshold(scores, K)
    return dict(q=q, k=k, v=v, do=do, scores=scores, lg=lg, sel=sel, block=block)


def torch_per_head(p):
    B, Hq, N, D = p["q"].shape
    Hkv = p["k"].shape[1]
    G = Hq // Hkv
    Hs = p["scores"].shape[1]
    Gs = Hq // Hs
    blk = p["block"]
    C = N // blk
    scale = 1.0 / math.sqrt(D)
    q = torch.tensor(p["q"], requires_grad=True)
    k = torch.tensor(p["k"], requires_grad=True)
    v = torch.tensor(p["v"], requires_grad=True)
    s = torch.tensor(p["scores"].astype(np.float64), requires_grad=True)
    tri = torch.tril(torch.ones(C, C, dtype=torch.bool), diagonal=-1)
    s_m = torch.where(tri, s, torch.tensor(-1e30, dtype=torch.float64))
    lg = torch.where(tri, s - torch.logsumexp(s_m, dim=-1, keepdim=True), torch.zeros_like(s))
    sel = torch.from_numpy(p["sel"])
    tok = torch.arange(N)
    tb = tok // blk
    same = tb[:, None] == tb[None, :]
    causal = tok[None, :] <= tok[:, None]
    outs = []
    for b in range(B):
        for h in range(Hq):
            sh, hk = h // Gs, h // G
            lgb = lg[b, sh][tb][:, tb]
            keep = (same & causal) | sel[b, sh][tb][:, tb]
            z = scale * q[b, h] @ k[b, hk].T + torch.where(same, torch.zeros_like(lgb), lgb)
            z = torch.where(keep, z, torch.tensor(-math.inf, dtype=torch.float64))
            outs.append(torch.softmax(z, -1) @ v[b, hk])
    o = torch.stack(outs).reshape(B, Hq, N, D)
    (o * torch.from_numpy(p["do"])).sum().backward()
    return o.detach().numpy(), q.grad.numpy(), k.grad.numpy(), v.grad.numpy(), s.grad.numpy()


def test_per_head_gates_match_torch_autograd():
    p = problem(1)
    o, _ = oracle.forward(p["q"], p["k"], p["v"], p["lg"], p["sel"], 4)
    dq, dk, dv, dlg = oracle.backward(p["q"], p["k"], p["v"], p["do"], p["lg"], p["sel"], 4)
    ds = oracle.dscores(dlg, p["lg"], p["sel"])
    o_t, dq_t, dk_t, dv_t, ds_t = torch_per_head(p)
    np.testing.assert_allclose(o, o_t, rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(dq, dq_t, rtol=1e-10, atol=1e-10)
    np.testing.assert_allclose(dk, dk_t, rtol=1e-10, atol=1e-10)
    np.testing.assert_allclose(dv, dv_t, rtol=1e-10, atol=1e-10)
    tri = np.tril(np.ones((10, 10), bool), -1)
    np.testing.assert_allclose(ds[..., tri], ds_t[..., tri], rtol=1e-10, atol=1e-10)
    # per-head selections really differ across the heads of a group
    assert not np.array_equal(p["sel"][0, 0], p["sel"][0, 1])


def test_identical_head_scores_reduce_to_group_gates():
    pg = problem(2, per_head=False)
    ph = dict(pg)
    ph["scores"] = np.repeat(pg["scores"], 2, axis=1)       # G = 2 heads per group
    ph["lg"], _, ph["sel"] = oracle.gate_threshold(ph["scores"], 3)
    og, lg_ = oracle.forward(pg["q"], pg["k"], pg["v"], pg["lg"], pg["sel"], 4)
    oh, lh = oracle.forward(ph["q"], ph["k"], ph["v"], ph["lg"], ph["sel"], 4)
    np.testing.assert_allclose(oh, og, rtol=1e-13, atol=1e-13)
    gg = oracle.backward(pg["q"], pg["k"], pg["v"], pg["do"], pg["lg"], pg["sel"], 4)
    gh = oracle.backward(ph["q"], ph["k"], ph["v"], ph["do"], ph["lg"], ph["sel"], 4)
    for a, b in zip(gg[:3], gh[:3]):
        np.testing.assert_allclose(b, a, rtol=1e-12, atol=1e-12)
    # the group's log-gate gradient is the sum over its heads' gradients
    np.testing.assert_allclose(gh[3].reshape(1, 2, 2, 10, 10).sum(2), gg[3], rtol=1e-12,
                               atol=1e-12)


def test_group_of_one_is_the_same_either_way():
    p = problem(3, Hq=2, Hkv=2, per_head=True)
    o, _ = oracle.forward(p["q"], p["k"], p["v"], p["lg"], p["sel"], 4)
    o_t, *_ = torch_per_head(p)
    np.testing.assert_allclose(o, o_t, rtol=1e-11, atol=1e-11)


def test_per_head_hard_gates_reduce_to_group_gates():
    """ste_gate_grad with per-head scores that repeat the group's scores sums
    to the group-gate result."""
    from oracle import sas_oracle
    pg = problem(4, per_head=False)
    scores_h = np.repeat(pg["scores"], 2, axis=1)
    lg_h, _, sel_h = oracle.gate_threshold(scores_h, 3)
    dg_g = sas_oracle.ste_gate_grad(pg["q"], pg["k"], pg["v"], pg["do"], pg["lg"], pg["sel"], 4)
    dg_h = sas_oracle.ste_gate_grad(pg["q"], pg["k"], pg["v"], pg["do"], lg_h, sel_h, 4)
    np.testing.assert_allclose(dg_h.reshape(1, 2, 2, 10, 10).sum(2), dg_g, rtol=1e-12, atol=1e-12)
