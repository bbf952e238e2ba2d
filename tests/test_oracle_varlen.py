"""Pins of the oracle's variable-length batches (the varlen sequences of the
pages' training kernel, in a padded layout): full lengths change nothing; a
ragged batch equals the padded fixed-length run with dO zeroed on the padding
rows (restricted to the valid rows and keys); padding outputs and padding-key
gradients are exactly zero; torch autograd of a per-sequence dense model over
the valid tokens.  All CPU.
"""

import math

import numpy as np
import torch

import oracle
from oracle import sas_oracle


def problem(seed, B=2, Hq=4, Hkv=2, N=48, D=8, block=4, K=3):
    rng = np.random.default_rng(seed)
    return dict(q=rng.standard_normal((B, Hq, N, D)), k=rng.standard_normal((B, Hkv, N, D)),
                v=rng.standard_normal((B, Hkv, N, D)), do=rng.standard_normal((B, Hq, N, D)),
                scores=(rng.standard_normal((B, Hkv, N // block, N // block)) * 1.5).astype(np.float32),
                block=block, K=K)


def run(p, lens):
    lg, tau, sel = oracle.gate_threshold(p["scores"], p["K"], seq_lens=lens, block=p["block"])
    o, lse = oracle.forward(p["q"], p["k"], p["v"], lg, sel, p["block"], seq_lens=lens)
    g = oracle.backward(p["q"], p["k"], p["v"], p["do"], lg, sel, p["block"], seq_lens=lens)
    return lg, tau, sel, o, lse, g


def test_full_lengths_change_nothing():
    p = problem(1)
    a = run(p, None)
    b = run(p, [48, 48])
    for x, y in zip(a[:5], b[:5]):
        np.testing.assert_array_equal(x, y)
    for x, y in zip(a[5], b[5]):
        np.testing.assert_array_equal(x, y)


def test_ragged_batch_equals_padded_run_with_zero_padding_gradients():
    p = problem(2)
    lens = [37, 22]                      # ragged last blocks (block 4)
    lg, tau, sel, o, lse, (dq, dk, dv, dlg) = run(p, lens)
    # the fixed-length run on the same tensors, dO zero on padding rows
    pz = dict(p)
    pz["do"] = p["do"].copy()
    for b, n in enumerate(lens):
        pz["do"][b, :, n:] = 0.0
    lg2, _, sel2 = oracle.gate_threshold(p["scores"], p["K"])
    o2, lse2 = oracle.forward(p["q"], p["k"], p["v"], lg2, sel2, 4)
    dq2, dk2, dv2, dlg2 = oracle.backward(pz["q"], pz["k"], pz["v"], pz["do"], lg2, sel2, 4)
    np.testing.assert_array_equal(lg, lg2)                   # gates are a function of the scores
    for b, n in enumerate(lens):
        cb = -(-n // 4)
        np.testing.assert_array_equal(sel[b, :, :cb], sel2[b, :, :cb])
        assert not sel[b, :, cb:].any() and np.all(np.isposinf(tau[b, :, cb:]))
        np.testing.assert_allclose(o[b, :, :n], o2[b, :, :n], rtol=1e-13, atol=1e-13)
        np.testing.assert_allclose(lse[b, :, :n], lse2[b, :, :n], rtol=1e-13, atol=1e-13)
        np.testing.assert_allclose(dq[b, :, :n], dq2[b, :, :n], rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(dk[b, :, :n], dk2[b, :, :n], rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(dv[b, :, :n], dv2[b, :, :n], rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(dlg[b, :, :cb], dlg2[b, :, :cb], rtol=1e-12, atol=1e-12)
        for t in (o, lse, dq):
            assert np.all(t[b, :, n:] == 0.0)
        assert np.all(dk[b, :, n:] == 0.0) and np.all(dv[b, :, n:] == 0.0)
        assert np.all(dlg[b, :, cb:] == 0.0)


def test_ragged_sequence_matches_torch_autograd():
    p = problem(3, B=1, Hq=2, Hkv=1, N=40, D=8, block=4, K=2)
    n = 27
    lg, tau, sel, o, lse, (dq, dk, dv, dlg) = run(p, [n])
    blk = 4
    scale = 1.0 / math.sqrt(8)
    q = torch.tensor(p["q"][0, :, :n], requires_grad=True)
    k = torch.tensor(p["k"][0, 0, :n], requires_grad=True)
    v = torch.tensor(p["v"][0, 0, :n], requires_grad=True)
    lgt = torch.tensor(np.where(np.isfinite(lg[0, 0]), lg[0, 0], 0.0), requires_grad=True)
    tok = torch.arange(n)
    tb = tok // blk
    same = tb[:, None] == tb[None, :]
    causal = tok[None, :] <= tok[:, None]
    selm = torch.from_numpy(sel[0, 0])[tb][:, tb]
    keep = (same & causal) | selm
    outs = []
    for h in range(2):
        z = scale * q[h] @ k.T + torch.where(same, torch.zeros(n, n, dtype=torch.float64),
                                             lgt[tb][:, tb])
        z = torch.where(keep, z, torch.tensor(-math.inf, dtype=torch.float64))
        outs.append(torch.softmax(z, -1) @ v)
    ot = torch.stack(outs)
    (ot * torch.from_numpy(p["do"][0, :, :n])).sum().backward()
    np.testing.assert_allclose(o[0, :, :n], ot.detach().numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dq[0, :, :n], q.grad.numpy(), rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(dk[0, 0, :n], k.grad.numpy(), rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(dv[0, 0, :n], v.grad.numpy(), rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(dlg[0, 0][sel[0, 0]], lgt.grad.numpy()[sel[0, 0]], rtol=1e-11,
                               atol=1e-11)


def test_varlen_hard_gates_equal_padded_run():
    p = problem(4)
    lens = [41, 13]
    lg, _, sel, *_ = run(p, lens)
    dg = sas_oracle.ste_gate_grad(p["q"], p["k"], p["v"], p["do"], lg, sel, 4, seq_lens=lens)
    do0 = p["do"].copy()
    for b, n in enumerate(lens):
        do0[b, :, n:] = 0.0
    lg2, _, sel2 = oracle.gate_threshold(p["scores"], p["K"])
    dg2 = sas_oracle.ste_gate_grad(p["q"], p["k"], p["v"], do0, lg2, sel2, 4)
    for b, n in enumerate(lens):
        cb = -(-n // 4)
        np.testing.assert_allclose(dg[b, :, :cb], dg2[b, :, :cb], rtol=1e-12, atol=1e-12)
        assert np.all(dg[b, :, cb:] == 0.0)


def test_backward_kv_block_with_lengths_equals_full_backward():
    """The one-key-block evaluation used to sample dK / dV at large shapes
    agrees with the full backward on a ragged batch (padding rows add
    nothing), at the inner and the outer gate position."""
    p = problem(19, B=2, Hq=4, Hkv=2, N=32, D=8, block=4, K=2)
    lens = np.array([32, 13])
    lg, _, sel = oracle.gate_threshold(p["scores"], 2, seq_lens=lens, block=4)
    for pos in ("inner", "outer"):
        _, dk, dv, _ = oracle.backward(p["q"], p["k"], p["v"], p["do"], lg, sel, 4, gate_pos=pos,
                                       seq_lens=lens)
        for (b, h, j) in [(0, 0, 0), (1, 1, 3), (1, 0, 2), (0, 1, 7)]:
            dkj, dvj = oracle.backward_kv_block(p["q"], p["k"], p["v"], p["do"], lg, sel, 4, b, h,
                                                j, gate_pos=pos, seq_lens=lens)
            np.testing.assert_allclose(dkj, dk[b, h, 4 * j:4 * j + 4], atol=1e-12)
            np.testing.assert_allclose(dvj, dv[b, h, 4 * j:4 * j + 4], atol=1e-12)
    assert np.all(dk[1, :, 13:] == 0.0) and np.all(dv[1, :, 13:] == 0.0)
