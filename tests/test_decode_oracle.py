"""Pins of the sparse-decode oracle against what the pages and the mathematics fix.

SAS inference step (Sec. 4.3 Alg. 2; Sec. 5.1 "Inference implementation"):
Top-K of the selector scores per query group, then softmax(q K_S^T) V_S over
the current block and the selected blocks, with no gates.  Pins:
  * the selection equals torch.topk on tie-free rows; edge cases (no
    history, K >= history, K = 0) and the keep-all-ties rule;
  * with every block selected the attention equals torch's
    scaled_dot_product_attention (float64, CPU) of the query over the whole
    contiguous cache, and with K = 0 over the current block alone; any
    selection equals SDPA with a boolean mask built from the selected set;
    the paged pool is built from the contiguous cache by an independent
    scatter through a shuffled block table;
  * closed form: q = 0 gives uniform weights, so o is the mean of the
    attended values and lse = log(#attended);
  * planted mistakes in the oracle fail these pins.
All CPU.
"""

import math

import numpy as np
import pytest
import torch

import oracle.sas_decode_oracle as dec


def make_case(seed, B=3, Hq=4, Hkv=2, D=16, block=4, cmax=9, lens=(1, 17, 36), K=3):
    g = torch.Generator().manual_seed(seed)
    n_max = cmax * block
    q = torch.randn(B, Hq, D, generator=g, dtype=torch.float64)
    kc = torch.randn(B, Hkv, n_max, D, generator=g, dtype=torch.float64)   # contiguous caches
    vc = torch.randn(B, Hkv, n_max, D, generator=g, dtype=torch.float64)
    scores = torch.randn(B, Hkv, cmax, generator=g).numpy().astype(np.float32)
    # paged pool: logical block m of sequence s -> a shuffled page
    P = B * cmax + 5
    perm = torch.randperm(P, generator=g)[:B * cmax].reshape(B, cmax)
    kp = torch.zeros(P, Hkv, block, D, dtype=torch.float64)
    vp = torch.zeros(P, Hkv, block, D, dtype=torch.float64)
    for s in range(B):
        for m in range(cmax):
            kp[perm[s, m]] = kc[s, :, m * block:(m + 1) * block].clone()
            vp[perm[s, m]] = vc[s, :, m * block:(m + 1) * block].clone()
    return dict(q=q, kc=kc, vc=vc, kp=kp, vp=vp, bt=perm.numpy(), scores=scores,
                lens=np.array(lens), block=block, K=K, G=Hq // Hkv)


def sdpa_masked(case, keep):
    """torch SDPA of each query over the contiguous cache with a boolean key mask
    keep[b, hk, pos] (independent of the oracle's gather)."""
    q, kc, vc = case["q"], case["kc"], case["vc"]
    B, Hq, D = q.shape
    G = case["G"]
    o = torch.zeros(B, Hq, D, dtype=torch.float64)
    lse = torch.zeros(B, Hq, dtype=torch.float64)
    for b in range(B):
        for h in range(Hq):
            hk = h // G
            m = torch.from_numpy(keep[b, hk])
            o[b, h] = torch.nn.functional.scaled_dot_product_attention(
                q[b, h][None, None, None], kc[b, hk][None, None], vc[b, hk][None, None],
                attn_mask=m[None, None, None])[0, 0, 0]
            z = (kc[b, hk][m] @ q[b, h]) / math.sqrt(D)
            lse[b, h] = torch.logsumexp(z, 0)
    return o.numpy(), lse.numpy()


def keep_from_blocks(case, sel):
    """Position mask: current block up to n - 1 plus every selected block."""
    B, Hkv = case["kc"].shape[:2]
    n_max = case["kc"].shape[2]
    blk = case["block"]
    keep = np.zeros((B, Hkv, n_max), bool)
    for b in range(B):
        n = int(case["lens"][b])
        c = (n - 1) // blk
        for hk in range(Hkv):
            keep[b, hk, c * blk:n] = True
            for m in range(c):
                if sel[b, hk, m]:
                    keep[b, hk, m * blk:(m + 1) * blk] = True
    return keep


def run_oracle(case, sel):
    return dec.decode_attn(case["q"].numpy(), case["kp"].numpy(), case["vp"].numpy(), case["bt"],
                           case["lens"], sel, case["block"])


# ---------------------------------------------------------------- selection

def test_select_matches_topk_on_tie_free_rows():
    rng = np.random.default_rng(0)
    B, H, cmax, blk = 4, 3, 40, 8
    scores = rng.standard_normal((B, H, cmax)).astype(np.float32)
    lens = np.array([1, 9, 150, 320])
    for K in (0, 1, 5, 19, 40):
        tau, sel = dec.decode_select(scores, lens, blk, K)
        for b in range(B):
            c = (lens[b] - 1) // blk
            for h in range(H):
                want = np.zeros(cmax, bool)
                if c > 0 and K > 0:
                    top = torch.topk(torch.from_numpy(scores[b, h, :c]), min(K, c)).indices.numpy()
                    want[top] = True
                assert np.array_equal(sel[b, h], want), (K, b, h)
                assert sel[b, h].sum() == min(K, c)
                assert not sel[b, h, c:].any()


def test_select_edge_cases_and_ties():
    s = np.array([[[1.0, 2.0, 2.0, 2.0, 0.5, 9.0, 9.0]]], np.float32)
    # n = 21 tokens, block 4 -> current block 5, history = blocks 0..4
    tau, sel = dec.decode_select(s, [21], 4, 2)
    assert tau[0, 0] == np.float32(2.0)
    assert sel[0, 0].tolist() == [False, True, True, True, False, False, False]   # all ties kept
    tau, sel = dec.decode_select(s, [21], 4, 0)
    assert np.isposinf(tau[0, 0]) and not sel.any()
    tau, sel = dec.decode_select(s, [21], 4, 5)
    assert np.isneginf(tau[0, 0]) and sel[0, 0, :5].all() and not sel[0, 0, 5:].any()
    tau, sel = dec.decode_select(s, [4], 4, 3)         # first block: no history
    assert not sel.any()


# ---------------------------------------------------------------- attention

@pytest.mark.parametrize("K", [0, 2, 100])
def test_attention_matches_masked_sdpa(K):
    case = make_case(1, K=K)
    _, sel = dec.decode_select(case["scores"], case["lens"], case["block"], K)
    o, lse = run_oracle(case, sel)
    keep = keep_from_blocks(case, sel)
    o_ref, lse_ref = sdpa_masked(case, keep)
    np.testing.assert_allclose(o, o_ref, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse, lse_ref, rtol=1e-12, atol=1e-12)


def test_all_selected_is_dense_attention_over_the_cache():
    case = make_case(2, K=1000)
    _, sel = dec.decode_select(case["scores"], case["lens"], case["block"], 1000)
    o, _ = run_oracle(case, sel)
    q, kc, vc = case["q"], case["kc"], case["vc"]
    for b, n in enumerate(case["lens"]):
        for h in range(q.shape[1]):
            hk = h // case["G"]
            want = torch.nn.functional.scaled_dot_product_attention(
                q[b, h][None, None, None], kc[b, hk, :n][None, None], vc[b, hk, :n][None, None])
            np.testing.assert_allclose(o[b, h], want[0, 0, 0].numpy(), rtol=1e-12, atol=1e-12)


def test_k0_attends_the_current_block_only():
    case = make_case(3, K=0)
    _, sel = dec.decode_select(case["scores"], case["lens"], case["block"], 0)
    o, lse = run_oracle(case, sel)
    blk = case["block"]
    for b, n in enumerate(case["lens"]):
        c0 = ((n - 1) // blk) * blk
        for h in range(case["q"].shape[1]):
            hk = h // case["G"]
            want = torch.nn.functional.scaled_dot_product_attention(
                case["q"][b, h][None, None, None], case["kc"][b, hk, c0:n][None, None],
                case["vc"][b, hk, c0:n][None, None])
            np.testing.assert_allclose(o[b, h], want[0, 0, 0].numpy(), rtol=1e-12, atol=1e-12)


def test_zero_query_gives_uniform_weights():
    case = make_case(4, K=2)
    case["q"] = torch.zeros_like(case["q"])
    _, sel = dec.decode_select(case["scores"], case["lens"], case["block"], 2)
    o, lse = run_oracle(case, sel)
    keep = keep_from_blocks(case, sel)
    for b in range(o.shape[0]):
        for h in range(o.shape[1]):
            hk = h // case["G"]
            m = keep[b, hk]
            np.testing.assert_allclose(o[b, h], case["vc"][b, hk][torch.from_numpy(m)].mean(0).numpy(),
                                       rtol=1e-12, atol=1e-12)
            assert abs(lse[b, h] - math.log(m.sum())) < 1e-12


def test_planted_mistakes_are_caught(monkeypatch):
    """A current block that stops one token short, or a selection that drops
    its smallest member, must fail the SDPA pin."""
    case = make_case(5, K=2)
    _, sel = dec.decode_select(case["scores"], case["lens"], case["block"], 2)
    keep = keep_from_blocks(case, sel)
    o_ref, _ = sdpa_masked(case, keep)

    real = dec.attended_positions

    def short(n, block, sel_row):
        return real(n, block, sel_row)[:-1] if n % block != 1 else real(n, block, sel_row)
    monkeypatch.setattr(dec, "attended_positions", short)
    o_bad, _ = run_oracle(case, sel)
    assert np.max(np.abs(o_bad - o_ref)) > 1e-3
    monkeypatch.setattr(dec, "attended_positions", real)

    sel_bad = sel.copy()
    for b in range(sel.shape[0]):
        for h in range(sel.shape[1]):
            idx = np.nonzero(sel[b, h])[0]
            if len(idx):
                sel_bad[b, h, idx[0]] = False
    o_bad, _ = run_oracle(case, sel_bad)
    assert np.max(np.abs(o_bad - o_ref)) > 1e-3
