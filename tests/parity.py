"""Helpers for the GPU parity tests: run the HIP pipeline through the C ABI and
compare it with the float64 oracle on the same seeded inputs."""

from __future__ import annotations

import math
import sys

import numpy as np
import torch

import oracle
from gated_block_sparse_attn_amd import api, workloads

TOL = {"bf16": (2e-2, 2e-2), "fp32": (1e-5, 1e-5)}   # (rtol, atol)


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def problem_of(w: workloads.Workload, K: int, o_dtype: str = "bf16", gate_act: str = "softmax",
               gate_pos: str = "inner", gate_rank: str = "soft", seq_lens=None) -> api.Problem:
    lens = None if seq_lens is None else \
        torch.as_tensor(np.asarray(seq_lens), dtype=torch.int32).to("cuda:0")
    return api.Problem(w.batch, w.n_q_heads, w.n_kv_heads, w.seq_len, w.head_dim, w.block,
                       K, w.dtype, 0.0, o_dtype if w.dtype == "bf16" else "fp32", gate_act,
                       gate_pos, gate_rank, w.score_heads, lens)


def run_gpu(p: api.Problem, inp: dict, cap=None, poison=True, status=None):
    """threshold -> forward -> backward on cuda:0; returns host tensors."""
    dev = torch.device("cuda:0")
    q = inp["q"].to(dev)
    k = inp["k"].to(dev)
    v = inp["v"].to(dev)
    do = inp["do"].to(dev)
    scores = inp["scores"].to(dev)
    lg, tau, sel_idx, sel_cnt = api.gate_threshold(p, scores, sel_cap=cap, status=status)
    o = torch.empty(q.shape, dtype=p.torch_o_dtype, device=dev)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
    outs = {}
    if poison:   # NaN-prefill: every element must be written
        o.fill_(float("nan"))
        lse.fill_(float("nan"))
        outs = dict(dq=torch.full_like(q, float("nan")), dk=torch.full_like(k, float("nan")),
                    dv=torch.full_like(v, float("nan")),
                    dlog_gate=torch.full_like(lg, float("nan")),
                    dscores=torch.full_like(lg, float("nan")))
    api.gated_attn_fwd(p, q, k, v, lg, sel_idx, sel_cnt, o=o, lse=lse)
    dq, dk, dv, dlg, dsc = api.gated_attn_bwd(p, q, k, v, o, do, lse, lg, sel_idx, sel_cnt,
                                              outputs=outs)
    torch.cuda.synchronize()
    res = dict(log_gate=lg, tau=tau, sel_idx=sel_idx, sel_cnt=sel_cnt, o=o, lse=lse, dq=dq,
               dk=dk, dv=dv, dlog_gate=dlg, dscores=dsc)
    return {n: t.cpu() for n, t in res.items()}


def f32(t: torch.Tensor) -> np.ndarray:
    return t.float().numpy()


def check_selection(gpu, scores_np, K, act="softmax", seq_lens=None, block=None):
    """Selected sets, counts and thresholds must match the oracle exactly."""
    lg, tau, sel = oracle.gate_threshold(scores_np, K, act=act, seq_lens=seq_lens, block=block)
    cnt = sel.sum(-1)
    assert np.array_equal(gpu["sel_cnt"].numpy(), cnt), "selection counts differ"
    assert np.array_equal(gpu["tau"].numpy(), tau), "thresholds differ"
    idx = gpu["sel_idx"].numpy()
    cap = idx.shape[-1]
    B, H, C, _ = sel.shape
    for b in range(B):
        for h in range(H):
            for i in range(C):
                want = np.nonzero(sel[b, h, i])[0]
                c = min(len(want), cap)
                assert np.array_equal(idx[b, h, i, :c], want[:c]), (b, h, i)
                assert np.all(idx[b, h, i, c:] == -1)
    # log gates: fp32 GPU vs fp64 oracle; -inf / 0 pattern exact
    g = gpu["log_gate"].numpy()
    fin = np.isfinite(lg)
    assert np.array_equal(np.isfinite(g), fin)
    np.testing.assert_allclose(g[fin], lg[fin], rtol=1e-5, atol=1e-5)
    return lg, tau, sel


def compare(name, got, ref, dtype, mask=None):
    """Elementwise |got - ref| <= atol + rtol |ref|; also bounds the error
    relative to the tensor's largest magnitude, so tiny-valued tensors are not
    passed vacuously by atol."""
    rtol, atol = TOL[dtype]
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    if mask is not None:
        got = got[mask]
        ref = ref[mask]
    assert got.shape == ref.shape
    assert np.all(np.isfinite(got)), f"{name}: non-finite values (unwritten or overflow)"
    err = np.abs(got - ref)
    scale = float(np.max(np.abs(ref))) if ref.size else 0.0
    rel_to_max = float(np.max(err)) / scale if scale > 0 else float(np.max(err, initial=0.0))
    log(f"  {name:10s} max|err| {np.max(err, initial=0):.3e}  max|ref| {scale:.3e}  "
        f"err/max {rel_to_max:.3e}")
    bad = err > atol + rtol * np.abs(ref)
    assert not bad.any(), (f"{name}: {int(bad.sum())} of {bad.size} elements out of tolerance; "
                           f"worst err {np.max(err):.3e}")
    assert rel_to_max <= rtol, f"{name}: max error {rel_to_max:.3e} of the tensor's max magnitude"


def full_parity(w, K, inp=None, cap=None, o_dtype="bf16", gate_act="softmax", gate_pos="inner",
                gate_rank="soft", seq_lens=None):
    """Whole-tensor parity of every output (sizes the oracle finishes quickly).
    ``seq_lens``: valid tokens per sequence (variable-length batch, padded)."""
    p = problem_of(w, K, o_dtype, gate_act, gate_pos, gate_rank, seq_lens)
    inp = inp or workloads.generate(w)
    gpu = run_gpu(p, inp, cap=cap)
    scores = inp["scores"].numpy()
    lens = None if seq_lens is None else np.asarray(seq_lens)
    lg, tau, sel = check_selection(gpu, scores, K, act=gate_act, seq_lens=lens, block=w.block)
    q, k, v, do = (f32(inp[n]) for n in ("q", "k", "v", "do"))
    if gate_rank == "hard_ste":
        # unit gates on the selected blocks; every historical block gets dg
        zero = np.where(np.isfinite(lg), 0.0, lg)
        o, lse = oracle.forward(q, k, v, zero, sel, w.block, seq_lens=lens)
        dq, dk, dv, _ = oracle.backward(q, k, v, do, zero, sel, w.block, seq_lens=lens)
        dlg = oracle.sas_oracle.ste_gate_grad(q, k, v, do, lg, sel, w.block, seq_lens=lens)
        dsc = oracle.sas_oracle.dscores_from_dg(dlg, lg)
    else:
        o, lse = oracle.forward(q, k, v, lg, sel, w.block, gate_pos=gate_pos, seq_lens=lens)
        dq, dk, dv, dlg = oracle.backward(q, k, v, do, lg, sel, w.block, gate_pos=gate_pos,
                                          seq_lens=lens)
        dsc = oracle.dscores(dlg, lg, sel, act=gate_act)
    dt = w.dtype
    compare("o", f32(gpu["o"]), o, dt)
    compare("lse", gpu["lse"].numpy(), lse, dt)
    compare("dq", f32(gpu["dq"]), dq, dt)
    compare("dk", f32(gpu["dk"]), dk, dt)
    compare("dv", f32(gpu["dv"]), dv, dt)
    compare("dlog_gate", gpu["dlog_gate"].numpy(), dlg, dt)
    compare("dscores", gpu["dscores"].numpy(), dsc, dt)
    # exact zero pattern of the block log-gate gradient (hard gates: only the
    # diagonal and the upper triangle)
    c = sel.shape[-1]
    hist = np.broadcast_to(np.tril(np.ones((c, c), bool), -1), sel.shape)
    zero_at = ~hist if gate_rank == "hard_ste" else ~sel
    if lens is not None:   # rows without a query hold no gradient
        for b in range(sel.shape[0]):
            zero_at[b, :, oracle.sas_oracle.n_blocks_of(lens[b], w.block):] = True
    assert np.all(gpu["dlog_gate"].numpy()[zero_at] == 0.0)
    return gpu


def sampled_parity(w, K, n_units=12, n_kv_blocks=6, inp=None, seed=7):
    """Full-size run; oracle on sampled query blocks and key blocks."""
    p = problem_of(w, K)
    inp = inp or workloads.generate(w)
    log(f"[{w.name} K={K}] running GPU pipeline")
    gpu = run_gpu(p, inp)
    scores = inp["scores"].numpy()
    log(f"[{w.name} K={K}] checking selection")
    lg, tau, sel = check_selection(gpu, scores, K)
    units = workloads.sample_units(w, n_units, seed=seed)
    q, k, v, do = (f32(inp[n]) for n in ("q", "k", "v", "do"))
    log(f"[{w.name} K={K}] oracle on {len(units)} query blocks")
    o, lse = oracle.forward(q, k, v, lg, sel, w.block, query_blocks=units)
    dq, _, _, dlg = oracle.backward(q, k, v, do, lg, sel, w.block, query_blocks=units)
    G = w.group
    blk = w.block
    dt = w.dtype
    rows_o, rows_g = [], []
    for (b, hk, i) in units:
        for hh in range(hk * G, (hk + 1) * G):
            rows_o.append((b, hh, slice(i * blk, (i + 1) * blk)))
        rows_g.append((b, hk, i))
    pick = lambda a, rs: np.concatenate([a[r].reshape(-1) for r in rs])   # noqa: E731
    compare("o", pick(f32(gpu["o"]), rows_o), pick(o, rows_o), dt)
    compare("lse", pick(gpu["lse"].numpy(), rows_o), pick(lse, rows_o), dt)
    compare("dq", pick(f32(gpu["dq"]), rows_o), pick(dq, rows_o), dt)
    gdlg = gpu["dlog_gate"].numpy()
    compare("dlog_gate", pick(gdlg, rows_g), pick(dlg, rows_g), dt)
    for (b, hk, i) in rows_g:
        assert np.all(gdlg[b, hk, i][~sel[b, hk, i]] == 0.0)
    # dscores rows from the exact dLogG rows
    dsc = oracle.dscores(dlg, lg, sel)
    compare("dscores", pick(gpu["dscores"].numpy(), rows_g), pick(dsc, rows_g), dt)
    # dK / dV of sampled key blocks (sum over every query block that attends them)
    kvu = workloads.sample_units(w, n_kv_blocks, seed=seed + 1)
    gk, gv = f32(gpu["dk"]), f32(gpu["dv"])
    for (b, hk, j) in kvu:
        log(f"[{w.name} K={K}] oracle dK/dV block {(b, hk, j)}")
        dkj, dvj = oracle.backward_kv_block(q, k, v, do, lg, sel, blk, b, hk, j)
        compare(f"dk{j}", gk[b, hk, j * blk:(j + 1) * blk], dkj, dt)
        compare(f"dv{j}", gv[b, hk, j * blk:(j + 1) * blk], dvj, dt)
    return gpu


# --------------------------------------------------------------------------
# packed variable-length batches (cu_seqlens layout)
# --------------------------------------------------------------------------

def pack(x: torch.Tensor, lens) -> torch.Tensor:
    """[B, H, N, D] -> [T, H, D]: the first lens[b] rows of each sequence,
    sequence after sequence."""
    return torch.cat([x[b, :, :n].transpose(0, 1) for b, n in enumerate(lens)], dim=0).contiguous()


def unpack(x: np.ndarray, lens, n_pad: int) -> np.ndarray:
    """[T, H, D] -> [B, H, N, D] (rows past each length are 0)."""
    t, h, d = x.shape
    out = np.zeros((len(lens), h, n_pad, d), dtype=x.dtype)
    off = 0
    for b, n in enumerate(lens):
        out[b, :, :n] = np.transpose(x[off:off + n], (1, 0, 2))
        off += n
    return out


def unpack_stat(x: np.ndarray, lens, n_pad: int) -> np.ndarray:
    """[H, T] -> [B, H, N]."""
    h, t = x.shape
    out = np.zeros((len(lens), h, n_pad), dtype=x.dtype)
    off = 0
    for b, n in enumerate(lens):
        out[b, :, :n] = x[:, off:off + n]
        off += n
    return out


def run_gpu_packed(w, K, inp, lens, cap, gate_act="softmax", gate_pos="inner", gate_rank="soft",
                   o_dtype="bf16"):
    """threshold -> forward -> backward of the packed batch on cuda:0 (NaN-prefilled outputs);
    returns host tensors in the packed layout."""
    dev = torch.device("cuda:0")
    lens = [int(n) for n in lens]
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32, device=dev)
    t = int(sum(lens))
    p = api.Problem(w.batch, w.n_q_heads, w.n_kv_heads, w.seq_len, w.head_dim, w.block, K,
                    w.dtype, 0.0, o_dtype if w.dtype == "bf16" else "fp32", gate_act, gate_pos,
                    gate_rank, w.score_heads, None, cu, t)
    q, k, v, do = (pack(inp[n], lens).to(dev) for n in ("q", "k", "v", "do"))
    scores = inp["scores"].to(dev)
    lg, tau, sel_idx, sel_cnt = api.gate_threshold(p, scores, sel_cap=cap)
    o = torch.full(q.shape, float("nan"), dtype=p.torch_o_dtype, device=dev)
    lse = torch.full((w.n_q_heads, t), float("nan"), dtype=torch.float32, device=dev)
    api.gated_attn_fwd(p, q, k, v, lg, sel_idx, sel_cnt, o=o, lse=lse)
    outs = dict(dq=torch.full_like(q, float("nan")), dk=torch.full_like(k, float("nan")),
                dv=torch.full_like(v, float("nan")), dlog_gate=torch.full_like(lg, float("nan")),
                dscores=torch.full_like(lg, float("nan")))
    dq, dk, dv, dlg, dsc = api.gated_attn_bwd(p, q, k, v, o, do, lse, lg, sel_idx, sel_cnt,
                                              outputs=outs)
    torch.cuda.synchronize()
    res = dict(log_gate=lg, tau=tau, sel_idx=sel_idx, sel_cnt=sel_cnt, o=o, lse=lse, dq=dq,
               dk=dk, dv=dv, dlog_gate=dlg, dscores=dsc)
    return {n: x.cpu() for n, x in res.items()}


def packed_parity(w, K, lens, cap=None, gate_act="softmax", gate_pos="inner", gate_rank="soft"):
    """Packed batch against the oracle run on the padded equivalent (seq_lens):
    every output row of the packed tensors is compared (each packed row is a
    valid row of its sequence)."""
    inp = workloads.generate(w)
    gpu = run_gpu_packed(w, K, inp, lens, cap, gate_act, gate_pos, gate_rank)
    lens_np = np.asarray(lens)
    scores = inp["scores"].numpy()
    lg, tau, sel = check_selection(gpu, scores, K, act=gate_act, seq_lens=lens_np, block=w.block)
    q, k, v, do = (f32(inp[n]) for n in ("q", "k", "v", "do"))
    if gate_rank == "hard_ste":
        zero = np.where(np.isfinite(lg), 0.0, lg)
        o, lse = oracle.forward(q, k, v, zero, sel, w.block, seq_lens=lens_np)
        dq, dk, dv, _ = oracle.backward(q, k, v, do, zero, sel, w.block, seq_lens=lens_np)
        dlg = oracle.sas_oracle.ste_gate_grad(q, k, v, do, lg, sel, w.block, seq_lens=lens_np)
        dsc = oracle.sas_oracle.dscores_from_dg(dlg, lg)
    else:
        o, lse = oracle.forward(q, k, v, lg, sel, w.block, gate_pos=gate_pos, seq_lens=lens_np)
        dq, dk, dv, dlg = oracle.backward(q, k, v, do, lg, sel, w.block, gate_pos=gate_pos,
                                          seq_lens=lens_np)
        dsc = oracle.dscores(dlg, lg, sel, act=gate_act)
    n_pad = w.seq_len
    valid = np.zeros((w.batch, 1, n_pad, 1), dtype=bool)
    for b, n in enumerate(lens):
        valid[b, :, :n] = True
    vq = np.broadcast_to(valid, (w.batch, w.n_q_heads, n_pad, w.head_dim))
    vk = np.broadcast_to(valid, (w.batch, w.n_kv_heads, n_pad, w.head_dim))
    vs = np.broadcast_to(valid[..., 0], (w.batch, w.n_q_heads, n_pad))
    dt = w.dtype
    compare("o", unpack(f32(gpu["o"]), lens, n_pad), o, dt, mask=vq)
    compare("lse", unpack_stat(gpu["lse"].numpy(), lens, n_pad), lse, dt, mask=vs)
    compare("dq", unpack(f32(gpu["dq"]), lens, n_pad), dq, dt, mask=vq)
    compare("dk", unpack(f32(gpu["dk"]), lens, n_pad), dk, dt, mask=vk)
    compare("dv", unpack(f32(gpu["dv"]), lens, n_pad), dv, dt, mask=vk)
    compare("dlog_gate", gpu["dlog_gate"].numpy(), dlg, dt)
    compare("dscores", gpu["dscores"].numpy(), dsc, dt)
    return gpu
