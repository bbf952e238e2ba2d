"""Helpers for the GPU parity tests: run the HIP pipeline through the C ABI and
compare it with the float64 oracle on the same seeded inputs.

Every device buffer the library writes (the gate outputs, o, lse, the
gradients and the backward workspace) is allocated with canary bands of
GUARD bytes before and after it; the bands must be intact after the run, so a
write outside any buffer fails the case.  Outputs are NaN-prefilled, so an
element the library never writes fails the comparison.
"""

from __future__ import annotations

import sys
import time

import numpy as np
import torch

import oracle
from gated_block_sparse_attn_amd import api, workloads

TOL = {"bf16": (2e-2, 2e-2), "fp32": (1e-5, 1e-5)}   # (rtol, atol)
GUARD = 4096          # canary bytes before and after every device buffer
CANARY = 0x5A         # canary byte (0x5A5A as bf16 and 0x5A5A5A5A as fp32 are finite)


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def f32(t: torch.Tensor) -> np.ndarray:
    return t.float().numpy()


# --------------------------------------------------------------------------
# guarded device buffers
# --------------------------------------------------------------------------

class Guard:
    """Device allocations with canary bands on both sides."""

    def __init__(self, dev):
        self.dev = dev
        self.items = []

    def tensor(self, name, shape, dtype, fill=None):
        esz = torch.empty((), dtype=dtype).element_size()
        n = int(np.prod(shape))
        g = GUARD // esz
        raw = torch.empty(n + 2 * g, dtype=dtype, device=self.dev)
        raw.view(torch.uint8).fill_(CANARY)
        t = raw[g:g + n].view(shape)
        if fill is not None:
            t.fill_(fill)
        self.items.append((name, raw, g * esz, n * esz))
        return t

    def workspace(self, nbytes):
        return self.tensor("workspace", (max(int(nbytes), 256),), torch.uint8)

    def check(self):
        for name, raw, g, nb in self.items:
            b = raw.view(torch.uint8)
            head_ok = bool(torch.all(b[:g] == CANARY))
            tail_ok = bool(torch.all(b[g + nb:] == CANARY))
            assert head_ok and tail_ok, f"{name}: bytes written outside the buffer " \
                                        f"({'before' if not head_ok else 'after'} it)"


# --------------------------------------------------------------------------
# running the HIP path
# --------------------------------------------------------------------------

def problem_of(w: workloads.Workload, K: int, o_dtype: str = "bf16", gate_act: str = "softmax",
               gate_pos: str = "inner", gate_rank: str = "soft", seq_lens=None,
               packed_lens=None) -> api.Problem:
    """The api.Problem of workload w at budget K.  ``seq_lens``: padded
    variable-length batch; ``packed_lens``: packed batch of these lengths."""
    lens = cu = None
    total = 0
    if seq_lens is not None:
        lens = torch.as_tensor(np.asarray(seq_lens), dtype=torch.int32).to("cuda:0")
    if packed_lens is not None:
        pl = [int(n) for n in packed_lens]
        cu = torch.tensor(np.concatenate([[0], np.cumsum(pl)]), dtype=torch.int32, device="cuda:0")
        total = int(sum(pl))
    return api.Problem(w.batch, w.n_q_heads, w.n_kv_heads, w.seq_len, w.head_dim, w.block,
                       K, w.dtype, 0.0, o_dtype if w.dtype == "bf16" else "fp32", gate_act,
                       gate_pos, gate_rank, w.score_heads, lens, cu, total)


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


def run_gpu(p: api.Problem, inp: dict, cap=None, poison=True, status=None, packed_lens=None,
            scores=None):
    """threshold -> forward -> backward on cuda:0 with every output and the
    workspace guarded (and NaN-prefilled when ``poison``); returns host
    tensors (packed layout for a packed batch).  ``scores`` replaces the
    workload's score table (same shape)."""
    dev = torch.device("cuda:0")
    if packed_lens is not None:
        q, k, v, do = (pack(inp[n], packed_lens).to(dev) for n in ("q", "k", "v", "do"))
    else:
        q, k, v, do = (inp[n].to(dev) for n in ("q", "k", "v", "do"))
    sc = (inp["scores"] if scores is None else scores).to(dev)
    cap = p.default_cap() if cap is None else cap
    sh = api._shapes(p, cap)
    gd = Guard(dev)
    nan = float("nan") if poison else None
    gate_out = (gd.tensor("log_gate", sh["table"], torch.float32, nan),
                gd.tensor("tau", sh["row"], torch.float32, nan),
                gd.tensor("sel_idx", sh["sel"], torch.int32, -7 if poison else None),
                gd.tensor("sel_cnt", sh["row"], torch.int32, -7 if poison else None))
    lg, tau, sel_idx, sel_cnt = api.gate_threshold(p, sc, sel_cap=cap, status=status,
                                                   outputs=gate_out)
    o = gd.tensor("o", sh["q"], p.torch_o_dtype, nan)
    lse = gd.tensor("lse", sh["lse"], torch.float32, nan)
    api.gated_attn_fwd(p, q, k, v, lg, sel_idx, sel_cnt, o=o, lse=lse)
    outs = dict(dq=gd.tensor("dq", sh["q"], p.torch_dtype, nan),
                dk=gd.tensor("dk", sh["kv"], p.torch_dtype, nan),
                dv=gd.tensor("dv", sh["kv"], p.torch_dtype, nan),
                dlog_gate=gd.tensor("dlog_gate", sh["table"], torch.float32, nan),
                dscores=gd.tensor("dscores", sh["table"], torch.float32, nan))
    ws = gd.workspace(api.bwd_workspace_size(p, cap))
    dq, dk, dv, dlg, dsc = api.gated_attn_bwd(p, q, k, v, o, do, lse, lg, sel_idx, sel_cnt,
                                              workspace=ws, outputs=outs)
    torch.cuda.synchronize()
    gd.check()
    res = dict(log_gate=lg, tau=tau, sel_idx=sel_idx, sel_cnt=sel_cnt, o=o, lse=lse, dq=dq,
               dk=dk, dv=dv, dlog_gate=dlg, dscores=dsc)
    return {n: t.cpu() for n, t in res.items()}


# --------------------------------------------------------------------------
# comparisons
# --------------------------------------------------------------------------

def check_selection(gpu, scores_np, K, act="softmax", seq_lens=None, block=None):
    """Selected sets, counts and thresholds must match the oracle exactly."""
    lg, tau, sel = oracle.gate_threshold(scores_np, K, act=act, seq_lens=seq_lens, block=block)
    cnt = sel.sum(-1)
    assert np.array_equal(gpu["sel_cnt"].numpy(), cnt), "selection counts differ"
    assert np.array_equal(gpu["tau"].numpy(), tau), "thresholds differ"
    idx = gpu["sel_idx"].numpy()
    cap = idx.shape[-1]
    # ascending lists: the row's first min(cnt, cap) selected blocks, then -1
    order = np.argsort(~sel, axis=-1, kind="stable")[..., :cap]   # selected blocks first, ascending
    if order.shape[-1] < cap:
        order = np.concatenate([order, np.full(order.shape[:-1] + (cap - order.shape[-1],), -1)], -1)
    take = np.arange(cap) < np.minimum(cnt, cap)[..., None]
    want = np.where(take, order, -1)
    assert np.array_equal(idx, want), "selected lists differ"
    # log gates: fp32 GPU vs fp64 oracle; -inf / 0 pattern exact
    g = gpu["log_gate"].numpy()
    fin = np.isfinite(lg)
    assert np.array_equal(np.isfinite(g), fin)
    np.testing.assert_allclose(g[fin], lg[fin], rtol=1e-5, atol=1e-5)
    return lg, tau, sel


def compare(name, got, ref, dtype, mask=None, scale=None):
    """Elementwise |got - ref| <= atol * scale + rtol |ref| (scale: 1, or a
    per-element magnitude bound such as a row's gate mass); also bounds the
    error relative to the tensor's largest magnitude, so tiny-valued tensors
    are not passed vacuously by atol."""
    rtol, atol = TOL[dtype]
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    sc = 1.0 if scale is None else np.broadcast_to(np.asarray(scale, np.float64), ref.shape)
    if mask is not None:
        got = got[mask]
        ref = ref[mask]
        if scale is not None:
            sc = sc[mask]
    assert got.shape == ref.shape
    assert np.all(np.isfinite(got)), f"{name}: non-finite values (unwritten or overflow)"
    err = np.abs(got - ref)
    big = float(np.max(np.abs(ref))) if ref.size else 0.0
    rel_to_max = float(np.max(err)) / big if big > 0 else float(np.max(err, initial=0.0))
    log(f"  {name:10s} max|err| {np.max(err, initial=0):.3e}  max|ref| {big:.3e}  "
        f"err/max {rel_to_max:.3e}")
    bad = err > atol * sc + rtol * np.abs(ref)
    assert not bad.any(), (f"{name}: {int(bad.sum())} of {bad.size} elements out of tolerance; "
                           f"worst err {np.max(err):.3e}")
    assert rel_to_max <= rtol, f"{name}: max error {rel_to_max:.3e} of the tensor's max magnitude"


# unit roundoff of bf16 (8-bit significand, round to nearest)
U_BF16 = 2.0 ** -8


def kv_scale(kmass, term_mass, dtype):
    """Per-element atol scale of dK / dV.  The key-major pass rounds P (for
    dV) and dS (for dK) to bf16 before its matrix products, so each element
    carries up to U_BF16 times the sum of the absolute values of its terms
    (the oracle's term mass); with many heads and rows attending a key, that
    exceeds the flat atol where the terms cancel.  The scale keeps twice that
    bound within atol * scale (and at least the gate-mass scale kmass)."""
    base = 1.0 if kmass is None else kmass
    if dtype != "bf16":
        return kmass
    return np.maximum(base, 2.0 * U_BF16 * term_mass / TOL["bf16"][1])


def _score_head_units(w, n, seed):
    """A seeded sample of (batch, score head, query block) units, always with
    the first and last block of the first and last (batch, score head)."""
    g = torch.Generator().manual_seed(seed)
    c = w.n_blocks
    hs = w.n_score_heads
    units = {(0, 0, 0), (0, 0, c - 1), (w.batch - 1, hs - 1, c - 1), (w.batch - 1, hs - 1, 1)}
    while len(units) < n:
        units.add((int(torch.randint(w.batch, (1,), generator=g)),
                   int(torch.randint(hs, (1,), generator=g)),
                   int(torch.randint(c, (1,), generator=g))))
    return sorted(units)


def column_lengths(w, sel):
    """[B, Hkv, C]: query blocks attending each key block (the diagonal one
    included), over the score heads of each kv head."""
    B, hs, c, _ = sel.shape
    per_head = sel.sum(axis=2) + 1                       # [B, Hs, C]
    ns = hs // w.n_kv_heads if hs >= w.n_kv_heads else 1
    return per_head.reshape(B, w.n_kv_heads, ns, c).sum(axis=2)


def longest_columns(w, sel, kv_heads="all", extra=0, seed=0):
    """For each (batch, kv head) -- or the listed ones -- its key block with
    the most attending query blocks (the column the key-major pass cuts into
    most chunks); plus ``extra`` seeded random key blocks."""
    L = column_lengths(w, sel)
    pairs = [(b, h) for b in range(w.batch) for h in range(w.n_kv_heads)] \
        if kv_heads == "all" else list(kv_heads)
    units = {(b, h, int(np.argmax(L[b, h]))) for (b, h) in pairs}
    g = torch.Generator().manual_seed(seed)
    while len(units) < len(pairs) + extra:
        units.add((int(torch.randint(w.batch, (1,), generator=g)),
                   int(torch.randint(w.n_kv_heads, (1,), generator=g)),
                   int(torch.randint(w.n_blocks, (1,), generator=g))))
    return sorted(units), L


def gate_mass(q, k, lg, sel, blk, lens, gate_pos, units=None):
    """Per query row, max(1, sum_k p_k g_k): the factor by which the outer
    gate position scales o and the row's gradients (the inner position's
    weights sum to 1).  From the oracle's forward with unit value rows;
    returned with o's shape (every head dim of a row holds its mass)."""
    if gate_pos != "outer":
        return None
    ones = np.ones(k.shape[:3] + (1,))
    m, _ = oracle.forward(q, k, ones, lg, sel, blk, gate_pos="outer", seq_lens=lens,
                          query_blocks=units)
    return np.maximum(m, 1.0)


def key_gate_mass(mass, lg, sel, n_kv_heads, blk):
    """Per key row, the magnitude its gradient terms carry at the outer gate
    position: dS = P (g dP - Delta) of a key in block m holds the block's
    gate g_{i,m} and the attending rows' Delta, which scales with their gate
    mass.  max(1, the largest such g or row mass over the query blocks that
    attend block m, its own block included); [B, Hkv, N, 1]."""
    if mass is None:
        return None
    B, Hq, N, _ = mass.shape
    _, Hs, C, _ = lg.shape
    rowm = mass[..., 0].reshape(B, Hq, C, blk).max(axis=-1)            # [B, Hq, C]
    rowm = rowm.reshape(B, Hs, Hq // Hs, C).max(axis=2)                 # per score head
    g = np.where(sel, np.exp(np.where(sel, lg, 0.0)), 0.0)              # selected gates
    att = sel | np.eye(C, dtype=bool)                                   # attending blocks
    val = np.where(att, np.maximum(rowm[..., :, None], g), 0.0)         # [B, Hs, C(i), C(m)]
    per_col = val.max(axis=2)                                           # [B, Hs, C(m)]
    if Hs > n_kv_heads:
        per_col = per_col.reshape(B, n_kv_heads, Hs // n_kv_heads, C).max(axis=2)
    return np.maximum(np.repeat(per_col, blk, axis=-1)[..., None], 1.0)


def parity(w, K, inp=None, cap=None, o_dtype="bf16", gate_act="softmax", gate_pos="inner",
           gate_rank="soft", seq_lens=None, packed=False, scores=None, units=None,
           kv_units=None, label=""):
    """One case: the GPU pipeline against the oracle.

    ``units`` None: whole-tensor parity of every output; else a list of
    (batch, score head, query block) units whose o / lse / dq rows and gate
    rows are compared, and ``kv_units`` (batch, kv head, key block) whose
    dK / dV rows are compared.  ``seq_lens`` with ``packed``: the same batch in
    the packed layout (cu_seqlens), compared row by row with the oracle on the
    padded equivalent.  Returns the GPU results (padded layout)."""
    t0 = time.time()
    inp = inp or workloads.generate(w)
    lens = None if seq_lens is None else np.asarray(seq_lens)
    p = problem_of(w, K, o_dtype, gate_act, gate_pos, gate_rank,
                   seq_lens=None if packed else seq_lens, packed_lens=seq_lens if packed else None)
    sc_np = (inp["scores"] if scores is None else scores).numpy()
    if cap is None:
        # room for every selected block: exact fp32 ties at a row's threshold
        # (scores shifted by a constant round distinct values together) select
        # more than K blocks, all of which the method attends
        _, _, sel0 = oracle.gate_threshold(sc_np, K, act=gate_act, seq_lens=lens, block=w.block)
        cap = max(p.default_cap(), int(sel0.sum(-1).max()))
    status = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    log(f"[{label or w.name} K={K}] GPU pipeline (sel_cap {cap})")
    raw = run_gpu(p, inp, cap=cap, packed_lens=seq_lens if packed else None, scores=scores,
                  status=status)
    assert int(status.item()) == 0, "the capacity flag is set although every selected block fits"
    gpu = dict(raw)
    n_pad = w.seq_len
    if packed:   # rows in the padded layout (0 on padding rows, which hold no query)
        for n in ("o", "dq", "dk", "dv"):
            gpu[n] = torch.from_numpy(unpack(f32(raw[n]), seq_lens, n_pad))
        gpu["lse"] = torch.from_numpy(unpack_stat(raw["lse"].numpy(), seq_lens, n_pad))
    lg, tau, sel = check_selection(gpu, sc_np, K, act=gate_act, seq_lens=lens, block=w.block)
    q, k, v, do = (f32(inp[n]) for n in ("q", "k", "v", "do"))
    blk = w.block
    hard = gate_rank == "hard_ste"
    glg = np.where(np.isfinite(lg), 0.0, lg) if hard else lg   # hard gates: unit on the selected
    log(f"[{label or w.name} K={K}] oracle ({'whole tensors' if units is None else f'{len(units)} query blocks'})")
    o, lse = oracle.forward(q, k, v, glg, sel, blk, gate_pos=gate_pos, seq_lens=lens,
                            query_blocks=units)
    dq, dk, dv, dlg, dkm, dvm = oracle.backward(q, k, v, do, glg, sel, blk, gate_pos=gate_pos,
                                                seq_lens=lens, query_blocks=units,
                                                term_mass=True)
    if hard:
        dlg = oracle.sas_oracle.ste_gate_grad(q, k, v, do, lg, sel, blk, seq_lens=lens,
                                              rows=units)
        dsc = oracle.sas_oracle.dscores_from_dg(dlg, lg)
    else:
        dsc = oracle.dscores(dlg, lg, sel, act=gate_act)
    mass = gate_mass(q, k, lg, sel, blk, lens, gate_pos, units)
    kmass = key_gate_mass(mass, lg, sel, w.n_kv_heads, blk)
    dt = w.dtype
    G = w.n_q_heads // w.n_score_heads
    # which rows to compare (a packed batch holds only its sequences' rows)
    valid = None
    if packed:
        valid = np.zeros((w.batch, 1, n_pad), bool)
        for b, n in enumerate(seq_lens):
            valid[b, :, :max(0, min(int(n), n_pad))] = True
    if units is None:
        gmask = None
        smask = None if valid is None else np.broadcast_to(valid, lse.shape)
    else:
        smask = np.zeros(lse.shape, bool)
        gmask = np.zeros(lg.shape[:3], bool)
        for (b, sh, i) in units:
            smask[b, sh * G:(sh + 1) * G, i * blk:(i + 1) * blk] = True
            gmask[b, sh, i] = True
        if valid is not None:
            smask &= valid
    qmask = None if smask is None else np.broadcast_to(smask[..., None], o.shape)
    compare("o", f32(gpu["o"]), o, dt, mask=qmask, scale=mass)
    compare("lse", gpu["lse"].numpy(), lse, dt, mask=smask)
    compare("dq", f32(gpu["dq"]), dq, dt, mask=qmask, scale=mass)
    gdlg = gpu["dlog_gate"].numpy()
    compare("dlog_gate", gdlg, dlg, dt, mask=gmask)
    compare("dscores", gpu["dscores"].numpy(), dsc, dt, mask=gmask)
    # exact zero pattern of the block log-gate gradient (hard gates: only the
    # diagonal and the upper triangle)
    c = w.n_blocks
    hist = np.broadcast_to(np.tril(np.ones((c, c), bool), -1), sel.shape)
    zero_at = (~hist if hard else ~sel).copy()
    if lens is not None:   # rows without a query hold no gradient
        for b in range(w.batch):
            zero_at[b, :, oracle.sas_oracle.n_blocks_of(lens[b], blk):] = True
    assert np.all(gdlg[zero_at] == 0.0), "dlog_gate: nonzero where no gradient flows"
    gk, gv = f32(gpu["dk"]), f32(gpu["dv"])
    if units is None:
        kmask = None if valid is None else np.broadcast_to(valid[..., None], dk.shape)
        compare("dk", gk, dk, dt, mask=kmask, scale=kv_scale(kmass, dkm, dt))
        compare("dv", gv, dv, dt, mask=kmask, scale=kv_scale(kmass, dvm, dt))
    else:
        for (b, hk, j) in kv_units or []:
            log(f"[{label or w.name} K={K}] oracle dK/dV of key block {(b, hk, j)}")
            dkj, dvj, dkmj, dvmj = oracle.backward_kv_block(q, k, v, do, glg, sel, blk, b, hk, j,
                                                            gate_pos=gate_pos, seq_lens=lens,
                                                            term_mass=True)
            rows = slice(j * blk, (j + 1) * blk)
            keep = np.ones((blk, 1), bool)
            if packed:   # rows past the sequence's end do not exist in the packed tensors
                keep[max(0, int(seq_lens[b]) - j * blk):] = False
            km = np.broadcast_to(keep, dkj.shape)
            ks = None if kmass is None else kmass[b, hk, rows]
            compare(f"dk{j}", gk[b, hk, rows], dkj, dt, mask=km, scale=kv_scale(ks, dkmj, dt))
            compare(f"dv{j}", gv[b, hk, rows], dvj, dt, mask=km, scale=kv_scale(ks, dvmj, dt))
    log(f"[{label or w.name} K={K}] ok ({time.time() - t0:.1f} s)")
    return gpu


def full_parity(w, K, inp=None, cap=None, o_dtype="bf16", gate_act="softmax", gate_pos="inner",
                gate_rank="soft", seq_lens=None):
    """Whole-tensor parity of every output (padded layout)."""
    return parity(w, K, inp=inp, cap=cap, o_dtype=o_dtype, gate_act=gate_act, gate_pos=gate_pos,
                  gate_rank=gate_rank, seq_lens=seq_lens)


def packed_parity(w, K, lens, cap=None, gate_act="softmax", gate_pos="inner", gate_rank="soft"):
    """Packed batch (cu_seqlens) against the oracle on the padded equivalent."""
    return parity(w, K, cap=cap, gate_act=gate_act, gate_pos=gate_pos, gate_rank=gate_rank,
                  seq_lens=lens, packed=True)


def sampled_parity(w, K, n_units=12, inp=None, seed=7, kv_heads="all", kv_extra=2,
                   **variant):
    """Full-size run; the oracle on sampled query blocks and on the longest
    key-block column of each listed (batch, kv head) plus a few random key
    blocks."""
    inp = inp or workloads.generate(w)
    units = _score_head_units(w, n_units, seed)
    # the key-block sample needs the selection: computed from the scores (the
    # same call check_selection makes), before the run
    lens = variant.get("seq_lens")
    sc = (inp["scores"] if variant.get("scores") is None else variant["scores"]).numpy()
    _, _, sel = oracle.gate_threshold(sc, K, act=variant.get("gate_act", "softmax"),
                                      seq_lens=None if lens is None else np.asarray(lens),
                                      block=w.block)
    kv_units, L = longest_columns(w, sel, kv_heads=kv_heads, extra=kv_extra, seed=seed + 1)
    log(f"[{w.name} K={K}] key blocks {kv_units} (attending blocks: "
        f"{[int(L[b, h, j]) for (b, h, j) in kv_units]})")
    return parity(w, K, inp=inp, units=units, kv_units=kv_units, **variant)
