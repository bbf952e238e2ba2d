"""Torch-facing binding of libsas: shape/dtype checks and pointer marshalling.

Every computation happens in the HIP library; this module only checks that
tensors are contiguous device tensors of the expected shapes, allocates
outputs with torch, and passes raw pointers plus torch's current HIP stream
through the C ABI (include/sas.h).  Names follow the C entry points.
"""

from __future__ import annotations

import dataclasses
import math
from typing import Optional

import torch

from . import _native
from ._native import SasError, SasProblem, check, lib

__all__ = ["Problem", "SasError", "gate_threshold", "gated_attn_fwd", "gated_attn_bwd",
           "gated_attn_bwd_dq", "gated_attn_bwd_dkdv", "bwd_workspace_size", "abi_version",
           "SASAttention", "sas_attention", "DecodeProblem", "decode_select",
           "decode_workspace_size", "decode_attn", "decode_attn_noalloc"]


@dataclasses.dataclass(frozen=True)
class Problem:
    """Sizes of one gated block-sparse attention problem (mirrors sas_problem)."""
    batch: int
    n_q_heads: int
    n_kv_heads: int
    seq_len: int
    head_dim: int
    block_size: int
    budget_k: int
    dtype: str = "bf16"        # "bf16" or "fp32": q, k, v, dO and the gradients
    sm_scale: float = 0.0      # <= 0: 1/sqrt(head_dim)
    o_dtype: str = "bf16"      # dtype of the forward output o (fp32 problems:
                               # always "fp32")
    gate_act: str = "softmax"  # "softmax" | "sigmoid" | "raw"
    gate_pos: str = "inner"    # "inner" (log g in the logits) | "outer" (g scales V)
    gate_rank: str = "soft"    # "soft" | "hard_ste" (hard Top-K gates, straight-through)
    score_heads: str = "group" # "group": gates per kv group; "head": per query head
    # Variable-length batches: optional int32 device tensor [batch] of valid tokens per
    # sequence (padded layout; None: every sequence holds seq_len tokens).
    seq_lens: Optional[torch.Tensor] = dataclasses.field(default=None, compare=False)
    # Packed variable-length batches: optional int32 device tensor [batch + 1] of
    # token offsets (q / o / dO / dq [T, Hq, D], k / v / dk / dv [T, Hkv, D],
    # lse [Hq, T], T = total_tokens; seq_len = the padded extent of the longest
    # sequence).  Exclusive with seq_lens.
    cu_seqlens: Optional[torch.Tensor] = dataclasses.field(default=None, compare=False)
    total_tokens: int = 0

    def __post_init__(self):
        if self.dtype == "fp32" and self.o_dtype != "fp32":
            object.__setattr__(self, "o_dtype", "fp32")

    @property
    def n_blocks(self) -> int:
        return self.seq_len // self.block_size

    @property
    def torch_dtype(self):
        return torch.bfloat16 if self.dtype == "bf16" else torch.float32

    @property
    def torch_o_dtype(self):
        return torch.bfloat16 if self.o_dtype == "bf16" else torch.float32

    def c(self) -> SasProblem:
        if self.seq_lens is not None:
            _expect(self.seq_lens, "seq_lens", (self.batch,), torch.int32)
        if self.cu_seqlens is not None:
            _expect(self.cu_seqlens, "cu_seqlens", (self.batch + 1,), torch.int32)
        return SasProblem(self.batch, self.n_q_heads, self.n_kv_heads, self.seq_len,
                          self.head_dim, self.block_size, self.budget_k,
                          _native.SAS_BF16 if self.dtype == "bf16" else _native.SAS_FP32,
                          _native.SAS_BF16 if self.o_dtype == "bf16" else _native.SAS_FP32,
                          float(self.sm_scale), _native.GATE_ACTS[self.gate_act],
                          _native.GATE_POS[self.gate_pos], _native.GATE_RANK[self.gate_rank],
                          self.n_score_heads, _ptr(self.seq_lens), _ptr(self.cu_seqlens),
                          int(self.total_tokens))

    def default_cap(self) -> int:
        return max(1, min(self.budget_k, self.n_blocks - 1))

    @property
    def n_score_heads(self) -> int:
        return self.n_q_heads if self.score_heads == "head" else self.n_kv_heads

    @staticmethod
    def from_tensors(q: torch.Tensor, k: torch.Tensor, block_size: int, budget_k: int,
                     sm_scale: float = 0.0, o_dtype: str = "bf16") -> "Problem":
        b, hq, n, d = q.shape
        dt = "bf16" if q.dtype == torch.bfloat16 else "fp32"
        return Problem(b, hq, k.shape[1], n, d, block_size, budget_k, dt, sm_scale,
                       "fp32" if dt == "fp32" else o_dtype)


def abi_version() -> int:
    return lib().sas_abi_version()


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _expect(t: torch.Tensor, name: str, shape, dtype):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor (got {t.device})")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _shapes(p: Problem, cap: int):
    c = p.n_blocks
    hs = p.n_score_heads
    if p.cu_seqlens is not None:   # packed batch
        t = p.total_tokens
        return dict(q=(t, p.n_q_heads, p.head_dim), kv=(t, p.n_kv_heads, p.head_dim),
                    lse=(p.n_q_heads, t), table=(p.batch, hs, c, c), row=(p.batch, hs, c),
                    sel=(p.batch, hs, c, cap))
    return dict(q=(p.batch, p.n_q_heads, p.seq_len, p.head_dim),
                kv=(p.batch, p.n_kv_heads, p.seq_len, p.head_dim),
                lse=(p.batch, p.n_q_heads, p.seq_len),
                table=(p.batch, hs, c, c),
                row=(p.batch, hs, c),
                sel=(p.batch, hs, c, cap))


def gate_threshold(p: Problem, scores: torch.Tensor, sel_cap: Optional[int] = None,
                   status: Optional[torch.Tensor] = None, outputs=None, stream=None):
    """sas_gate_threshold: returns (log_gate, tau, sel_idx, sel_cnt).

    ``outputs``: optional preallocated (log_gate, tau, sel_idx, sel_cnt)."""
    cap = p.default_cap() if sel_cap is None else sel_cap
    sh = _shapes(p, cap)
    _expect(scores, "scores", sh["table"], torch.float32)
    dev = scores.device
    if outputs is None:
        log_gate = torch.empty(sh["table"], dtype=torch.float32, device=dev)
        tau = torch.empty(sh["row"], dtype=torch.float32, device=dev)
        sel_idx = torch.empty(sh["sel"], dtype=torch.int32, device=dev)
        sel_cnt = torch.empty(sh["row"], dtype=torch.int32, device=dev)
    else:
        log_gate, tau, sel_idx, sel_cnt = outputs
        _expect(log_gate, "log_gate", sh["table"], torch.float32)
        _expect(tau, "tau", sh["row"], torch.float32)
        _expect(sel_idx, "sel_idx", sh["sel"], torch.int32)
        _expect(sel_cnt, "sel_cnt", sh["row"], torch.int32)
    if status is not None:
        _expect(status, "status", (1,), torch.int32)
    pc = p.c()
    check(lib().sas_gate_threshold(ctypes_ref(pc), _ptr(scores), _ptr(log_gate), _ptr(tau),
                                   _ptr(sel_idx), _ptr(sel_cnt), cap, _ptr(status),
                                   _stream(stream)))
    return log_gate, tau, sel_idx, sel_cnt


def gated_attn_fwd(p: Problem, q, k, v, log_gate, sel_idx, sel_cnt, o=None, lse=None,
                   stream=None):
    """sas_gated_attn_fwd: returns (o, lse)."""
    cap = sel_idx.shape[-1]
    sh = _shapes(p, cap)
    dt = p.torch_dtype
    _expect(q, "q", sh["q"], dt)
    _expect(k, "k", sh["kv"], dt)
    _expect(v, "v", sh["kv"], dt)
    _expect(log_gate, "log_gate", sh["table"], torch.float32)
    _expect(sel_idx, "sel_idx", sh["sel"], torch.int32)
    _expect(sel_cnt, "sel_cnt", sh["row"], torch.int32)
    odt = p.torch_o_dtype
    if o is None:
        o = torch.empty(sh["q"], dtype=odt, device=q.device)
    if lse is None:
        lse = torch.empty(sh["lse"], dtype=torch.float32, device=q.device)
    _expect(o, "o", sh["q"], odt)
    _expect(lse, "lse", sh["lse"], torch.float32)
    pc = p.c()
    check(lib().sas_gated_attn_fwd(ctypes_ref(pc), _ptr(q), _ptr(k), _ptr(v), _ptr(log_gate),
                                   _ptr(sel_idx), _ptr(sel_cnt), cap, _ptr(o), _ptr(lse),
                                   _stream(stream)))
    return o, lse


def bwd_workspace_size(p: Problem, sel_cap: int) -> int:
    pc = p.c()
    n = lib().sas_gated_attn_bwd_workspace_size(ctypes_ref(pc), sel_cap)
    if n == 0:
        check(_native.SAS_E_INVALID)
    return int(n)


def gated_attn_bwd(p: Problem, q, k, v, o, do, lse, log_gate, sel_idx, sel_cnt,
                   want_dscores: bool = True, workspace: Optional[torch.Tensor] = None,
                   outputs: Optional[dict] = None, stream=None):
    """sas_gated_attn_bwd: returns (dq, dk, dv, dlog_gate, dscores or None)."""
    cap = sel_idx.shape[-1]
    sh = _shapes(p, cap)
    dt = p.torch_dtype
    for name, t, s, tdt in (("q", q, sh["q"], dt), ("k", k, sh["kv"], dt), ("v", v, sh["kv"], dt),
                            ("o", o, sh["q"], p.torch_o_dtype), ("do", do, sh["q"], dt),
                            ("lse", lse, sh["lse"], torch.float32),
                            ("log_gate", log_gate, sh["table"], torch.float32),
                            ("sel_idx", sel_idx, sh["sel"], torch.int32),
                            ("sel_cnt", sel_cnt, sh["row"], torch.int32)):
        _expect(t, name, s, tdt)
    out = outputs or {}
    dev = q.device
    dq = out.get("dq", None)
    if dq is None:
        dq = torch.empty(sh["q"], dtype=dt, device=dev)
    dk = out.get("dk", None)
    if dk is None:
        dk = torch.empty(sh["kv"], dtype=dt, device=dev)
    dv = out.get("dv", None)
    if dv is None:
        dv = torch.empty(sh["kv"], dtype=dt, device=dev)
    dlg = out.get("dlog_gate", None)
    if dlg is None:
        dlg = torch.empty(sh["table"], dtype=torch.float32, device=dev)
    dsc = out.get("dscores", None)
    if dsc is None and want_dscores:
        dsc = torch.empty(sh["table"], dtype=torch.float32, device=dev)
    need = bwd_workspace_size(p, cap)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    pc = p.c()
    check(lib().sas_gated_attn_bwd(ctypes_ref(pc), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(do),
                                   _ptr(lse), _ptr(log_gate), _ptr(sel_idx), _ptr(sel_cnt), cap,
                                   _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dlg),
                                   _ptr(dsc) if want_dscores else None,
                                   _ptr(workspace), workspace.numel(), _stream(stream)))
    return dq, dk, dv, dlg, (dsc if want_dscores else None)


def _check_bwd_inputs(p, q, k, v, do, lse, log_gate, sel_idx, sel_cnt, o=None):
    cap = sel_idx.shape[-1]
    sh = _shapes(p, cap)
    dt = p.torch_dtype
    items = [("q", q, sh["q"], dt), ("k", k, sh["kv"], dt), ("v", v, sh["kv"], dt),
             ("do", do, sh["q"], dt), ("lse", lse, sh["lse"], torch.float32),
             ("log_gate", log_gate, sh["table"], torch.float32),
             ("sel_idx", sel_idx, sh["sel"], torch.int32),
             ("sel_cnt", sel_cnt, sh["row"], torch.int32)]
    if o is not None:
        items.append(("o", o, sh["q"], p.torch_o_dtype))
    for name, t, s, tdt in items:
        _expect(t, name, s, tdt)
    return cap, sh


def gated_attn_bwd_dq(p: Problem, q, k, v, o, do, lse, log_gate, sel_idx, sel_cnt, dq,
                      workspace, stream=None):
    """sas_gated_attn_bwd_dq (first backward stage) into preallocated outputs."""
    cap, sh = _check_bwd_inputs(p, q, k, v, do, lse, log_gate, sel_idx, sel_cnt, o)
    _expect(dq, "dq", sh["q"], p.torch_dtype)
    pc = p.c()
    check(lib().sas_gated_attn_bwd_dq(ctypes_ref(pc), _ptr(q), _ptr(k), _ptr(v), _ptr(o),
                                      _ptr(do), _ptr(lse), _ptr(log_gate), _ptr(sel_idx),
                                      _ptr(sel_cnt), cap, _ptr(dq), _ptr(workspace),
                                      workspace.numel(), _stream(stream)))


def gated_attn_bwd_dkdv(p: Problem, q, k, v, do, lse, log_gate, sel_idx, sel_cnt, dk, dv,
                        dlog_gate, dscores, workspace, stream=None):
    """sas_gated_attn_bwd_dkdv (second backward stage) into preallocated outputs."""
    cap, sh = _check_bwd_inputs(p, q, k, v, do, lse, log_gate, sel_idx, sel_cnt)
    _expect(dk, "dk", sh["kv"], p.torch_dtype)
    _expect(dv, "dv", sh["kv"], p.torch_dtype)
    _expect(dlog_gate, "dlog_gate", sh["table"], torch.float32)
    if dscores is not None:
        _expect(dscores, "dscores", sh["table"], torch.float32)
    pc = p.c()
    check(lib().sas_gated_attn_bwd_dkdv(ctypes_ref(pc), _ptr(q), _ptr(k), _ptr(v), _ptr(do),
                                        _ptr(lse), _ptr(log_gate), _ptr(sel_idx), _ptr(sel_cnt),
                                        cap, _ptr(dk), _ptr(dv), _ptr(dlog_gate), _ptr(dscores),
                                        _ptr(workspace), workspace.numel(), _stream(stream)))


def ctypes_ref(pc: SasProblem):
    import ctypes
    return ctypes.byref(pc)


class SASAttention(torch.autograd.Function):
    """Differentiable SAS attention: selector scores -> gates/Top-K -> Eq. 9.

    forward(q, k, v, scores, block_size, budget_k, sm_scale) -> o
    Gradients flow to q, k, v and to the selector scores (App. D.3); the
    Top-K selection itself is piecewise constant and passes no gradient.

    The selected lists hold min(budget_k, C - 1) entries per row.  Scores tied
    at a row's threshold can select more blocks than that (every tied block is
    kept); the library then flags SAS_E_CAPACITY on the device, and this
    function raises SasError (the check reads the flag back, one host
    synchronisation per call).
    """

    @staticmethod
    def forward(ctx, q, k, v, scores, block_size: int, budget_k: int, sm_scale: float = 0.0):
        p = Problem.from_tensors(q, k, block_size, budget_k, sm_scale)
        status = torch.zeros(1, dtype=torch.int32, device=q.device)
        log_gate, _, sel_idx, sel_cnt = gate_threshold(p, scores, status=status)
        code = int(status.item())
        if code != _native.SAS_OK:
            raise SasError(code, "sas_gate_threshold: more blocks tied at a row's threshold than "
                           f"the {sel_idx.shape[-1]} entries of its selected list (SAS_E_CAPACITY)")
        o, lse = gated_attn_fwd(p, q, k, v, log_gate, sel_idx, sel_cnt)
        ctx.save_for_backward(q, k, v, o, lse, log_gate, sel_idx, sel_cnt)
        ctx.problem = p
        ctx.mark_non_differentiable(lse)
        return o.to(q.dtype) if o.dtype != q.dtype else o

    @staticmethod
    def backward(ctx, do):
        q, k, v, o, lse, log_gate, sel_idx, sel_cnt = ctx.saved_tensors
        dq, dk, dv, _, dsc = gated_attn_bwd(ctx.problem, q, k, v, o, do.to(q.dtype).contiguous(),
                                            lse,
                                            log_gate, sel_idx, sel_cnt, want_dscores=True)
        return dq, dk, dv, dsc, None, None, None


def sas_attention(q, k, v, scores, block_size: int, budget_k: int, sm_scale: float = 0.0):
    """Functional form of SASAttention."""
    return SASAttention.apply(q, k, v, scores, block_size, budget_k, sm_scale)


def default_scale(head_dim: int, sm_scale: float = 0.0) -> float:
    return sm_scale if sm_scale > 0 else 1.0 / math.sqrt(head_dim)


# ---------------------------------------------------------------------------
# sparse decode
# ---------------------------------------------------------------------------

@dataclasses.dataclass(frozen=True)
class DecodeProblem:
    """Sizes of one batched sparse-decode step (mirrors sas_decode_problem)."""
    batch: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    block_size: int
    max_blocks: int
    pool_blocks: int
    budget_k: int
    dtype: str = "bf16"
    sm_scale: float = 0.0

    @property
    def torch_dtype(self):
        return torch.bfloat16 if self.dtype == "bf16" else torch.float32

    def c(self) -> _native.SasDecodeProblem:
        return _native.SasDecodeProblem(self.batch, self.n_q_heads, self.n_kv_heads,
                                        self.head_dim, self.block_size, self.max_blocks,
                                        self.pool_blocks, self.budget_k,
                                        _native.SAS_BF16 if self.dtype == "bf16"
                                        else _native.SAS_FP32, float(self.sm_scale))

    def default_cap(self) -> int:
        return max(1, min(self.budget_k, self.max_blocks - 1))


def decode_select(p: DecodeProblem, scores, seq_lens, sel_cap: Optional[int] = None,
                  status: Optional[torch.Tensor] = None, outputs=None, stream=None):
    """sas_decode_select: returns (tau, sel_idx, sel_cnt)."""
    cap = p.default_cap() if sel_cap is None else sel_cap
    _expect(scores, "scores", (p.batch, p.n_kv_heads, p.max_blocks), torch.float32)
    _expect(seq_lens, "seq_lens", (p.batch,), torch.int32)
    dev = scores.device
    if outputs is None:
        tau = torch.empty(p.batch, p.n_kv_heads, dtype=torch.float32, device=dev)
        sel_idx = torch.empty(p.batch, p.n_kv_heads, cap, dtype=torch.int32, device=dev)
        sel_cnt = torch.empty(p.batch, p.n_kv_heads, dtype=torch.int32, device=dev)
    else:
        tau, sel_idx, sel_cnt = outputs
        if tau is not None:
            _expect(tau, "tau", (p.batch, p.n_kv_heads), torch.float32)
        _expect(sel_idx, "sel_idx", (p.batch, p.n_kv_heads, cap), torch.int32)
        _expect(sel_cnt, "sel_cnt", (p.batch, p.n_kv_heads), torch.int32)
    if status is not None:
        _expect(status, "status", (1,), torch.int32)
    pc = p.c()
    check(lib().sas_decode_select(ctypes_ref(pc), _ptr(scores), _ptr(seq_lens), _ptr(tau),
                                  _ptr(sel_idx), _ptr(sel_cnt), cap, _ptr(status),
                                  _stream(stream)))
    return tau, sel_idx, sel_cnt


def decode_workspace_size(p: DecodeProblem, sel_cap: int) -> int:
    pc = p.c()
    n = lib().sas_decode_workspace_size(ctypes_ref(pc), sel_cap)
    if n == 0:
        check(_native.SAS_E_INVALID)
    return int(n)


def decode_attn(p: DecodeProblem, q, k_pool, v_pool, block_table, seq_lens, sel_idx, sel_cnt,
                o=None, lse=None, workspace=None, status: Optional[torch.Tensor] = None,
                stream=None):
    """sas_decode_attn: returns (o, lse)."""
    cap = sel_idx.shape[-1]
    dt = p.torch_dtype
    pool = (p.pool_blocks, p.n_kv_heads, p.block_size, p.head_dim)
    _expect(q, "q", (p.batch, p.n_q_heads, p.head_dim), dt)
    _expect(k_pool, "k_pool", pool, dt)
    _expect(v_pool, "v_pool", pool, dt)
    _expect(block_table, "block_table", (p.batch, p.max_blocks), torch.int32)
    _expect(seq_lens, "seq_lens", (p.batch,), torch.int32)
    _expect(sel_idx, "sel_idx", (p.batch, p.n_kv_heads, cap), torch.int32)
    _expect(sel_cnt, "sel_cnt", (p.batch, p.n_kv_heads), torch.int32)
    if o is None:
        o = torch.empty(p.batch, p.n_q_heads, p.head_dim, dtype=dt, device=q.device)
    if lse is None:
        lse = torch.empty(p.batch, p.n_q_heads, dtype=torch.float32, device=q.device)
    _expect(o, "o", (p.batch, p.n_q_heads, p.head_dim), dt)
    _expect(lse, "lse", (p.batch, p.n_q_heads), torch.float32)
    if workspace is None:
        workspace = torch.empty(decode_workspace_size(p, cap), dtype=torch.uint8, device=q.device)
    if status is not None:
        _expect(status, "status", (1,), torch.int32)
    pc = p.c()
    check(lib().sas_decode_attn(ctypes_ref(pc), _ptr(q), _ptr(k_pool), _ptr(v_pool),
                                _ptr(block_table), _ptr(seq_lens), _ptr(sel_idx), _ptr(sel_cnt),
                                cap, _ptr(o), _ptr(lse), _ptr(workspace), workspace.numel(),
                                _ptr(status), _stream(stream)))
    return o, lse


def decode_attn_noalloc(p: DecodeProblem, q, k_pool, v_pool, block_table, seq_lens, sel_idx,
                        sel_cnt, o, lse, status: Optional[torch.Tensor] = None, stream=None):
    """sas_decode_attn_noalloc: sas_decode_attn with the library's fixed
    per-device scratch instead of a workspace; o and lse are the caller's
    (nothing is allocated here or in the library)."""
    cap = sel_idx.shape[-1]
    dt = p.torch_dtype
    pool = (p.pool_blocks, p.n_kv_heads, p.block_size, p.head_dim)
    _expect(q, "q", (p.batch, p.n_q_heads, p.head_dim), dt)
    _expect(k_pool, "k_pool", pool, dt)
    _expect(v_pool, "v_pool", pool, dt)
    _expect(block_table, "block_table", (p.batch, p.max_blocks), torch.int32)
    _expect(seq_lens, "seq_lens", (p.batch,), torch.int32)
    _expect(sel_idx, "sel_idx", (p.batch, p.n_kv_heads, cap), torch.int32)
    _expect(sel_cnt, "sel_cnt", (p.batch, p.n_kv_heads), torch.int32)
    _expect(o, "o", (p.batch, p.n_q_heads, p.head_dim), dt)
    _expect(lse, "lse", (p.batch, p.n_q_heads), torch.float32)
    if status is not None:
        _expect(status, "status", (1,), torch.int32)
    pc = p.c()
    check(lib().sas_decode_attn_noalloc(ctypes_ref(pc), _ptr(q), _ptr(k_pool), _ptr(v_pool),
                                        _ptr(block_table), _ptr(seq_lens), _ptr(sel_idx),
                                        _ptr(sel_cnt), cap, _ptr(o), _ptr(lse), _ptr(status),
                                        _stream(stream)))
    return o, lse
