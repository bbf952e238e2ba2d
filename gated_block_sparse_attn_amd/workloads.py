"""Seeded synthetic workloads shared by the tests, the smoke check and the benchmark.

This module only draws random inputs.  It holds none of the attention
method's arithmetic, so both the HIP path and the CPU oracle can be fed from
it without sharing any computation.

Every tensor is drawn on the CPU with ``torch.Generator().manual_seed(seed)``
in a fixed order -- Q, K, V, dO, selector scores, then the per-config extra
(boosted columns or Gumbel noise) -- in float32 and then cast to the config
dtype, so the oracle (which upcasts the cast values) and the GPU see identical
bits.

The five named workloads take the shapes of the paper's evaluation models
(Qwen3-4B / 8B / 14B attention: 32 or 40 query heads over 8 KV heads,
head_dim 128, blocks of 64 tokens) and its budgets (1024- and 2048-token
budgets = 16 and 32 blocks, plus a sweep); the value distributions are the
ones stated beside each entry.
"""

from __future__ import annotations

import dataclasses
import math
from typing import Optional

import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    n_q_heads: int
    n_kv_heads: int
    seq_len: int
    head_dim: int
    block: int
    budgets: tuple
    dtype: str              # "fp32" or "bf16"
    seed: int
    qkv_std: float = 1.0    # Q, K, V ~ N(0, qkv_std^2)
    score_kind: str = "normal"   # "normal" | "normal_boost" | "gumbel"
    score_std: float = 1.0
    boost_frac: float = 0.0
    boost_value: float = 0.0
    score_heads: str = "group"   # "group": score rows per kv head; "head": per query head

    @property
    def n_blocks(self) -> int:
        return self.seq_len // self.block

    @property
    def n_score_heads(self) -> int:
        return self.n_q_heads if self.score_heads == "head" else self.n_kv_heads

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    def torch_dtype(self):
        return torch.float32 if self.dtype == "fp32" else torch.bfloat16


WORKLOADS = {
    # 1: tiny fp32 case, small enough for the brute-force oracle
    "tiny_fp32": Workload("tiny_fp32", 1, 1, 1, 256, 64, 16, (4,), "fp32", 1),
    # 2: Qwen3-4B attention shape, 8k context, 1024-token budget, scaled inputs
    "qwen3_4b_8k": Workload("qwen3_4b_8k", 1, 32, 8, 8192, 128, 64, (16,), "bf16", 2,
                            qkv_std=1.0 / math.sqrt(128.0), score_std=2.0),
    # 3: Qwen3-8B attention shape, 32k context, K = 16, peaked ranking
    #    (5% of context-block columns boosted by +4)
    "qwen3_8b_32k": Workload("qwen3_8b_32k", 1, 32, 8, 32768, 128, 64, (16,), "bf16", 3,
                             score_kind="normal_boost", score_std=2.0,
                             boost_frac=0.05, boost_value=4.0),
    # 4: Qwen3-14B attention shape (GQA 5), batch 2, 16k context, budget sweep
    "qwen3_14b_16k": Workload("qwen3_14b_16k", 2, 40, 8, 16384, 128, 64, (8, 16, 32, 64),
                              "bf16", 4),
    # 5: long context, 128k, K = 32 (2048-token budget), Gumbel selector scores
    "qwen3_8b_128k": Workload("qwen3_8b_128k", 1, 32, 8, 131072, 128, 64, (32,), "bf16", 5,
                              score_kind="gumbel"),
}

# Order used by the tests and the benchmark; index 2 is the headline workload.
WORKLOAD_ORDER = ["tiny_fp32", "qwen3_4b_8k", "qwen3_8b_32k", "qwen3_14b_16k", "qwen3_8b_128k"]


def custom(batch, n_q_heads, n_kv_heads, seq_len, head_dim, block, budget, dtype="fp32",
           seed=0, qkv_std=1.0, score_std=1.0, score_kind="normal",
           score_heads="group") -> Workload:
    """An ad-hoc workload (used for small parity and edge-case tests)."""
    return Workload(f"custom_{seed}", batch, n_q_heads, n_kv_heads, seq_len, head_dim, block,
                    (budget,), dtype, seed, qkv_std=qkv_std, score_kind=score_kind,
                    score_std=score_std, score_heads=score_heads)


def generate(w: Workload, with_grad_out: bool = True, seed: Optional[int] = None):
    """Draw the inputs of workload ``w`` on the CPU.

    Returns a dict with q [B,Hq,N,D], k and v [B,Hkv,N,D], do (like q, if
    requested) in the workload dtype, and scores float32 [B,Hs,C,C] (Hs = Hkv,
    or Hq for per-head scores; the whole square table is drawn; entries on or
    above the diagonal are never read).
    """
    g = torch.Generator().manual_seed(w.seed if seed is None else seed)
    dt = w.torch_dtype()
    qshape = (w.batch, w.n_q_heads, w.seq_len, w.head_dim)
    kshape = (w.batch, w.n_kv_heads, w.seq_len, w.head_dim)
    c = w.n_blocks

    def normal(shape, std):
        x = torch.randn(shape, generator=g, dtype=torch.float32)
        if std != 1.0:
            x.mul_(std)
        return x.to(dt)

    out = {
        "q": normal(qshape, w.qkv_std),
        "k": normal(kshape, w.qkv_std),
        "v": normal(kshape, w.qkv_std),
    }
    # dO is always drawn, so the scores that follow do not depend on the flag
    do = normal(qshape, 1.0)
    if with_grad_out:
        out["do"] = do
    else:
        del do
    sshape = (w.batch, w.n_score_heads, c, c)
    if w.score_kind == "gumbel":
        u = torch.rand(sshape, generator=g, dtype=torch.float32)
        tiny = torch.finfo(torch.float32).tiny
        u.clamp_(min=tiny, max=1.0 - 2.0 ** -24)
        scores = -torch.log(-torch.log(u))
    else:
        scores = torch.randn(sshape, generator=g, dtype=torch.float32) * w.score_std
        if w.score_kind == "normal_boost":
            nb = int(math.ceil(w.boost_frac * c))
            for b in range(w.batch):
                for h in range(w.n_score_heads):
                    cols = torch.randperm(c, generator=g)[:nb]
                    scores[b, h][:, cols] += w.boost_value
    out["scores"] = scores.contiguous()
    return out


def sample_units(w: Workload, count: int, seed: int = 1234):
    """A seeded sample of (batch, kv head, block) units, always including the
    first and last block of the first and last (batch, kv head)."""
    g = torch.Generator().manual_seed(seed)
    c = w.n_blocks
    units = {(0, 0, 0), (0, 0, c - 1), (w.batch - 1, w.n_kv_heads - 1, c - 1)}
    while len(units) < count:
        b = int(torch.randint(w.batch, (1,), generator=g))
        h = int(torch.randint(w.n_kv_heads, (1,), generator=g))
        i = int(torch.randint(c, (1,), generator=g))
        units.add((b, h, i))
    return sorted(units)


# ---------------------------------------------------------------------------
# sparse decode workloads: one new token per sequence over a paged KV cache
# ---------------------------------------------------------------------------

@dataclasses.dataclass(frozen=True)
class DecodeWorkload:
    name: str
    batch: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    block: int
    seq_lens: tuple         # tokens in the cache per sequence (the last one is the query's)
    budget: int
    dtype: str
    seed: int
    pool_pages: int = 0     # 0: one page per logical block; else a shared pool of this size
    score_kind: str = "normal"   # "normal" | "normal_boost" | "gumbel"
    boost_frac: float = 0.05
    boost_value: float = 4.0

    @property
    def max_blocks(self) -> int:
        return (max(self.seq_lens) + self.block - 1) // self.block

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @property
    def pages(self) -> int:
        return self.pool_pages or self.batch * self.max_blocks

    def torch_dtype(self):
        return torch.float32 if self.dtype == "fp32" else torch.bfloat16


_LENS_64K = tuple(65536 - x for x in (0, 1, 17, 63, 64, 100, 501, 1000))

DECODE_WORKLOADS = {
    # Qwen3-4B attention shape (32 / 8 heads, D = 128), block 64, 2048-token
    # budget (K = 32); batch 8 of ~64k-token sequences (ragged lengths), the
    # decode setting of the paper's batched measurement; peaked scores
    "qwen3_4b_decode_b8_64k": DecodeWorkload("qwen3_4b_decode_b8_64k", 8, 32, 8, 128, 64,
                                             _LENS_64K, 32, "bf16", 21, pool_pages=4096,
                                             score_kind="normal_boost"),
    # the same model at batch 1 and 512k tokens (8192 blocks per row): the
    # long-context point where Top-K selection dominates the step
    "qwen3_4b_decode_b1_512k": DecodeWorkload("qwen3_4b_decode_b1_512k", 1, 32, 8, 128, 64,
                                              (524288,), 32, "bf16", 22, pool_pages=2048,
                                              score_kind="gumbel"),
}


def decode_custom(batch, n_q_heads, n_kv_heads, head_dim, block, seq_lens, budget,
                  dtype="bf16", seed=0, pool_pages=0, score_kind="normal") -> DecodeWorkload:
    return DecodeWorkload(f"decode_custom_{seed}", batch, n_q_heads, n_kv_heads, head_dim, block,
                          tuple(seq_lens), budget, dtype, seed, pool_pages=pool_pages,
                          score_kind=score_kind)


def generate_decode(w: DecodeWorkload):
    """Draw a decode problem on the CPU, in the fixed order q, k_pool, v_pool,
    page table, scores (then the boost columns).

    q [B,Hq,D] and the pools [P,Hkv,b,D] ~ N(0, 1) in the workload dtype; the
    page of logical block m of sequence s is a seeded random page (a
    permutation when every logical block has its own page, else drawn with
    replacement from the shared pool); scores fp32 [B,Hkv,max_blocks].
    """
    g = torch.Generator().manual_seed(w.seed)
    dt = w.torch_dtype()
    cmax = w.max_blocks
    P = w.pages

    def normal(shape):
        return torch.randn(shape, generator=g, dtype=torch.float32).to(dt)

    q = normal((w.batch, w.n_q_heads, w.head_dim))
    kp = normal((P, w.n_kv_heads, w.block, w.head_dim))
    vp = normal((P, w.n_kv_heads, w.block, w.head_dim))
    if w.pool_pages:
        bt = torch.randint(P, (w.batch, cmax), generator=g, dtype=torch.int64)
    else:
        bt = torch.randperm(P, generator=g).reshape(w.batch, cmax)
    sshape = (w.batch, w.n_kv_heads, cmax)
    if w.score_kind == "gumbel":
        u = torch.rand(sshape, generator=g, dtype=torch.float32)
        u.clamp_(min=torch.finfo(torch.float32).tiny, max=1.0 - 2.0 ** -24)
        scores = -torch.log(-torch.log(u))
    else:
        scores = torch.randn(sshape, generator=g, dtype=torch.float32)
        if w.score_kind == "normal_boost":
            nb = int(math.ceil(w.boost_frac * cmax))
            for b in range(w.batch):
                for h in range(w.n_kv_heads):
                    cols = torch.randperm(cmax, generator=g)[:nb]
                    scores[b, h, cols] += w.boost_value
    return {"q": q, "k_pool": kp, "v_pool": vp, "block_table": bt.to(torch.int32),
            "seq_lens": torch.tensor(w.seq_lens, dtype=torch.int32), "scores": scores.contiguous()}
