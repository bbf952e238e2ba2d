"""GPU parity of the sparse-decode path (through the C ABI) against the float64
decode oracle.

Selected sets, counts and thresholds are compared exactly; o and lse within
rtol = atol = 2e-2 (bf16) or 1e-5 (fp32), and within that fraction of each
tensor's largest magnitude.  Cases: ragged batches (a single token, exactly
one block, one block plus a token, a full cache), K = 0, K >= history, GQA
1 / 4 / 5 / 32 / 40, head_dim 64 / 128, blocks of 16 / 32 / 64, fp32 and bf16, paged
caches with shuffled and with shared pages, exact ties, the capacity flag,
out-of-range lengths / pages / selections flagged from the host side (every
access stays in bounds), 8192-block rows (512k tokens), and bitwise
run-to-run determinism.
"""

import numpy as np
import pytest
import torch

import oracle.sas_decode_oracle as dec
from gated_block_sparse_attn_amd import api, workloads

from parity import compare, log

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.empty_cache()


def problem_of(w: workloads.DecodeWorkload, K=None) -> api.DecodeProblem:
    return api.DecodeProblem(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.block,
                             w.max_blocks, w.pages, w.budget if K is None else K, w.dtype)


def run_gpu(p, inp, cap=None, status=None):
    dev = torch.device("cuda:0")
    t = {k: v.to(dev) for k, v in inp.items()}
    tau, si, sc = api.decode_select(p, t["scores"], t["seq_lens"], sel_cap=cap, status=status)
    o = torch.full((p.batch, p.n_q_heads, p.head_dim), float("nan"), dtype=p.torch_dtype,
                   device=dev)
    lse = torch.full((p.batch, p.n_q_heads), float("nan"), dtype=torch.float32, device=dev)
    api.decode_attn(p, t["q"], t["k_pool"], t["v_pool"], t["block_table"], t["seq_lens"], si, sc,
                    o=o, lse=lse, status=status)
    torch.cuda.synchronize()
    return {k: v.cpu() for k, v in dict(tau=tau, sel_idx=si, sel_cnt=sc, o=o, lse=lse).items()}


def check_select(gpu, inp, block, K):
    tau, sel = dec.decode_select(inp["scores"].numpy(), inp["seq_lens"].numpy(), block, K)
    assert np.array_equal(gpu["sel_cnt"].numpy(), sel.sum(-1)), "selection counts differ"
    assert np.array_equal(gpu["tau"].numpy(), tau), "thresholds differ"
    idx = gpu["sel_idx"].numpy()
    cap = idx.shape[-1]
    for b in range(sel.shape[0]):
        for h in range(sel.shape[1]):
            want = np.nonzero(sel[b, h])[0]
            c = min(len(want), cap)
            assert np.array_equal(idx[b, h, :c], want[:c]), (b, h)
            assert np.all(idx[b, h, c:] == -1)
    return sel


def decode_parity(w, K=None, cap=None):
    K = w.budget if K is None else K
    p = problem_of(w, K)
    inp = workloads.generate_decode(w)
    log(f"decode {w.name} B={w.batch} G={w.group} D={w.head_dim} b={w.block} K={K} {w.dtype}")
    gpu = run_gpu(p, inp, cap=cap)
    sel = check_select(gpu, inp, w.block, K)
    f = lambda x: x.float().numpy()   # noqa: E731
    o, lse = dec.decode_attn(f(inp["q"]), f(inp["k_pool"]), f(inp["v_pool"]),
                             inp["block_table"].numpy(), inp["seq_lens"].numpy(), sel, w.block)
    compare("o", f(gpu["o"]), o, w.dtype)
    compare("lse", gpu["lse"].numpy(), lse, w.dtype)
    return gpu


CASES = [
    # name, B, Hq, Hkv, D, blk, seq_lens, K, dtype, pool_pages
    ("g4_d128_b64", 4, 8, 2, 128, 64, (1, 64, 65, 1000), 3, "bf16", 0),
    ("g4_full_cache", 2, 8, 2, 128, 64, (640, 577), 4, "bf16", 0),
    ("g5_shared_pages", 3, 10, 2, 128, 64, (300, 129, 1024), 5, "bf16", 7),
    ("g1_d64_b16", 2, 3, 3, 64, 16, (200, 17), 4, "bf16", 0),
    ("g4_d64_b32_fp32", 2, 4, 1, 64, 32, (97, 320), 2, "fp32", 0),
    ("g2_d128_b16_fp32", 1, 4, 2, 128, 16, (333,), 6, "fp32", 0),
    ("k0", 2, 8, 2, 128, 64, (500, 64), 0, "bf16", 0),
    ("k_all", 2, 8, 2, 128, 64, (500, 64), 50, "bf16", 0),
    # bf16 / D = 128 / b = 64 runs on the matrix-core tile kernel up to G = 32
    # heads per group (one MFMA column per head); larger groups on the other
    ("g32_mfma_columns_full", 2, 32, 1, 128, 64, (700, 63), 4, "bf16", 0),
    ("g40_beyond_mfma_columns", 1, 40, 1, 128, 64, (700,), 4, "bf16", 0),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_decode_small_parity(case):
    name, B, Hq, Hkv, D, blk, lens, K, dt, pool = case
    w = workloads.decode_custom(B, Hq, Hkv, D, blk, lens, K, dtype=dt,
                                seed=sum(map(ord, name)) % 997, pool_pages=pool)
    decode_parity(w, cap=max(1, min(K, w.max_blocks - 1)))


@pytest.mark.parametrize("name", list(workloads.DECODE_WORKLOADS))
def test_decode_named_workloads(name):
    decode_parity(workloads.DECODE_WORKLOADS[name])


def test_decode_ties_and_capacity_flag():
    w = workloads.decode_custom(1, 4, 1, 64, 16, (16 * 7 + 3,), 2, dtype="fp32", seed=3)
    p = problem_of(w)
    inp = workloads.generate_decode(w)
    inp["scores"][0, 0, :7] = torch.tensor([1.0, 2.0, 2.0, 2.0, 0.5, -0.0, 0.0])
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    gpu = run_gpu(p, inp, cap=2, status=status)
    assert int(status.item()) == -4                       # SAS_E_CAPACITY
    assert int(gpu["sel_cnt"][0, 0]) == 3 and float(gpu["tau"][0, 0]) == 2.0
    assert gpu["sel_idx"][0, 0].tolist() == [1, 2]
    status.zero_()
    gpu = run_gpu(p, inp, cap=6, status=status)
    assert int(status.item()) == 0
    check_select(gpu, inp, w.block, 2)


@pytest.mark.parametrize("blocks,K,kind", [(8192, 32, "gumbel"), (16384, 32, "gumbel"),
                                            (8192, 100, "gumbel"), (8192, 32, "halves"),
                                            (16384, 64, "few_ties"), (600, 32, "halves")],
                         ids=["c8192_k32", "c16384_k32", "c8192_k100", "c8192_heavy_ties",
                              "c16384_tied_top", "c600_heavy_ties"])
def test_decode_select_long_rows(blocks, K, kind):
    """The selection alone on long rows (up to the 16384-block limit): Gumbel
    scores; scores rounded to multiples of 1/2, so most keys tie and the
    tied candidates exceed what the exact search gathers; and rows whose top
    scores tie at the threshold.  Sets, counts and thresholds exact."""
    B, Hkv = 2, 2
    lens = (blocks * 64, blocks * 64 - 5000)
    g = torch.Generator().manual_seed(blocks + K)
    u = torch.rand(B, Hkv, blocks, generator=g).clamp_(1e-30, 1 - 2 ** -24)
    s = -torch.log(-torch.log(u))
    if kind == "halves":
        s = torch.floor(s * 2.0) / 2.0
    elif kind == "few_ties":
        s[:, :, 100:100 + 3 * K:3] = 30.0    # K tied maxima, then the Gumbel rest
        s[:, :, 7] = 30.0                    # one more tie at the top
    p = api.DecodeProblem(B, 8, Hkv, 128, 64, blocks, 1, K, "bf16")
    cap = K + 8
    dev = torch.device("cuda:0")
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    tau, si, sc = api.decode_select(p, s.to(dev), torch.tensor(lens, dtype=torch.int32, device=dev),
                                    sel_cap=cap, status=status)
    torch.cuda.synchronize()
    inp = {"scores": s, "seq_lens": torch.tensor(lens, dtype=torch.int32)}
    gpu = {"tau": tau.cpu(), "sel_idx": si.cpu(), "sel_cnt": sc.cpu()}
    sel = check_select(gpu, inp, 64, K)
    over = sel.sum(-1) > cap
    assert int(status.item()) == (-4 if over.any() else 0)


def test_decode_out_of_range_inputs_are_flagged():
    """Lengths, pages and selected indices outside their ranges are clamped or
    skipped by the kernels (every access stays in bounds) and flagged."""
    w = workloads.decode_custom(2, 4, 1, 128, 64, (200, 300), 2, seed=5)
    p = problem_of(w)
    for what in ("len", "page", "sel"):
        inp = workloads.generate_decode(w)
        if what == "len":
            inp["seq_lens"][1] = w.max_blocks * 64 + 5
        elif what == "page":
            inp["block_table"][0, 1] = w.pages + 3
        status = torch.zeros(1, dtype=torch.int32, device="cuda")
        dev = torch.device("cuda:0")
        t = {k: v.to(dev) for k, v in inp.items()}
        _, si, sc = api.decode_select(p, t["scores"], t["seq_lens"], status=status)
        if what == "sel":
            si[0, 0, 0] = 3          # block 3 is not historical for a 200-token sequence
            sc[0, 0] = 1
        # every row selects block 1 of sequence 0 (K >= 1) so the bad page is read
        if what == "page":
            si[0, 0, 0] = 1
            sc[0, 0] = 1
        o, lse = api.decode_attn(p, t["q"], t["k_pool"], t["v_pool"], t["block_table"],
                                 t["seq_lens"], si, sc, status=status)
        torch.cuda.synchronize()
        log(f"  {what}: status {int(status.item())}")
        assert int(status.item()) == -1, what             # SAS_E_INVALID
        assert torch.isfinite(o.float()).all() and torch.isfinite(lse).all()


def test_decode_bitwise_deterministic():
    w = workloads.decode_custom(3, 8, 2, 128, 64, (777, 2000, 64), 6, seed=9, pool_pages=40)
    p = problem_of(w)
    inp = workloads.generate_decode(w)
    a = run_gpu(p, inp)
    b = run_gpu(p, inp)
    bits = {torch.bfloat16: torch.int16, torch.float32: torch.int32, torch.int32: torch.int32}
    for n in a:
        assert torch.equal(a[n].view(bits[a[n].dtype]), b[n].view(bits[b[n].dtype])), n
