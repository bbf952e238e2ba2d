"""The allocation-free decode entry point (sas_decode_attn_noalloc) against
the workspace-taking one (sas_decode_attn), through the C ABI.

Both run the same kernels; the allocation-free one keeps its tile partials in
the library's fixed per-device scratch.  Two calls in a row, the second with
a smaller problem (the scratch then holds the first call's partials), must
each give the bits of sas_decode_attn.  (Its refusal of problems larger than
the scratch is a host-side check, tested with the other ABI checks.)
"""

import numpy as np
import pytest
import torch

from gated_block_sparse_attn_amd import api, workloads

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield


def _problem(w):
    return api.DecodeProblem(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.block,
                             w.max_blocks, w.pages, w.budget, w.dtype)


def _bits(x: torch.Tensor) -> np.ndarray:
    return x.cpu().view(torch.int16 if x.dtype == torch.bfloat16 else torch.int32).numpy()


def _both(w):
    p = _problem(w)
    dev = torch.device("cuda:0")
    t = {k: v.to(dev) for k, v in workloads.generate_decode(w).items()}
    cap = max(p.default_cap(), 1)
    _, si, sc = api.decode_select(p, t["scores"], t["seq_lens"], sel_cap=cap)
    args = (t["q"], t["k_pool"], t["v_pool"], t["block_table"], t["seq_lens"], si, sc)
    o_ref, lse_ref = api.decode_attn(p, *args)
    o = torch.full_like(o_ref, float("nan"))
    lse = torch.full_like(lse_ref, float("nan"))
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    api.decode_attn_noalloc(p, *args, o=o, lse=lse, status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    return (o_ref, lse_ref), (o, lse)


def test_noalloc_matches_workspace_entry_two_calls():
    """A larger call, then a smaller one on the same scratch: each bit-equal to
    sas_decode_attn (the matrix-core bf16 kernel and the vector-ALU fp32 one)."""
    big = workloads.decode_custom(4, 32, 8, 128, 64, (9000, 1, 4097, 130), 32, dtype="bf16",
                                  seed=51, pool_pages=600)
    small = workloads.decode_custom(2, 8, 2, 128, 64, (700, 65), 4, dtype="bf16", seed=52)
    fp32 = workloads.decode_custom(2, 10, 2, 64, 16, (300, 17), 5, dtype="fp32", seed=53)
    for w in (big, small, fp32):
        (o_ref, lse_ref), (o, lse) = _both(w)
        assert np.array_equal(_bits(o), _bits(o_ref)), "o differs from sas_decode_attn"
        assert np.array_equal(_bits(lse), _bits(lse_ref)), "lse differs from sas_decode_attn"
        assert torch.isfinite(o.float()).all()
