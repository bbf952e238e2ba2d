"""One whole step (threshold -> forward -> backward) captured in a HIP graph and
replayed: every replay must reproduce the eager run bit for bit (the kernels
are deterministic and clear their own scratch with fill kernels, so a replay
carries no state over from the previous one).  Between replays the program
runs eager work of its own and synchronises, and the inputs are overwritten
in place with new values before the last replays, which must then match a
new eager run."""
import pytest
import torch

from gated_block_sparse_attn_amd import api, workloads
from parity import log, problem_of

pytestmark = pytest.mark.gpu


def _bits(t: torch.Tensor) -> torch.Tensor:
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


@pytest.mark.parametrize("shape", [(1, 8, 2, 2048, 128, 64, 4, "bf16"),    # matrix-core path
                                   (1, 2, 1, 512, 64, 32, 3, "fp32")],     # vector-ALU path
                         ids=["mfma", "generic"])
def test_graph_replays_match_eager(shape):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B, Hq, Hkv, N, D, blk, K, dt = shape
    log(f"graph capture {shape}")
    dev = torch.device("cuda:0")
    w = workloads.custom(B, Hq, Hkv, N, D, blk, K, dtype=dt, seed=41, score_std=2.0)
    p = problem_of(w, K)
    cap = max(1, min(K, N // blk - 1))
    inp = workloads.generate(w)
    x = {n: inp[n].to(dev) for n in ("q", "k", "v", "do", "scores")}

    def step():
        lg, tau, si, sc = api.gate_threshold(p, x["scores"], sel_cap=cap)
        o, lse = api.gated_attn_fwd(p, x["q"], x["k"], x["v"], lg, si, sc)
        dq, dk, dv, dlg, dsc = api.gated_attn_bwd(p, x["q"], x["k"], x["v"], o, x["do"], lse,
                                                  lg, si, sc)
        return dict(log_gate=lg, sel_idx=si, sel_cnt=sc, o=o, lse=lse, dq=dq, dk=dk, dv=dv,
                    dlog_gate=dlg, dscores=dsc)

    def eager():
        r = step()
        torch.cuda.synchronize()
        return {n: t.clone() for n, t in r.items()}

    ref = eager()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):   # warm-up outside the capture
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        out = step()
    torch.cuda.synchronize()

    def check(want, tag):
        for n, t in want.items():
            assert torch.equal(_bits(out[n]), _bits(t)), f"{tag}: {n} differs from the eager run"

    for r in range(3):
        g.replay()
        torch.cuda.synchronize()
        check(ref, f"replay {r}")
        eager()   # the program's own eager work between replays
    # new inputs written in place: replays follow them
    g2 = torch.Generator().manual_seed(7)
    for n in ("q", "k", "v", "do", "scores"):
        x[n].copy_(torch.randn(x[n].shape, generator=g2).to(x[n].dtype))
    ref2 = eager()
    for r in range(2):
        g.replay()
        torch.cuda.synchronize()
        check(ref2, f"replay {r} after new inputs")
