#!/usr/bin/env python3
"""Benchmark of the SAS gated block-sparse attention hot path on one MI355X.

One step = the whole hot path on one batch of synthetic input already resident
in HBM: gate activation + Top-K threshold (sas_gate_threshold), forward
(sas_gated_attn_fwd) and backward (sas_gated_attn_bwd_dq, then
sas_gated_attn_bwd_dkdv, which also writes dlog_gate and dscores).

Metric: fwd+bwd effective TFLOP/s = 14 * D * pairs / step time, where pairs
counts only the attended (query, key) pairs: per query block the causal
diagonal triangle plus the selected 64x64 blocks, times the G heads of a kv
group.  Recomputation inside the backward is not counted.

Prints one JSON line.  Default workload: Qwen3-8B attention shape, 32k
context, K = 16 (batch 1, 32 query / 8 kv heads, head_dim 128, block 64).
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "fwd+bwd effective TFLOP/s at Qwen3-8B shape, 32k ctx, K=16 blocks"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 matrix peak
PEAK_HBM_GBS = 8000.0
PEAK_FP32_VALU_TFLOPS = 157.3   # MI355X fp32 vector peak


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="qwen3_8b_32k")
    ap.add_argument("--budget", type=int, default=None)
    ap.add_argument("--o-dtype", default="bf16", choices=["fp32", "bf16"])
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="wall-clock budget of the CPU-oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--fwd-only", action="store_true",
                    help="time gate/threshold + forward only (metric: 4 D pairs / time)")
    # variants of the method (each measured on the chosen workload)
    ap.add_argument("--gate-act", default="softmax", choices=["softmax", "sigmoid", "raw"])
    ap.add_argument("--gate-pos", default="inner", choices=["inner", "outer"])
    ap.add_argument("--gate-rank", default="soft", choices=["soft", "hard_ste"])
    ap.add_argument("--score-heads", default="group", choices=["group", "head"])
    ap.add_argument("--varlen", default=None, choices=["padded", "packed"],
                    help="variable-length batch: seeded lengths in [N/2, N] per sequence")
    ap.add_argument("--decode", nargs="?", const="qwen3_4b_decode_b8_64k", default=None,
                    metavar="WORKLOAD",
                    help="time the sparse-decode step (select + attention) of a decode workload "
                         "instead of the training step")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy (reference for the "
                         "FETCH_SIZE / WRITE_SIZE counter scale) and exit")
    return ap.parse_args()


# HBM traffic of the dominant kernel, from rocprofv3 counter runs recorded in
# profiles/ (FETCH_SIZE and WRITE_SIZE per dispatch, scaled by what the same
# counters read for a plain copy of known size).  Used only while the kernel
# sources still hash to the value recorded with the counters.
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_bwd_dkdv_kernel_qwen3_8b_32k.txt")
KERNEL_SOURCES = ["gated_block_sparse_attn_amd/csrc/sas_mfma_bwd.hip",
                  "gated_block_sparse_attn_amd/csrc/sas_internal.h"]


def kernel_source_hash():
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def recorded_traffic(workload, budget):
    """Bytes per launch of the key-major kernel if the recorded counters are
    for this workload and the current sources, else None."""
    try:
        with open(TRAFFIC_FILE) as fh:
            kv = dict(line.split("=", 1) for line in fh.read().splitlines()
                      if "=" in line and not line.startswith("#"))
    except OSError:
        return None
    if (kv.get("source_sha", "").strip() != kernel_source_hash()
            or kv.get("workload", "").strip() != workload
            or int(kv.get("budget_k", "-1")) != budget):
        return None
    return float(kv["hbm_bytes_per_launch"])


def calibrate_copy():
    """A plain copy of known size: 1 GiB read + 1 GiB written per call."""
    import torch
    n = 1 << 30
    x = torch.empty(n, dtype=torch.uint8, device="cuda")
    y = torch.empty_like(x)
    x.fill_(1)
    for _ in range(3):
        y.copy_(x)
    torch.cuda.synchronize()
    print(json.dumps({"calibrate_copy_bytes": n, "calls": 3}), flush=True)


def count_pairs(sel_cnt, cap, block, group):
    import torch
    cnt = torch.clamp(sel_cnt.to(torch.int64), max=cap)
    units = cnt.numel()
    return group * (units * block * (block + 1) // 2 + block * block * int(cnt.sum().item()))


def unit_pairs(units, cnt, block, heads_per_row, lens=None):
    """Attended (query, key) pairs of the gate rows `units` = (b, s, i):
    the causal triangle of the valid rows of block i plus those rows times
    every selected (full) block, times the query heads of the row."""
    total = 0
    for (b, s, i) in units:
        nv = block if lens is None else max(0, min(block, int(lens[b]) - i * block))
        total += heads_per_row * (nv * (nv + 1) // 2 + nv * block * int(cnt[b, s, i]))
    return total


def cpu_baseline(w, K, inp, budget_s, total_pairs, fwd_only=False, act="softmax", pos="inner",
                 rank="soft", lens=None):
    """Time the float64 CPU oracle on a bounded sample of the same workload
    (forward and backward, or the forward alone; with the run's gate variant
    and sequence lengths)."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        blas = [x for x in threadpool_info() if x.get("user_api") == "blas"]
        threads = int(blas[0]["num_threads"]) if blas else (os.cpu_count() or 1)
        vendor = blas[0].get("internal_api", "?") if blas else "?"
    except Exception:   # threadpoolctl missing
        threads, vendor = os.cpu_count() or 1, "?"
    scores = inp["scores"].numpy()
    t0 = time.perf_counter()
    lg, _, sel = oracle.gate_threshold(scores, K, act=act, seq_lens=lens, block=w.block)
    t_thr = time.perf_counter() - t0
    if rank == "hard_ste":   # unit gates on the selected blocks
        lg = np.where(np.isfinite(lg), 0.0, lg)
    q, k, v, do = (inp[n].float().numpy() for n in ("q", "k", "v", "do"))
    c = w.n_blocks
    hs = scores.shape[1]
    rng = np.random.default_rng(0)
    all_units = [(b, h, i) for b in range(w.batch) for h in range(hs) for i in range(c)]
    order = rng.permutation(len(all_units))
    cnt = sel.sum(-1)

    def pairs_of(units):
        return unit_pairs(units, cnt, w.block, w.n_q_heads // hs, lens)

    def run(units):
        t = time.perf_counter()
        oracle.forward(q, k, v, lg, sel, w.block, query_blocks=units, gate_pos=pos, seq_lens=lens)
        if not fwd_only:
            oracle.backward(q, k, v, do, lg, sel, w.block, query_blocks=units, gate_pos=pos,
                            seq_lens=lens)
        return time.perf_counter() - t

    probe = [all_units[j] for j in order[:2]]
    t_probe = run(probe)
    per = t_probe / 2
    n = int(max(2, min(len(all_units), (budget_s - t_thr - t_probe) / max(per, 1e-6))))
    sample = [all_units[j] for j in order[2:2 + n]] or probe
    t_fb = run(sample)
    sp = pairs_of(sample)
    est = t_thr + t_fb * total_pairs / sp
    flops = (4 if fwd_only else 14) * w.head_dim * total_pairs
    part = "fwd" if fwd_only else "fwd+bwd"
    return {"value": flops / est / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": (f"float64 numpy oracle: gate/threshold over all {len(all_units)} rows "
                       f"({t_thr:.2f} s) + {part} of {len(sample)} of {len(all_units)} query "
                       f"blocks ({t_fb:.2f} s), scaled by attended pairs to the whole workload "
                       f"(est. {est:.1f} s per step); BLAS={vendor}")}


def decode_bench(args):
    """One step = sas_decode_select + sas_decode_attn for a batch of sequences,
    inputs resident in HBM.  value = sequences (new tokens) per second."""
    import numpy as np
    import torch
    from gated_block_sparse_attn_amd import api, workloads

    w = workloads.DECODE_WORKLOADS[args.decode]
    p = api.DecodeProblem(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.block, w.max_blocks,
                          w.pages, w.budget, w.dtype)
    cap = p.default_cap()
    print(f"[bench] generating {w.name} inputs", file=sys.stderr, flush=True)
    inp = workloads.generate_decode(w)
    dev = torch.device("cuda:0")
    t = {k: v.to(dev) for k, v in inp.items()}
    tau = torch.empty(w.batch, w.n_kv_heads, dtype=torch.float32, device=dev)
    si = torch.empty(w.batch, w.n_kv_heads, cap, dtype=torch.int32, device=dev)
    sc = torch.empty(w.batch, w.n_kv_heads, dtype=torch.int32, device=dev)
    o = torch.empty(w.batch, w.n_q_heads, w.head_dim, dtype=p.torch_dtype, device=dev)
    lse = torch.empty(w.batch, w.n_q_heads, dtype=torch.float32, device=dev)
    ws = torch.empty(api.decode_workspace_size(p, cap), dtype=torch.uint8, device=dev)

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        api.decode_select(p, t["scores"], t["seq_lens"], sel_cap=cap, outputs=(tau, si, sc))
        if ev is not None:
            ev[1].record()
        api.decode_attn(p, t["q"], t["k_pool"], t["v_pool"], t["block_table"], t["seq_lens"],
                        si, sc, o=o, lse=lse, workspace=ws)
        if ev is not None:
            ev[2].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for k in range(args.steps):
        step(events[k])
    end.record()
    torch.cuda.synchronize()
    ms_step = start.elapsed_time(end) / args.steps
    stage_ms = {}
    for si_, name in enumerate(("select", "attn")):
        vals = sorted(events[k][si_].elapsed_time(events[k][si_ + 1]) for k in range(args.steps))
        stage_ms[name] = {"mean": sum(vals) / len(vals), "median": vals[len(vals) // 2],
                          "min": vals[0]}
    # algorithmic HBM bytes of the attention stage: the attended K / V rows of
    # every (sequence, kv head) once, q, o and lse
    el = 2 if w.dtype == "bf16" else 4
    cnt = np.minimum(sc.cpu().numpy(), cap)
    lens = np.array(w.seq_lens)
    cur = lens - ((lens - 1) // w.block) * w.block
    rows = w.block * cnt.sum() + w.n_kv_heads * cur.sum()
    attn_bytes = (2 * rows * w.head_dim * el + 2 * w.batch * w.n_q_heads * w.head_dim * el
                  + 4 * w.batch * w.n_q_heads)
    achieved = attn_bytes / (stage_ms["attn"]["mean"] * 1e-3) / 1e9
    o_eager, lse_eager = o.clone(), lse.clone()

    # The same step captured once in a HIP graph and replayed (how a serving
    # loop runs decode): the attention goes through the allocation-free entry
    # point, so nothing is allocated under capture.  Every replay's o / lse
    # is checked bit-equal to the eager step.
    def step_noalloc():
        api.decode_select(p, t["scores"], t["seq_lens"], sel_cap=cap, outputs=(tau, si, sc))
        api.decode_attn_noalloc(p, t["q"], t["k_pool"], t["v_pool"], t["block_table"],
                                t["seq_lens"], si, sc, o, lse)

    cs = torch.cuda.Stream()
    cs.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cs):
        step_noalloc()   # first use of the per-device scratch outside the capture
        cs.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=cs):
            step_noalloc()
    torch.cuda.current_stream().wait_stream(cs)
    torch.cuda.synchronize()
    for _ in range(args.warmup):
        graph.replay()
    torch.cuda.synchronize()
    g0 = torch.cuda.Event(enable_timing=True)
    g1 = torch.cuda.Event(enable_timing=True)
    g0.record()
    for _ in range(args.steps):
        graph.replay()
    g1.record()
    torch.cuda.synchronize()
    ms_graph = g0.elapsed_time(g1) / args.steps
    assert torch.equal(o.view(torch.int16 if o.dtype == torch.bfloat16 else torch.int32),
                       o_eager.view(torch.int16 if o.dtype == torch.bfloat16 else torch.int32)), \
        "graph replay differs from the eager step"
    assert torch.equal(lse, lse_eager), "graph replay differs from the eager step"

    result = {
        "metric": "sparse decode tokens/s (select + attention, one new token per sequence)",
        "value": w.batch / (ms_graph * 1e-3), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_graph,
        "timing": "HIP graph replay of the whole step (eager launches: ms_per_step_eager)",
        "ms_per_step_eager": ms_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": w.dtype,
        "data": "synthetic (seeded torch generator; Qwen3-shaped paged cache, random values)",
        "config": {"workload": w.name, "batch": w.batch, "n_q_heads": w.n_q_heads,
                   "n_kv_heads": w.n_kv_heads, "head_dim": w.head_dim, "block": w.block,
                   "budget_k": w.budget, "max_seq_len": int(max(w.seq_lens)),
                   "max_blocks": w.max_blocks},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": achieved / PEAK_HBM_GBS, "traffic": None,
                     "kernel": ("decode_attn_mfma_kernel" if (w.dtype == "bf16" and w.head_dim == 128
                                                                 and w.block == 64 and w.group <= 32)
                                else "decode_attn_kernel") + " + decode_combine_kernel",
                     "stage_ms_mean": stage_ms["attn"]["mean"],
                     "algorithmic_bytes_per_launch": int(attn_bytes)},
        "stage_ms": stage_ms,
    }
    if not args.no_cpu_baseline:
        import oracle.sas_decode_oracle as dec
        f = lambda x: x.float().numpy()   # noqa: E731
        t0 = time.perf_counter()
        _, sel = dec.decode_select(inp["scores"].numpy(), inp["seq_lens"].numpy(), w.block,
                                   w.budget)
        dec.decode_attn(f(inp["q"]), f(inp["k_pool"]), f(inp["v_pool"]),
                        inp["block_table"].numpy(), inp["seq_lens"].numpy(), sel, w.block)
        dt = time.perf_counter() - t0
        result["cpu_baseline"] = {"value": w.batch / dt, "unit": "tokens/s", "cores": 1,
                                  "kind": "oracle",
                                  "sample": f"float64 numpy decode oracle, the whole step "
                                            f"({w.batch} sequences) once: {dt:.3f} s"}
    print(json.dumps(result), flush=True)


def main():
    args = parse()
    if args.calibrate_copy:
        calibrate_copy()
        return
    if args.decode:
        if args.gpus != 1:
            print("bench.py measures one GPU only", file=sys.stderr)
            sys.exit(2)
        decode_bench(args)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the path shards over (batch, kv head) with no exchange; see the design notes)",
              file=sys.stderr)
        sys.exit(2)
    import torch
    from gated_block_sparse_attn_amd import api, workloads

    import dataclasses

    import numpy as np

    w = workloads.WORKLOADS[args.workload]
    if args.score_heads != "group":
        w = dataclasses.replace(w, score_heads=args.score_heads)
    K = args.budget if args.budget is not None else w.budgets[0]
    dev = torch.device("cuda:0")
    lens = None
    if args.varlen:   # seeded lengths, uniform in [N/2, N]
        lens = np.random.default_rng(1234).integers(w.seq_len // 2, w.seq_len + 1, size=w.batch)
    seq_t = cu_t = None
    total_tokens = 0
    if args.varlen == "padded":
        seq_t = torch.tensor(lens, dtype=torch.int32, device=dev)
    elif args.varlen == "packed":
        cu_t = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32, device=dev)
        total_tokens = int(lens.sum())
    p = api.Problem(w.batch, w.n_q_heads, w.n_kv_heads, w.seq_len, w.head_dim, w.block, K,
                    w.dtype, 0.0, args.o_dtype if w.dtype == "bf16" else "fp32", args.gate_act,
                    args.gate_pos, args.gate_rank, args.score_heads, seq_t, cu_t, total_tokens)
    variant = {n: x for n, x in (("gate_act", args.gate_act), ("gate_pos", args.gate_pos),
                                  ("gate_rank", args.gate_rank),
                                  ("score_heads", args.score_heads))
               if x not in ("softmax", "inner", "soft", "group")}
    if args.varlen:
        variant["varlen"] = args.varlen
        variant["seq_lens"] = [int(x) for x in lens]
    # the matrix-core kernels serve bf16 / D = 128 / b = 64 with inner gates
    # (any activation, soft or hard, per-group or per-head, fixed or variable
    # lengths); the outer position runs on the vector-ALU kernels
    on_mfma = w.dtype == "bf16" and w.head_dim == 128 and w.block == 64
    cap = p.default_cap()
    print(f"[bench] generating {w.name} inputs", file=sys.stderr, flush=True)
    inp = workloads.generate(w)
    if args.varlen == "packed":
        pk = lambda x: torch.cat([x[b, :, :int(n)].transpose(0, 1) for b, n in enumerate(lens)],
                                 dim=0).contiguous()   # noqa: E731
        q, k, v, do = (pk(inp[n]).to(dev) for n in ("q", "k", "v", "do"))
        lse_shape = (w.n_q_heads, total_tokens)
    else:
        q, k, v, do = (inp[n].to(dev) for n in ("q", "k", "v", "do"))
        lse_shape = tuple(q.shape[:3])
    scores = inp["scores"].to(dev)
    sh_q, sh_kv = q.shape, k.shape
    c = w.n_blocks
    hs = p.n_score_heads
    lg = torch.empty(w.batch, hs, c, c, dtype=torch.float32, device=dev)
    tau = torch.empty(w.batch, hs, c, dtype=torch.float32, device=dev)
    sel_idx = torch.empty(w.batch, hs, c, cap, dtype=torch.int32, device=dev)
    sel_cnt = torch.empty(w.batch, hs, c, dtype=torch.int32, device=dev)
    o = torch.empty(sh_q, dtype=p.torch_o_dtype, device=dev)
    lse = torch.empty(lse_shape, dtype=torch.float32, device=dev)
    dq = torch.empty(sh_q, dtype=p.torch_dtype, device=dev)
    dk = torch.empty(sh_kv, dtype=p.torch_dtype, device=dev)
    dv = torch.empty(sh_kv, dtype=p.torch_dtype, device=dev)
    dlg = torch.empty_like(lg)
    dsc = torch.empty_like(lg)
    ws = torch.empty(api.bwd_workspace_size(p, cap), dtype=torch.uint8, device=dev)
    stages = ["threshold", "fwd"] if args.fwd_only else ["threshold", "fwd", "bwd_dq", "bwd_dkdv"]

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        api.gate_threshold(p, scores, sel_cap=cap, outputs=(lg, tau, sel_idx, sel_cnt))
        if ev is not None:
            ev[1].record()
        api.gated_attn_fwd(p, q, k, v, lg, sel_idx, sel_cnt, o=o, lse=lse)
        if ev is not None:
            ev[2].record()
        if args.fwd_only:
            return
        api.gated_attn_bwd_dq(p, q, k, v, o, do, lse, lg, sel_idx, sel_cnt, dq, ws)
        if ev is not None:
            ev[3].record()
        api.gated_attn_bwd_dkdv(p, q, k, v, do, lse, lg, sel_idx, sel_cnt, dk, dv, dlg, dsc, ws)
        if ev is not None:
            ev[4].record()

    print(f"[bench] warmup {args.warmup}", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    nev = len(stages) + 1
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(nev)] for _ in range(args.steps)]
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    print(f"[bench] timing {args.steps} steps", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    start.record()
    for s in range(args.steps):
        step(events[s])
    end.record()
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    ms_total = start.elapsed_time(end)
    ms_step = ms_total / args.steps
    # one cold step after a 1 GiB write has evicted L2 and MALL (context only)
    scratch = torch.empty(1 << 28, dtype=torch.float32, device=dev)
    scratch.fill_(1.0)
    cold = [torch.cuda.Event(enable_timing=True) for _ in range(nev)]
    torch.cuda.synchronize()
    step(cold)
    torch.cuda.synchronize()
    cold_ms = cold[0].elapsed_time(cold[-1])
    del scratch
    stage_ms = {}
    for si, name in enumerate(stages):
        vals = sorted(events[s][si].elapsed_time(events[s][si + 1]) for s in range(args.steps))
        stage_ms[name] = {"mean": sum(vals) / len(vals), "median": vals[len(vals) // 2],
                          "min": vals[0]}

    cnt_np = np.minimum(sel_cnt.cpu().numpy(), cap)
    if lens is None and args.score_heads == "group":
        pairs = count_pairs(sel_cnt, cap, w.block, w.group)
    else:
        pairs = unit_pairs([(b, s, i) for b in range(w.batch) for s in range(hs) for i in range(c)],
                           cnt_np, w.block, w.n_q_heads // hs, lens)
    D = w.head_dim
    flops = (4 if args.fwd_only else 14) * D * pairs
    value = flops / (ms_step * 1e-3) / 1e12
    # algorithmic flops of the main kernel of each stage
    if on_mfma:
        kflops = {"fwd": 4 * D * pairs, "bwd_dq": 6 * D * pairs, "bwd_dkdv": 4 * D * pairs}
        nh = 1 if args.score_heads == "head" else 2
        knames = {"fwd": f"fwd_mfma_kernel<{nh}>", "bwd_dq": f"bwd_dq_kernel<{2 * nh if nh > 1 else 1}>",
                  "bwd_dkdv": "bwd_dkdv_kernel"}
        bound, peak = "mfma", PEAK_BF16_TFLOPS
    else:   # vector-ALU kernels: the same algorithmic flops against the fp32 vector peak
        kflops = {"fwd": 4 * D * pairs, "bwd_dq": 6 * D * pairs, "bwd_dkdv": 4 * D * pairs}
        knames = {"fwd": "fwd_generic_kernel", "bwd_dq": "bwd_q_generic_kernel",
                  "bwd_dkdv": "bwd_kv_generic_kernel"}
        bound, peak = "alu", PEAK_FP32_VALU_TFLOPS
    kflops = {n: f for n, f in kflops.items() if n in stages}
    dom = max(kflops, key=lambda n: stage_ms[n]["mean"])
    achieved = kflops[dom] / (stage_ms[dom]["mean"] * 1e-3) / 1e12
    traffic = recorded_traffic(w.name, K) if (dom == "bwd_dkdv" and on_mfma and not variant) \
        else None
    roofline = {"bound": bound, "achieved": achieved, "peak": peak,
                "unit": "TFLOP/s", "frac": achieved / peak, "traffic": traffic,
                "kernel": knames[dom],
                "stage_ms_mean": stage_ms[dom]["mean"],
                "algorithmic_flops_per_launch": kflops[dom]}
    vtag = "".join(f", {n}={x}" for n, x in variant.items() if n != "seq_lens")
    if args.fwd_only:
        metric = f"forward effective TFLOP/s (gate/threshold + forward), {w.name}, K={K}{vtag}"
    elif w.name == "qwen3_8b_32k" and K == 16 and not variant:
        metric = METRIC
    else:
        metric = f"fwd+bwd effective TFLOP/s, {w.name}, K={K}{vtag}"
    fwd_ms = stage_ms["threshold"]["mean"] + stage_ms["fwd"]["mean"]
    result = {
        "metric": metric, "value": value, "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": w.dtype,
        "data": "synthetic (seeded torch generator; Qwen3-shaped, random values)",
        "config": {"workload": w.name, "batch": w.batch, "n_q_heads": w.n_q_heads,
                   "n_kv_heads": w.n_kv_heads, "seq_len": w.seq_len, "head_dim": D,
                   "block": w.block, "budget_k": K, "o_dtype": p.o_dtype,
                   "attended_pairs": pairs, "flops_per_step": flops, **variant},
        "roofline": roofline,
        "stage_ms": stage_ms,
        "wall_s_timed_region": t_wall,
        "frac_of_bf16_peak": value / PEAK_BF16_TFLOPS,
        # forward-only figure from the same steps: 4 D pairs / (threshold + forward)
        "fwd_only": {"tflops": 4 * D * pairs / (fwd_ms * 1e-3) / 1e12, "ms": fwd_ms},
        "cold_ms_per_step": cold_ms,
    }
    if not args.no_cpu_baseline:
        print("[bench] CPU oracle baseline", file=sys.stderr, flush=True)
        del q, k, v, do
        result["cpu_baseline"] = cpu_baseline(w, K, inp, args.cpu_seconds, pairs, args.fwd_only,
                                              args.gate_act, args.gate_pos, args.gate_rank, lens)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
