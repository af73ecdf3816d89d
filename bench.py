"""Benchmark of one Prism sparse-attention layer on one MI355X.

A step is the whole hot path over one batch of synthetic input: the plan
(zone statistics, shapes, re-layout and pooling, block scores, Top-k U Top-p
selection, key-major lists), the sparse attention forward and the backward.
Default workload: the 2K training-scale layer (72 x 120 x 120 = 1,036,800
tokens, 40 heads of 128, bf16, k = 16, p = 0.9).

Prints one JSON line.  `value` is the effective throughput of the selected
block attention over the whole step: (4 + 10) * head_dim * sum over selected
(query block, key block) pairs of B_i * B_j FLOP (forward + backward with the
QK^T recompute, the FlashAttention convention) divided by the step time.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E

# algorithmic FLOP per selected pair (B_i * B_j tokens), per head_dim channel
FLOP_PER_PAIR = {"attn.fwd": 4, "bwd.dkdv": 8, "bwd.dq": 6}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--workload", default="train2k")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU-oracle baseline leg")
    ap.add_argument("--cpu-blocks", type=int, default=0,
                    help="query blocks in the CPU-oracle sample (0 = host cores)")
    ap.add_argument("--fwd-only", action="store_true")
    return ap.parse_args()


def cpu_baseline(wl, x, nblocks):
    """The oracle as it is, on a bounded sample: the forward of `nblocks`
    query blocks of head 0 (smallest volumes first), fp64, OpenMP over
    blocks.  Rate in TFLOP/s of the same 4 * D * B_i * B_j accounting."""
    import numpy as np
    import torch

    from dynamic_block_sparse_zone_amd import synth
    from oracle import oracle as O

    h0 = {n: x[n][0:1].contiguous() for n in ("q", "k", "v")}
    bits = {n: synth.to_numpy_bits(h0[n]) for n in h0}
    av = x["av"].detach().cpu().numpy()
    cfg = O.Config(wl.T, wl.H, wl.W, 1, wl.head_dim, top_k=wl.top_k, top_p=wl.top_p,
                   top_k_frac=wl.top_k_frac,
                   volume_mask=wl.volume_mask, fixed_shape=tuple(wl.fixed_shape))
    pl = O.plan(bits["q"], bits["k"], bits["v"], av, cfg)
    lens = pl.blk_len[: pl.nblk(0)]
    order = np.argsort(lens, kind="stable")
    rng = np.random.default_rng(0)
    small = order[: max(nblocks * 8, nblocks)]
    pick = sorted(rng.choice(small, min(nblocks, len(small)), replace=False).tolist())
    items = [(0, int(i)) for i in pick]
    pairs = 0
    for _, i in items:
        sel = O.select_row(pl, 0, i)
        pairs += int(lens[i]) * int(pl.blk_len[sel].sum())
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    t0 = time.perf_counter()
    O.attn_fwd(bits["q"], bits["k"], bits["v"], pl, items)
    dt = time.perf_counter() - t0
    flops = 4.0 * wl.head_dim * pairs
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": min(threads, len(items)),
            "kind": "oracle",
            "sample": f"fp64 oracle forward of {len(items)} query blocks of head 0 "
                      f"({pairs} selected token pairs, {dt:.1f} s)"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: this build has no multi-GPU path "
              f"(asked for --gpus {args.gpus})", file=sys.stderr)
        sys.exit(2)
    import torch

    import dynamic_block_sparse_zone_amd as prism
    from dynamic_block_sparse_zone_amd import synth

    wl = synth.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    t0 = time.time()
    x = synth.make_inputs(wl, device=dev, with_grad=not args.fwd_only)
    torch.cuda.synchronize()
    print(f"[bench] inputs {wl.name} drawn in {time.time() - t0:.1f}s", file=sys.stderr,
          flush=True)
    q, k, v, do, av = x["q"], x["k"], x["v"], x["do"], x["av"]
    kw = dict(T=wl.T, H=wl.H, W=wl.W, top_k=wl.top_k, top_p=wl.top_p, top_k_frac=wl.top_k_frac,
              volume_mask=wl.volume_mask, fixed_shape=tuple(wl.fixed_shape),
              need_backward=not args.fwd_only)
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:2], dtype=torch.float32, device=dev)
    grads = None if args.fwd_only else (torch.empty_like(q), torch.empty_like(k),
                                        torch.empty_like(v))
    # first plan sizes the workspace once
    pl = prism.plan(q, k, v, av, **kw)
    ws, cap = pl.workspace, pl.nnz
    bws = None if args.fwd_only else torch.empty(prism.attn_bwd_workspace_bytes(pl),
                                                 dtype=torch.uint8, device=dev)
    pl.close()
    del pl

    long_steps = wl.N >= 500_000

    def note(msg):
        # progress of multi-second steps (the plan already synchronises)
        if long_steps:
            torch.cuda.synchronize()
            print(f"[bench]   {msg} at {time.time() - t0:.1f}s", file=sys.stderr, flush=True)

    def step():
        p = prism.plan(q, k, v, av, nnz_capacity=cap, workspace=ws, **kw)
        note("plan done")
        prism.attn_fwd(p, q, k, v, o, lse)
        note("forward done")
        if grads is not None:
            prism.attn_bwd(p, q, k, v, o, lse, do, *grads, workspace=bws)
            note("backward done")
        return p

    for i in range(args.warmup):
        step().close()
        torch.cuda.synchronize()
        print(f"[bench] warmup step {i} done", file=sys.stderr, flush=True)
    prism.timing_enable(True)
    prism.timing_read()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t_start = time.perf_counter()
    ev0.record()
    last = None
    for i in range(args.steps):
        if last is not None:
            last.close()
        last = step()
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    stages = prism.timing_read()
    prism.timing_enable(False)
    ms_step = ev0.elapsed_time(ev1) / args.steps
    info = last.info()
    print(f"[bench] timed {args.steps} step(s): {ms_step:.1f} ms/step (wall {wall:.1f}s)",
          file=sys.stderr, flush=True)

    D = wl.head_dim
    pairs = info["pair_tokens"]
    per_pair = 4 + (0 if args.fwd_only else 10)
    flops = per_pair * D * pairs
    value = flops / (ms_step * 1e-3) / 1e12
    ms = {name: tot / args.steps for name, (cnt, tot) in stages.items()}
    attn_ms = sum(ms.get(s, 0.0) for s in ("attn.fwd", "bwd.prep", "bwd.dkdv", "bwd.dq"))
    # dominant kernel and its roofline
    cand = {s: stages[s] for s in FLOP_PER_PAIR if s in stages}
    dom = max(cand, key=lambda s: cand[s][1])
    launches, tot = cand[dom]
    achieved = FLOP_PER_PAIR[dom] * D * pairs / (tot / launches * 1e-3) / 1e12
    es = 2 if wl.dtype == "bf16" else 4
    tensor_bytes = wl.heads * wl.N * D * es
    plan_ms = sum(v for s, v in ms.items() if s.startswith("plan."))
    nblk2 = None
    try:
        off = last.export("blk_off")
        nblk2 = float(sum((off[h + 1] - off[h]) ** 2 for h in range(wl.heads)))
    except Exception:
        pass
    out = {
        "metric": "selected-block attn TFLOP/s (% bf16 MFMA peak) + ms/layer fwd+bwd, N≈1M tok",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if wl.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": f"{wl.name}: T*H*W={wl.T}x{wl.H}x{wl.W} ({wl.N} tokens), "
                               f"{wl.heads} heads x {D}, "
                               f"k={f'{wl.top_k_frac:g} of N_blk' if wl.top_k_frac else wl.top_k}, "
                               f"p={wl.top_p}, "
                               f"{'fwd' if args.fwd_only else 'fwd+bwd'}",
                   "tokens": wl.N, "heads": wl.heads, "head_dim": D, "top_k": wl.top_k,
                   "top_k_frac": wl.top_k_frac,
                   "top_p": wl.top_p, "parallelism": "single GPU"},
        "roofline": {"bound": "mfma", "kernel": dom, "achieved": round(achieved, 2),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": None},
        "pct_bf16_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
        "attn_tflops": round(flops / (attn_ms * 1e-3) / 1e12, 2) if attn_ms else None,
        "stage_ms": {s: round(v, 3) for s, v in sorted(ms.items())},
        "plan_ms": round(plan_ms, 2),
        "plan_stats_gbs": round(tensor_bytes / (ms["plan.stats"] * 1e-3) / 1e9, 1)
        if ms.get("plan.stats") else None,
        "plan_permute_gbs": round(5 * tensor_bytes / (ms["plan.permute"] * 1e-3) / 1e9, 1)
        if ms.get("plan.permute") else None,
        "selected_pairs": info["nnz"],
        "selected_token_pairs": pairs,
        "density": round(info["nnz"] / nblk2, 4) if nblk2 else None,
        "total_blocks": info["total_blocks"],
        "shape_hist": info["shape_hist"],
        "wall_s": round(wall, 2),
    }
    if not args.no_cpu:
        nb = args.cpu_blocks or max(1, min(16, os.cpu_count() or 1))
        print(f"[bench] cpu baseline: oracle on {nb} query blocks", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(wl, x, nb)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
