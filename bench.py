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

# timing stage -> (kernel symbol, the sources its code comes from)
KERNELS = {
    "attn.fwd": ("k_attn_fwd_bf16", ["prism_attn_fwd.hip"]),
    "bwd.dkdv": ("k_bwd_dkdv", ["prism_attn_bwd.hip"]),
    "bwd.dq": ("k_bwd_dq", ["prism_attn_bwd.hip"]),
}
COMMON_SOURCES = ["prism_attn_common.h", "prism_common.h", "prism_kernels.h"]
CALIB_BYTES = 1 << 30       # the calibration copy reads and writes this many bytes


def kernel_source_sha(stage):
    """sha256 over the sources of a stage's kernel (its counters go stale
    when these change)."""
    import hashlib
    h = hashlib.sha256()
    for name in KERNELS[stage][1] + COMMON_SOURCES:
        with open(os.path.join(ROOT, "dynamic_block_sparse_zone_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def traffic_file(stage, workload):
    return os.path.join(ROOT, "profiles", f"{KERNELS[stage][0]}_{workload}_traffic.md")


def read_traffic(stage, workload):
    """HBM bytes per launch from the committed counter summary, or None when
    there is none or the kernel's sources changed since it was taken."""
    path = traffic_file(stage, workload)
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as f:
        for line in f:
            if line.startswith("- ") and ": " in line:
                k, v = line[2:].split(": ", 1)
                vals[k.strip()] = v.strip().strip("`")
    if vals.get("source_sha256") != kernel_source_sha(stage):
        return None
    return float(vals["traffic_bytes_per_launch"])


def _kernel_rows(path, counter):
    """{kernel name: [(counter value, duration s), ...]} of a counter-collection CSV."""
    import csv
    out = {}
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] != counter:
            continue
        name = r["Kernel_Name"]
        key = "bitwise_not" if "bitwise_not" in name else name.split("(")[0].replace("void ", "")
        dur = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9
        out.setdefault(key, []).append((float(r["Counter_Value"]), dur))
    return out


def summarize_hbm_table(fetch_csv, write_csv, workload, cmds, out):
    """Measured HBM traffic and rate of every library kernel in the two
    counter passes (KiB per dispatch, calibrated by the copy)."""
    f = _kernel_rows(fetch_csv, "FETCH_SIZE")
    w = _kernel_rows(write_csv, "WRITE_SIZE")
    fs = CALIB_BYTES / (f["bitwise_not"][0][0] * 1024)
    ws = CALIB_BYTES / (w["bitwise_not"][0][0] * 1024)
    lines = [f"# HBM traffic and rate of every kernel, {workload}", "",
             "Same two counter passes as the dominant kernel's traffic summary "
             f"(`FETCH_SIZE` x {fs:.4f}, `WRITE_SIZE` x {ws:.4f}, from the 1 GiB calibration "
             "copy).  Durations are the profiled dispatches' own (counter collection "
             "serialises dispatches); rates against the 8 TB/s HBM3E peak.", "",
             "Commands (from /tmp, TMPDIR=/tmp):", "", *[f"    {c}" for c in cmds], "",
             "| kernel | dispatches | time ms | fetch GB | write GB | TB/s | % of 8 TB/s |",
             "|---|---:|---:|---:|---:|---:|---:|"]
    keys = [k for k in f if k.startswith("prism::")]
    for k in sorted(keys, key=lambda k: -sum(d for _, d in f[k])):
        t = sum(d for _, d in f[k])
        fb = sum(v for v, _ in f[k]) * 1024 * fs
        wb = sum(v for v, _ in w.get(k, [])) * 1024 * ws
        rate = (fb + wb) / t / 1e12 if t > 0 else 0.0
        lines.append(f"| `{k[7:]}` | {len(f[k])} | {t * 1e3:.2f} | {fb / 1e9:.2f} | "
                     f"{wb / 1e9:.2f} | {rate:.2f} | {100 * rate / 8:.1f} |")
    lines.append("")
    with open(out, "w") as fh:
        fh.write("\n".join(lines))
    print("\n".join(lines))


def summarize_mfma(csv_path, agent_csv, workload, cmds, out):
    """MFMA utilisation of the attention kernels from one counter pass of
    SQ_VALU_MFMA_BUSY_CYCLES, GRBM_GUI_ACTIVE and SQ_INSTS_VALU_MFMA_MOPS_BF16."""
    import csv
    busy = _kernel_rows(csv_path, "SQ_VALU_MFMA_BUSY_CYCLES")
    gui = _kernel_rows(csv_path, "GRBM_GUI_ACTIVE")
    mops = _kernel_rows(csv_path, "SQ_INSTS_VALU_MFMA_MOPS_BF16")
    gpu = next(r for r in csv.DictReader(open(agent_csv)) if r.get("Simd_Count", "0") != "0")
    simds, xcc = int(gpu["Simd_Count"]), int(gpu["Num_Xcc"])
    lines = [f"# MFMA utilisation of the attention kernels, {workload}", "",
             "One counter pass over a profiled step: `SQ_VALU_MFMA_BUSY_CYCLES` (summed over "
             f"the {simds} SIMDs), `GRBM_GUI_ACTIVE` (busy cycles, summed over the {xcc} XCDs) "
             "and `SQ_INSTS_VALU_MFMA_MOPS_BF16` (x 512 = bf16 MFMA flops).  Utilisation = "
             f"busy / (active / {xcc} x {simds}), rocprofv3's MfmaUtil, i.e. against the "
             "clock the chip actually ran; the clock is active / XCDs / duration.  The "
             "bench line's fractions are against 2.5 PFLOP/s, the peak at 2.4 GHz.", "",
             "Command (from /tmp, TMPDIR=/tmp):", "", *[f"    {c}" for c in cmds], "",
             "| kernel | s | clock GHz | MFMA busy % | MFMA TFLOP/s (counted) | % of 2.5 PFLOP/s |",
             "|---|---:|---:|---:|---:|---:|"]
    for stage, (sym, _) in KERNELS.items():
        k = next((n for n in busy if sym in n), None)
        if k is None:
            continue
        b = sum(v for v, _ in busy[k])
        t = sum(d for _, d in busy[k])
        g = sum(v for v, _ in gui[k]) / xcc
        fl = sum(v for v, _ in mops[k]) * 512
        lines.append(f"| `{sym}` ({stage}) | {t:.2f} | {g / t / 1e9:.2f} | "
                     f"{100 * b / (g * simds):.1f} | {fl / t / 1e12:.1f} | "
                     f"{100 * fl / t / 1e12 / PEAK_BF16_TFLOPS:.1f} |")
    lines.append("")
    with open(out, "w") as fh:
        fh.write("\n".join(lines))
    print("\n".join(lines))


def summarize_pmc(fetch_csv, write_csv, stage, workload, cmds, out):
    """Turns two rocprofv3 counter-collection CSVs (FETCH_SIZE, WRITE_SIZE,
    in KiB per dispatch) of a profiled step that ends with the calibration
    copy into per-launch HBM traffic of a stage's kernel, each counter
    scaled by its reading for the copy of known size."""
    import csv
    sym = KERNELS[stage][0]

    def per_kernel(path, counter):
        rows = [r for r in csv.DictReader(open(path)) if r["Counter_Name"] == counter]
        kern = [float(r["Counter_Value"]) * 1024 for r in rows if sym in r["Kernel_Name"]]
        # the calibration copy is the run's only bitwise-not kernel
        copies = [float(r["Counter_Value"]) * 1024 for r in rows
                  if "bitwise_not" in r["Kernel_Name"]]
        if not kern or len(copies) != 1:
            raise SystemExit(f"{path}: {len(kern)} {sym} and {len(copies)} copy dispatches "
                             f"with {counter}")
        return sum(kern) / len(kern), copies[0]

    fk, fc = per_kernel(fetch_csv, "FETCH_SIZE")
    wk, wc = per_kernel(write_csv, "WRITE_SIZE")
    f_scale, w_scale = CALIB_BYTES / fc, CALIB_BYTES / wc
    fetch, write = fk * f_scale, wk * w_scale
    lines = [
        f"# {sym}: HBM traffic per launch, {workload}",
        "",
        "Two `rocprofv3 --pmc` passes over one profiled step that ends with a plain",
        f"copy of {CALIB_BYTES >> 20} MiB (read and write); each counter is scaled by "
        "the factor that makes it read the copy's known size.",
        "",
        "Commands (from /tmp, TMPDIR=/tmp):",
        "",
        *[f"    {c}" for c in cmds],
        "",
        f"- kernel: `{sym}` (stage `{stage}`)",
        f"- fetch_raw_bytes_per_launch: {fk:.6g}",
        f"- write_raw_bytes_per_launch: {wk:.6g}",
        f"- copy_fetch_raw_bytes: {fc:.6g}",
        f"- copy_write_raw_bytes: {wc:.6g}",
        f"- fetch_scale: {f_scale:.4f}",
        f"- write_scale: {w_scale:.4f}",
        f"- fetch_bytes_per_launch: {fetch:.6g}",
        f"- write_bytes_per_launch: {write:.6g}",
        f"- traffic_bytes_per_launch: {fetch + write:.6g}",
        f"- source_sha256: `{kernel_source_sha(stage)}`",
        "",
    ]
    with open(out, "w") as f:
        f.write("\n".join(lines))
    print("\n".join(lines))


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
    ap.add_argument("--calib-copy", action="store_true",
                    help="end with a plain copy of known size (counter calibration)")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write the traffic summary of the dominant kernel from two "
                         "rocprofv3 counter-collection CSVs, then exit")
    ap.add_argument("--stage", default="bwd.dkdv", help="kernel stage for --summarize-pmc")
    ap.add_argument("--summarize-mfma", nargs=2, metavar=("COUNTER_CSV", "AGENT_CSV"),
                    help="write the attention kernels' MFMA utilisation summary from one "
                         "rocprofv3 counter pass (and its agent info), then exit")
    ap.add_argument("--cmd", action="append", default=[],
                    help="profiling command lines to record in the summary")
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
    if args.summarize_pmc:
        summarize_pmc(*args.summarize_pmc, args.stage, args.workload, args.cmd,
                      traffic_file(args.stage, args.workload))
        summarize_hbm_table(*args.summarize_pmc, args.workload, args.cmd,
                            os.path.join(ROOT, "profiles", f"kernels_{args.workload}_hbm.md"))
        return
    if args.summarize_mfma:
        summarize_mfma(*args.summarize_mfma, args.workload, args.cmd,
                       os.path.join(ROOT, "profiles", f"attention_{args.workload}_mfma.md"))
        return
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
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": read_traffic(dom, wl.name) if dom in KERNELS else None},
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
    if args.calib_copy:
        # one elementwise kernel that reads and writes CALIB_BYTES each (an
        # op that nothing else in the run uses, so its dispatch is found by
        # name)
        a = torch.zeros(CALIB_BYTES // 2, dtype=torch.int16, device=dev)
        b = torch.bitwise_not(a)
        torch.cuda.synchronize()
        del a, b
    if not args.no_cpu:
        nb = args.cpu_blocks or max(1, min(16, os.cpu_count() or 1))
        print(f"[bench] cpu baseline: oracle on {nb} query blocks", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(wl, x, nb)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
