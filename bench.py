"""Throughput of the block-sparse attention hot path on one MI355X.

A timed step is one pass of the prefill path on the 1.3B-shaped workload
(B=4, H=16, N=8192, D=128, bf16; window 4 blocks, stride 8, heads 0-1 dense):
s2_build_layout followed by s2_attn_fwd.  `value` is the effective forward
throughput counted over active 64x64 tiles only (4 * 64 * 64 * D flop per
tile) divided by the step time.  The decode path (64 sequences x 32 heads x
32768 context, D=128, bf16, window 8, stride 16) is timed in its own loop in
the same run and reported under "decode" as GB/s over the active K/V bytes.

Prints exactly one JSON line on stdout.  Usage:
    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import synth  # noqa: E402

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
FWD_WORKLOAD, DECODE_WORKLOAD = 2, 5


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def tile_flops(D: int) -> float:
    return 4.0 * 64 * 64 * D


def time_launches(fn, steps: int, stream):
    """Run fn `steps` times; return (total ms from events bracketing the loop, per-launch ms list)."""
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for a, b in evs:
        a.record(stream)
        fn()
        b.record(stream)
    stop.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(stop), [a.elapsed_time(b) for a, b in evs]


def cpu_baseline(q, k, v, c, budget_s: float = 20.0):
    """The fp64 oracle on a bounded sample of the forward workload (batch 0, all heads,
    query blocks strided so that the sample takes about `budget_s` seconds)."""
    import oracle
    from threadpoolctl import threadpool_info

    H, N, D, W, S = c["H"], c["N"], c["D"], c["W"], c["S"]
    nqb = N // 64
    rp, ci = oracle.build_layout(H, nqb, W, S, synth.dense_flags(H, c["dense"]))
    q0, k0, v0 = q[:1].float().numpy(), k[:1].float().numpy(), v[:1].float().numpy()
    step = 16
    t0 = time.perf_counter()
    done_tiles = 0
    blocks_done = []
    while True:
        # sweep offsets of a strided sample until the time budget is used
        off = len(blocks_done)
        if off >= step:
            break
        blocks = list(range(off, nqb, step))
        oracle.attn_fwd_blocks(q0, k0, v0, rp, ci, nqb, heads=range(H), q_blocks=blocks)
        blocks_done.append(off)
        for h in range(H):
            for i in blocks:
                r = h * nqb + i
                done_tiles += int(rp[r + 1] - rp[r])
        if time.perf_counter() - t0 > budget_s:
            break
    secs = time.perf_counter() - t0
    threads = max([x.get("num_threads", 1) for x in threadpool_info()] + [1])
    flops = done_tiles * tile_flops(D)
    return {"value": flops / secs / 1e12, "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle", "seconds": round(secs, 3),
            "sample": f"fp64 numpy oracle, batch 0, all {H} heads, query blocks i = o (mod {step}) "
                      f"for offsets o < {len(blocks_done)}: {done_tiles} active tiles "
                      f"({flops:.3e} flop)"}


def run_decode(args, s2, dev, stream):
    cd = synth.WORKLOADS[DECODE_WORKLOAD]
    Bd, Hd, L, Dd = cd["B"], cd["H"], cd["N"], cd["D"]
    log(f"decode workload {cd['name']}: filling 2 x {Bd * Hd * L * Dd * 2 / 1e9:.1f} GB caches")
    kc = synth.randn_device(synth.seed_of(DECODE_WORKLOAD, synth.TENSOR_K, 0, 0), (Bd, Hd, L, Dd),
                            cd["dtype"], dev)
    vc = synth.randn_device(synth.seed_of(DECODE_WORKLOAD, synth.TENSOR_V, 0, 0), (Bd, Hd, L, Dd),
                            cd["dtype"], dev)
    qdec = synth.decode_query(DECODE_WORKLOAD, Bd, Hd, Dd, cd["dtype"]).to(dev)
    layd = s2.s2_build_layout(s2.Pattern(Hd, cd["W"], cd["S"], cd["dense"]), L // 64, dev)
    seq = torch.full((Bd,), L, dtype=torch.int32, device=dev)
    rp = layd.row_ptr.cpu().numpy().astype(np.int64)
    i_last = (L - 1) // 64
    nqb = L // 64
    blocks = sum(int(rp[h * nqb + i_last + 1] - rp[h * nqb + i_last]) for h in range(Hd))
    kv_bytes = Bd * blocks * 64 * Dd * 2 * 2
    splits = args.splits
    ws = torch.empty(s2.s2_attn_decode_workspace(layd, Bd, Dd, splits), dtype=torch.uint8, device=dev)
    od = torch.empty((Bd, Hd, Dd), dtype=torch.bfloat16, device=dev)
    ld = torch.empty((Bd, Hd), dtype=torch.float32, device=dev)
    dec = lambda: s2.s2_attn_decode(qdec, kc, vc, seq, layd, splits=splits, workspace=ws, out=od, lse=ld)
    for _ in range(args.warmup):
        dec()
    _, dms = time_launches(dec, args.steps, stream)
    davg = float(np.mean(dms))
    gbs = kv_bytes / (davg * 1e-3) / 1e9
    log(f"decode: {davg:.4f} ms (min {min(dms):.4f}), {gbs:.1f} GB/s over active K/V")
    del kc, vc
    torch.cuda.empty_cache()
    return {
        "workload": "7B-shaped decode: 64 seqs x 1 token, context 32768, H=32 D=128 bf16, "
                    "window 8 + stride 16, split-KV + logsumexp merge",
        "ms_per_step": round(davg, 5), "value": round(gbs, 2), "unit": "GB/s",
        "active_kv_bytes": kv_bytes, "splits": splits or "auto",
        "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": None},
    }


def copy_calibration(args, dev, stream):
    """A plain device copy of 1 GiB (read 1 GiB, write 1 GiB): the reference for scaling
    the FETCH_SIZE / WRITE_SIZE counters of the attention kernels."""
    n = 1 << 29  # bf16 elements = 1 GiB
    src = torch.ones(n, dtype=torch.bfloat16, device=dev)
    dst = torch.empty_like(src)
    for _ in range(args.warmup):
        dst.copy_(src)
    _, ms = time_launches(lambda: dst.copy_(src), args.steps, stream)
    avg = float(np.mean(ms))
    log(f"copy: {avg:.4f} ms per 1 GiB copy, {2 * (1 << 30) / (avg * 1e-3) / 1e9:.1f} GB/s read+write")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--splits", type=int, default=0, help="decode splits (0 = automatic)")
    ap.add_argument("--only", choices=["fwd", "decode", "copy"], default=None,
                    help="profiling runs: time one part only and print its log line")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this library has no multi-GPU path "
              "(each GPU would run the same kernels on its own heads); run with --gpus 1",
              file=sys.stderr)
        sys.exit(2)

    import head_heterogeneous_block_amd as s2

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    if args.only == "copy":
        copy_calibration(args, dev, stream)
        return
    if args.only == "decode":
        run_decode(args, s2, dev, stream)
        return
    c = synth.WORKLOADS[FWD_WORKLOAD]
    B, H, N, D = c["B"], c["H"], c["N"], c["D"]
    log(f"fwd workload {c['name']}: generating inputs")
    q, k, v = synth.fwd_inputs(FWD_WORKLOAD, B, H, N, D, c["dtype"])
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    pat = s2.Pattern(H, c["W"], c["S"], c["dense"])
    nqb = N // 64
    lay = s2.s2_build_layout(pat, nqb, dev)
    out = torch.empty_like(qd)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    tiles = B * lay.nnz
    flops = tiles * tile_flops(D)

    def step():
        s2.s2_build_layout(pat, nqb, dev, row_ptr=lay.row_ptr, col_idx=lay.col_idx)
        s2.s2_attn_fwd(qd, kd, vd, lay, out=out, lse=lse)

    fwd_only = lambda: s2.s2_attn_fwd(qd, kd, vd, lay, out=out, lse=lse)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    total_ms, _ = time_launches(step, args.steps, stream)
    wall = time.perf_counter() - t0
    ms_step = total_ms / args.steps
    _, fwd_ms = time_launches(fwd_only, args.steps, stream)
    fwd_avg = float(np.mean(fwd_ms))
    achieved = flops / (fwd_avg * 1e-3) / 1e12
    log(f"fwd: {ms_step:.4f} ms/step (layout+fwd), fwd kernel {fwd_avg:.4f} ms "
        f"(min {min(fwd_ms):.4f}), {achieved:.1f} TFLOP/s, wall {wall:.3f} s")

    result = {
        "metric": "sparse-attn fwd effective TFLOP/s (active blocks) + decode KV GB/s, % of peak",
        "value": round(flops / (ms_step * 1e-3) / 1e12, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "1.3B-shaped prefill: B=4 H=16 N=8192 D=128 bf16, 64-token blocks, "
                               "window 4 + stride 8, heads 0-1 dense; step = s2_build_layout + s2_attn_fwd",
                   "B": B, "H": H, "N": N, "D": D, "W": c["W"], "S": c["S"],
                   "dense_heads": list(c["dense"]), "active_tiles": tiles,
                   "flop_per_step": flops},
        "roofline": {"bound": "mfma", "kernel": "fwd_bf16_kernel<128,2>",
                     "achieved": round(achieved, 3), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": None,
                     "launch_ms_avg": round(fwd_avg, 5),
                     "flop_per_launch": flops},
    }

    if args.only == "fwd":
        return
    if not args.no_decode:
        del qd, kd, vd, out, lse
        torch.cuda.empty_cache()
        result["decode"] = run_decode(args, s2, dev, stream)
    if not args.no_cpu_baseline:
        log("cpu baseline: oracle on a sample of the forward workload")
        result["cpu_baseline"] = cpu_baseline(q, k, v, c)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
