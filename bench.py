"""Throughput of the block-sparse attention hot path on one MI355X.

A timed step is one pass of the prefill path on the largest single-GPU
workload, the 7B long-context one (B=1, H=32, N=131072, D=128, bf16; window 16
blocks, stride 32, heads 0-3 dense): s2_build_layout followed by s2_attn_fwd.
`value` is the effective forward throughput counted over active 64x64 tiles
only (4 * 64 * 64 * D flop per tile) divided by the step time.  The other
workloads are timed in the same run as sub-objects: the 7B-shaped 32K prefill
("fwd_7B_32K"), the 1.3B-shaped prefill ("fwd_1.3B", with its backward and
varlen legs), the tiny fp32 forward ("fwd_tiny_f32", time only: launch-bound),
and the decode path (64 sequences x 32 heads x 32768 context, D=128, bf16,
window 8, stride 16) as GB/s over the active K/V bytes, with the serving and
query-aware decode legs beside it.

Timing: an untimed quarter second of the same work first lets the GPU clocks
leave their idle state, then W warm-up steps, then K steps back to back between
two HIP events on the launch stream.  For the forward workloads a pair of HIP
events brackets every s2_attn_fwd launch inside those K steps, so the kernel's
roofline figure comes from the same loop as the step time.

Prints exactly one JSON line on stdout.  Usage:
    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import synth  # noqa: E402

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
HEADLINE_WORKLOAD = 4       # the largest single-GPU forward workload
FWD_WORKLOAD, DECODE_WORKLOAD = 2, 5   # the backward / varlen legs use workload 2's shape
FWD_NAMES = {
    1: "tiny fp32 prefill: B=1 H=4 N=512 D=64 fp32, 64-token blocks, window 2 + stride 4, no dense heads",
    2: "1.3B-shaped prefill: B=4 H=16 N=8192 D=128 bf16, 64-token blocks, window 4 + stride 8, heads 0-1 dense",
    3: "7B-shaped prefill: B=1 H=32 N=32768 D=128 bf16, 64-token blocks, window 8 + stride 16, no dense heads",
    4: "7B long-context prefill: B=1 H=32 N=131072 D=128 bf16, 64-token blocks, window 16 + stride 32, "
       "heads 0-3 dense",
}

# HBM traffic per launch from `rocprofv3 --pmc FETCH_SIZE` and `--pmc WRITE_SIZE` runs of
# this script (profiles/ holds the summaries and commands).  The counters read a
# plain 1 GiB device copy as FETCH 512 MiB / WRITE 1 GiB, so FETCH_SIZE is scaled by
# 2 and WRITE_SIZE by 1.  A figure is used only while the kernel sources hash to the
# value recorded with it (comments excluded): after any change to the kernel code,
# "traffic" is null until it is measured again.
FETCH_SCALE, WRITE_SCALE = 2.0, 1.0
KERNEL_SOURCES = {
    "fwd": ["head_heterogeneous_block_amd/csrc/s2_fwd_bf16.hip",
            "head_heterogeneous_block_amd/csrc/s2_internal.h"],
    "decode": ["head_heterogeneous_block_amd/csrc/s2_decode.hip",
               "head_heterogeneous_block_amd/csrc/s2_decode_common.h",
               "head_heterogeneous_block_amd/csrc/s2_internal.h"],
    "paged": ["head_heterogeneous_block_amd/csrc/s2_decode_paged.hip",
              "head_heterogeneous_block_amd/csrc/s2_decode_common.h",
              "head_heterogeneous_block_amd/csrc/s2_internal.h"],
    "bwd": ["head_heterogeneous_block_amd/csrc/s2_bwd_bf16.hip",
            "head_heterogeneous_block_amd/csrc/s2_internal.h"],
}
KERNEL_SOURCES["varlen"] = KERNEL_SOURCES["fwd"]   # the same kernel, its varlen instantiation
KERNEL_SOURCES["select"] = ["head_heterogeneous_block_amd/csrc/s2_select.hip"] + KERNEL_SOURCES["decode"]
KERNEL_SOURCES["select_paged"] = ["head_heterogeneous_block_amd/csrc/s2_select.hip"] + KERNEL_SOURCES["paged"]
MEASURED_TRAFFIC = {
    # part: (sources_hash(part), FETCH_SIZE KiB, WRITE_SIZE KiB per launch; for bwd the sum over the
    # three kernels of one s2_attn_bwd call, for select / select_paged over the launches of one step).
    # "fwd:w" is the forward kernel on workload w.
    "fwd:4": ('882d55ad4013', 9879107.9, 1066353.6),
    "fwd:3": ('882d55ad4013', 491651.0, 266751.0),
    "fwd:2": ('882d55ad4013', 228522.0, 133515.6),
    "varlen:2": ('882d55ad4013', 257135.2, 133805.3),
    "bwd": ('fda6ff183b2e', 2246439.9, 405294.9),
    "decode": ('56d98b74cc5a', 1294648.9, 579.4),
    "paged": ('c74d427d55de', 1148634.3, 528.0),
    "select": ('4a9b1c8481ec', 1573423.2, 1026.2),
    "select_paged": ('26537a45594c', 1075080.9, 3040.5),
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def tile_flops(D: int) -> float:
    return 4.0 * 64 * 64 * D


def sources_hash(part: str) -> str:
    """Hash of the part's kernel code: comments and blank lines do not count."""
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[part]:
        with open(os.path.join(ROOT, rel)) as f:
            text = re.sub(r"/\*.*?\*/", "", f.read(), flags=re.S)
        for line in text.splitlines():
            line = line.split("//", 1)[0].rstrip()
            if line.strip():
                h.update(line.encode() + b"\n")
    return h.hexdigest()[:12]


def measured_traffic(part: str):
    """HBM bytes per launch of the part's dominant kernel, or None (not measured for
    the current sources)."""
    rec = MEASURED_TRAFFIC.get(part)
    if rec is None or rec[0] != sources_hash(part.split(":")[0]):
        return None
    return int(round(rec[1] * 1024 * FETCH_SCALE + rec[2] * 1024 * WRITE_SCALE))


def time_loop(fn, steps: int, stream) -> float:
    """Run fn `steps` times back to back between two HIP events recorded on the stream
    the kernels are launched on; return the elapsed ms.  No event sits between the
    launches, so the mean per call is the kernels' own duration plus dispatch gaps."""
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for _ in range(steps):
        fn()
    stop.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(stop)


def time_steps_bracketed(pre, fn, steps: int, stream):
    """K steps of pre() then fn() back to back between two HIP events on the launch
    stream, with a further event pair around every fn() call.  Returns (total ms of the
    K steps, mean ms of fn alone).  The inner events sit between launches on the same
    stream, so they time exactly the kernels fn enqueues."""
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for a, b in ev:
        pre()
        a.record(stream)
        fn()
        b.record(stream)
    stop.record(stream)
    torch.cuda.synchronize()
    inner = sum(a.elapsed_time(b) for a, b in ev) / steps
    return start.elapsed_time(stop), inner


def settle_clocks(fn, stream, seconds: float = 0.25):
    """Untimed: keep the GPU busy with fn for about `seconds` so that its clocks have
    left their idle state before warm-up and timing (the first ~40 launches after
    idle run up to 15% slower)."""
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(20):
            fn()
        torch.cuda.synchronize()


def blas_threads() -> int:
    from threadpoolctl import threadpool_info
    return int(max([x.get("num_threads", 1) for x in threadpool_info()] + [1]))


def cpu_baseline(q, k, v, c, budget_s: float = 20.0, step: int = 16):
    """The fp64 oracle on a bounded sample of a forward workload: batch by batch, all
    heads, query blocks i = o (mod step) for offsets o = 0, 1, ..., until about `budget_s`
    seconds have passed or the whole workload is done.  q, k, v: CPU tensors."""
    import oracle

    B, H, N, D, W, S = c["B"], c["H"], c["N"], c["D"], c["W"], c["S"]
    nqb = N // 64
    rp, ci = oracle.build_layout(H, nqb, W, S, synth.dense_flags(H, c["dense"]))
    tiles_per_off = [sum(int(rp[h * nqb + i + 1] - rp[h * nqb + i])
                         for h in range(H) for i in range(off, nqb, step)) for off in range(step)]
    t0 = time.perf_counter()
    done_tiles = done_units = 0
    for b in range(B):
        q0, k0, v0 = (x[b:b + 1].float().numpy() for x in (q, k, v))
        for off in range(step):
            oracle.attn_fwd_blocks(q0, k0, v0, rp, ci, nqb, heads=range(H),
                                   q_blocks=list(range(off, nqb, step)))
            done_tiles += tiles_per_off[off]
            done_units += 1
            if time.perf_counter() - t0 > budget_s:
                break
        if time.perf_counter() - t0 > budget_s:
            break
    secs = time.perf_counter() - t0
    flops = done_tiles * tile_flops(D)
    return {"value": flops / secs / 1e12, "unit": "TFLOP/s", "cores": blas_threads(),
            "kind": "oracle", "seconds": round(secs, 3),
            "sample": f"fp64 numpy oracle, all {H} heads, query blocks i = o (mod {step}); "
                      f"{done_units} of {B * step} (batch, offset o) slices in order, "
                      f"{done_tiles} active tiles ({flops:.3e} flop)"}


def cpu_baseline_decode(kc, vc, q, seq_lens, rp, ci, nqb, pairs, budget_s: float = 15.0):
    """The fp64 oracle's decode on a sample of (sequence, head) pairs of the decode
    workload.  The active K/V blocks of the sampled pairs are copied to the host first
    (not timed); then oracle.attn_decode runs pair by pair until about `budget_s` seconds
    have passed.  Reported as GB/s over the active K/V bytes of the pairs done."""
    import oracle

    L, D = kc.shape[2], kc.shape[3]
    host = {}
    for b, h in pairs:
        i = (int(seq_lens[b]) - 1) // 64
        js = [int(j) for j in ci[rp[h * nqb + i]:rp[h * nqb + i + 1]]]
        idx = torch.tensor(js, device=kc.device)
        # the row's active blocks gathered on the device, one copy to the host per tensor
        kb = kc[b, h].view(-1, 64, D).index_select(0, idx).float().cpu().numpy()
        vb = vc[b, h].view(-1, 64, D).index_select(0, idx).float().cpu().numpy()
        for n, j in enumerate(js):
            host[(b, h, j)] = (kb[n], vb[n])
    qh = q.float().cpu().numpy()
    t0 = time.perf_counter()
    done = nbytes = 0
    for b, h in pairs:
        oracle.attn_decode(qh, lambda bb, hh, jj: host[(bb, hh, jj)], seq_lens, rp, ci, nqb, pairs=[(b, h)],
                           cache_len=L)
        i = (int(seq_lens[b]) - 1) // 64
        nbytes += int(rp[h * nqb + i + 1] - rp[h * nqb + i]) * 64 * kc.shape[3] * kc.element_size() * 2
        done += 1
        if time.perf_counter() - t0 > budget_s:
            break
    secs = time.perf_counter() - t0
    return {"value": nbytes / secs / 1e9, "unit": "GB/s", "cores": blas_threads(), "kind": "oracle",
            "seconds": round(secs, 3),
            "sample": f"fp64 numpy oracle decode, {done} of the {len(pairs)} sampled (sequence, head) pairs "
                      f"(sequences 0-{max(b for b, _ in pairs)}, all heads), {nbytes} bytes of active K/V "
                      f"(the bf16 bytes the GPU reads for them)"}


SELECT_BUDGET = 40  # blocks per (sequence, head): about the static pattern's 39.5 at this context


def run_select(args, s2, dev, stream, kc, vc, q, seq, static_row):
    """Query-aware decode on the decode workload's caches: per-block key bounds
    (built once per cache, timed apart), then per step the top-budget block lists
    and decode over them."""
    Bd, Hd, L, Dd = kc.shape
    nb = L // 64
    kmin = torch.empty((Bd, Hd, nb, Dd), dtype=kc.dtype, device=dev)
    kmax = torch.empty_like(kmin)

    def meta():
        s2.s2_block_minmax(kc, seq, kmin=kmin, kmax=kmax)
    settle_clocks(meta, stream)
    for _ in range(max(1, args.warmup // 4)):
        meta()
    msteps = max(3, args.steps // 10)
    mavg = time_loop(meta, msteps, stream) / msteps
    key_bytes = Bd * Hd * L * Dd * kc.element_size()
    od = torch.empty((Bd, Hd, Dd), dtype=kc.dtype, device=dev)
    ld = torch.empty((Bd, Hd), dtype=torch.float32, device=dev)
    step = s2.PreparedSelectDecode(q, kc, vc, seq, kmin, kmax, SELECT_BUDGET, od, ld, splits=args.splits)
    settle_clocks(step, stream)
    for _ in range(args.warmup):
        step()
    savg = time_loop(step, args.steps, stream) / args.steps
    # the two launches alone, back to back (selection rewrites the same rows every call)
    lib, sel_args, dec_args = step._lib, step._sel, step._dec
    st = stream.cuda_stream
    check = s2.s2attn._check
    sel_only = lambda: check(lib.s2_select_blocks(*sel_args, st))
    dec_only = lambda: check(lib.s2_attn_decode_rows(*dec_args, st))
    sel_avg = time_loop(sel_only, args.steps, stream) / args.steps
    dec_avg = time_loop(dec_only, args.steps, stream) / args.steps
    i_last = (L - 1) // 64
    meta_bytes = Bd * Hd * i_last * 2 * Dd * kc.element_size()       # bounds of the blocks before the query's
    kv_bytes = Bd * Hd * SELECT_BUDGET * 64 * Dd * kc.element_size() * 2
    step_bytes = meta_bytes + kv_bytes
    gbs = step_bytes / (savg * 1e-3) / 1e9
    log(f"select decode: bounds build {mavg:.4f} ms ({key_bytes / (mavg * 1e-3) / 1e9:.1f} GB/s over the keys); "
        f"step {savg:.4f} ms = select {sel_avg:.4f} + decode {dec_avg:.4f}, {gbs:.1f} GB/s")
    return {
        "workload": f"7B-shaped query-aware decode: 64 seqs x 1 token, context 32768, H=32 D=128 bf16, "
                    f"per-block key bounds, the query's block + the {SELECT_BUDGET - 1} highest-bounded earlier "
                    f"blocks per (sequence, head); step = s2_select_blocks + s2_attn_decode_rows",
        "ms_per_step": round(savg, 5), "value": round(gbs, 2), "unit": "GB/s",
        "budget_blocks": SELECT_BUDGET, "static_pattern_mean_row": round(float(static_row), 2),
        "bytes_per_step": step_bytes, "bound_bytes": meta_bytes, "kv_bytes": kv_bytes,
        "select_ms": round(sel_avg, 5), "decode_ms": round(dec_avg, 5),
        "bounds_build_ms": round(mavg, 5), "bounds_build_gbs": round(key_bytes / (mavg * 1e-3) / 1e9, 2),
        "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(gbs / PEAK_HBM_GBS, 4),
                     "traffic": measured_traffic("select"), "traffic_unit": "bytes/step",
                     "sources": sources_hash("select")},
    }


def run_decode(args, s2, dev, stream, parts=("decode", "select")):
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
    sel = run_select(args, s2, dev, stream, kc, vc, qdec, seq, blocks / Hd) if "select" in parts else None
    if "decode" not in parts:
        del kc, vc
        torch.cuda.empty_cache()
        return None, sel
    ws = torch.empty(s2.s2_attn_decode_workspace(layd, Bd, Dd, splits), dtype=torch.uint8, device=dev)
    od = torch.empty((Bd, Hd, Dd), dtype=torch.bfloat16, device=dev)
    ld = torch.empty((Bd, Hd), dtype=torch.float32, device=dev)
    dec = s2.PreparedDecode(qdec, kc, vc, seq, layd, od, ld, ws, splits=splits)
    settle_clocks(dec, stream)
    for _ in range(args.warmup):
        dec()
    davg = time_loop(dec, args.steps, stream) / args.steps
    gbs = kv_bytes / (davg * 1e-3) / 1e9
    log(f"decode: {davg:.4f} ms per launch, {gbs:.1f} GB/s over active K/V")
    cpu = None
    if not args.no_cpu_baseline:
        log("cpu baseline: oracle decode on a sample of (sequence, head) pairs")
        ci = layd.col_idx.cpu().numpy()
        seq_h = [L] * Bd
        pairs = [(b, h) for b in range(Bd) for h in range(Hd)]   # the whole workload
        cpu = cpu_baseline_decode(kc, vc, qdec, seq_h, rp, ci, nqb, pairs)
    del kc, vc
    torch.cuda.empty_cache()
    res = {
        "workload": "7B-shaped decode: 64 seqs x 1 token, context 32768, H=32 D=128 bf16, "
                    "window 8 + stride 16, split-KV + logsumexp merge",
        "ms_per_step": round(davg, 5), "value": round(gbs, 2), "unit": "GB/s",
        "active_kv_bytes": kv_bytes, "splits": splits or "auto",
        "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
                     "traffic": measured_traffic("decode"), "traffic_unit": "bytes/launch",
                     "bytes_per_launch": kv_bytes, "sources": sources_hash("decode")},
    }
    if cpu is not None:
        res["cpu_baseline"] = cpu
    return res, sel


PAGED_KV_HEADS, PAGE_SIZE = 8, 16
VARLEN_LENS = [8192, 5000, 3000, 1, 12000, 4511, 64]  # 32768 tokens, as the prefill batch


def run_varlen(args, s2, dev, stream):
    """Packed variable-length prefill: the prefill workload's 32768 tokens as seven
    ragged sequences, its heads, head size and pattern."""
    c = synth.WORKLOADS[FWD_WORKLOAD]
    H, D = c["H"], c["D"]
    cu = torch.tensor([0] + np.cumsum(VARLEN_LENS).tolist(), dtype=torch.int32)
    T = int(cu[-1])
    nqb = -(-max(VARLEN_LENS) // 64)
    lay = s2.s2_build_layout(s2.Pattern(H, c["W"], c["S"], c["dense"]), nqb, dev)
    rp = lay.row_ptr.cpu().numpy().astype(np.int64)
    # active tiles: every sequence reads its own rows 0 .. ceil(len / 64) - 1 (a partial
    # last block counts as a whole tile)
    tiles = 0
    for n in VARLEN_LENS:
        nb = -(-n // 64)
        tiles += sum(int(rp[h * nqb + nb] - rp[h * nqb]) for h in range(H))
    flops = tiles * tile_flops(D)
    q, k, v = (synth.randn_device(synth.seed_of(FWD_WORKLOAD, t, 9, 0), (T, H, D), c["dtype"], dev)
               for t in (synth.TENSOR_Q, synth.TENSOR_K, synth.TENSOR_V))
    out = torch.empty_like(q)
    lse = torch.empty((H, T), dtype=torch.float32, device=dev)
    f = s2.PreparedFwdVarlen(q, k, v, cu.to(dev), lay, out, lse)
    settle_clocks(f, stream)
    for _ in range(args.warmup):
        f()
    avg = time_loop(f, args.steps, stream) / args.steps
    achieved = flops / (avg * 1e-3) / 1e12
    log(f"varlen: {avg:.4f} ms per launch, {achieved:.1f} TFLOP/s")
    return {
        "workload": "1.3B-shaped varlen prefill: 32768 tokens in 7 sequences " + str(VARLEN_LENS) +
                    ", H=16 D=128 bf16, window 4 + stride 8, heads 0-1 dense",
        "ms_per_step": round(avg, 5), "value": round(achieved, 3), "unit": "TFLOP/s",
        "active_tiles": tiles, "flop_per_launch": flops,
        "roofline": {"bound": "mfma", "kernel": "fwd_bf16_kernel<128,2,2,varlen>",
                     "achieved": round(achieved, 3), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": measured_traffic("varlen:2"), "traffic_unit": "bytes/launch",
                     "sources": sources_hash("varlen"), "launch_ms_avg": round(avg, 5)},
    }


def run_select_paged(args, s2, dev, stream, kp, vp, table, q, seq):
    """Query-aware serving decode on the paged pools: per-block key bounds per K/V
    head through the block tables (once per cache, timed apart), then per step each
    query head's top-budget lists and the paged decode over them."""
    Bd, Hd, Dd = q.shape
    Hkv, P = kp.shape[1], kp.shape[2]
    L = table.shape[1] * P
    nb = L // 64
    kmin = torch.empty((Bd, Hkv, nb, Dd), dtype=kp.dtype, device=dev)
    kmax = torch.empty_like(kmin)

    def meta():
        s2.s2_block_minmax_paged(kp, table, seq, nb, kmin=kmin, kmax=kmax)
    settle_clocks(meta, stream)
    msteps = max(3, args.steps // 10)
    mavg = time_loop(meta, msteps, stream) / msteps
    od = torch.empty((Bd, Hd, Dd), dtype=kp.dtype, device=dev)
    ld = torch.empty((Bd, Hd), dtype=torch.float32, device=dev)
    step = s2.PreparedSelectDecodePaged(q, kp, vp, table, seq, kmin, kmax, SELECT_BUDGET, od, ld,
                                        splits=args.splits)
    settle_clocks(step, stream)
    for _ in range(args.warmup):
        step()
    savg = time_loop(step, args.steps, stream) / args.steps
    lib, sel_args, dec_args = step._lib, step._sel, step._dec
    st, check = stream.cuda_stream, s2.s2attn._check
    sel_avg = time_loop(lambda: check(lib.s2_select_blocks(*sel_args, st)), args.steps, stream) / args.steps
    dec_avg = time_loop(lambda: check(lib.s2_attn_decode_paged_rows(*dec_args, st)), args.steps, stream) / args.steps
    # unique bytes: each K/V head's bounds of the blocks before the query's, and per
    # (sequence, K/V head) the union of its query heads' lists
    rp, ci = step.row_ptr.cpu().numpy(), step.col_idx.cpu().numpy()
    g = Hd // Hkv
    union = 0
    for b in range(Bd):
        for kh in range(Hkv):
            r0 = b * Hd + kh * g
            union += len(set(ci[rp[r0]:rp[r0 + g]].tolist()))
    elt = kp.element_size()
    bound_bytes = Bd * Hkv * ((L - 1) // 64) * 2 * Dd * elt
    kv_bytes = union * 64 * Dd * elt * 2
    gbs = (bound_bytes + kv_bytes) / (savg * 1e-3) / 1e9
    key_bytes = Bd * Hkv * L * Dd * elt
    log(f"paged select decode: bounds build {mavg:.4f} ms ({key_bytes / (mavg * 1e-3) / 1e9:.1f} GB/s); "
        f"step {savg:.4f} ms = select {sel_avg:.4f} + decode {dec_avg:.4f}, {gbs:.1f} GB/s over unique bytes")
    return {
        "workload": f"7B-shaped query-aware serving decode: 64 seqs x 1 token, context 32768, H=32 over {Hkv} K/V "
                    f"heads, D=128 bf16, {P}-token pages; per-K/V-head block key bounds, each query head's block + "
                    f"its {SELECT_BUDGET - 1} highest-bounded earlier blocks; "
                    f"step = s2_select_blocks + s2_attn_decode_paged_rows",
        "ms_per_step": round(savg, 5), "value": round(gbs, 2), "unit": "GB/s",
        "budget_blocks": SELECT_BUDGET, "bytes_per_step": bound_bytes + kv_bytes, "bound_bytes": bound_bytes,
        "unique_kv_bytes": kv_bytes, "select_ms": round(sel_avg, 5), "decode_ms": round(dec_avg, 5),
        "bounds_build_ms": round(mavg, 5), "bounds_build_gbs": round(key_bytes / (mavg * 1e-3) / 1e9, 2),
        "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(gbs / PEAK_HBM_GBS, 4),
                     "traffic": measured_traffic("select_paged"), "traffic_unit": "bytes/step",
                     "sources": sources_hash("select_paged")},
    }


def run_decode_paged(args, s2, dev, stream, parts=("paged", "select_paged")):
    """Serving decode: the decode workload's sequences, heads and pattern with 8 K/V
    heads (groups of 4 query heads) in a pool of 16-token pages, shuffled."""
    cd = synth.WORKLOADS[DECODE_WORKLOAD]
    Bd, Hd, L, Dd = cd["B"], cd["H"], cd["N"], cd["D"]
    Hkv, P = PAGED_KV_HEADS, PAGE_SIZE
    npb = L // P
    n = Bd * npb
    log(f"paged decode: filling 2 x {n * Hkv * P * Dd * 2 / 1e9:.1f} GB page pools")
    kp = synth.randn_device(synth.seed_of(DECODE_WORKLOAD, synth.TENSOR_K, 1, 0), (n, Hkv, P, Dd),
                            cd["dtype"], dev)
    vp = synth.randn_device(synth.seed_of(DECODE_WORKLOAD, synth.TENSOR_V, 1, 0), (n, Hkv, P, Dd),
                            cd["dtype"], dev)
    gen = torch.Generator().manual_seed(synth.seed_of(DECODE_WORKLOAD, 9, 0, 0))
    table = torch.randperm(n, generator=gen).to(torch.int32).view(Bd, npb).to(dev)
    qdec = synth.decode_query(DECODE_WORKLOAD, Bd, Hd, Dd, cd["dtype"]).to(dev)
    layd = s2.s2_build_layout(s2.Pattern(Hd, cd["W"], cd["S"], cd["dense"]), L // 64, dev)
    seq = torch.full((Bd,), L, dtype=torch.int32, device=dev)
    sel = run_select_paged(args, s2, dev, stream, kp, vp, table, qdec, seq) if "select_paged" in parts else None
    if "paged" not in parts:
        del kp, vp
        torch.cuda.empty_cache()
        return None, sel
    # unique K/V bytes: per (sequence, K/V head) the union of its query heads' blocks
    rp = layd.row_ptr.cpu().numpy().astype(np.int64)
    ci = layd.col_idx.cpu().numpy()
    nqb, i_last, g = L // 64, (L - 1) // 64, Hd // Hkv
    rows = [set(ci[rp[h * nqb + i_last]:rp[h * nqb + i_last + 1]].tolist()) for h in range(Hd)]
    union_blocks = sum(len(set().union(*rows[k * g:(k + 1) * g])) for k in range(Hkv))
    per_head_blocks = sum(len(r) for r in rows)
    blk = 64 * Dd * 2 * 2
    kv_bytes = Bd * union_blocks * blk
    ws = torch.empty(s2.s2_attn_decode_paged_workspace(layd, Bd, Hkv, Dd, args.splits), dtype=torch.uint8,
                     device=dev)
    od = torch.empty((Bd, Hd, Dd), dtype=torch.bfloat16, device=dev)
    ld = torch.empty((Bd, Hd), dtype=torch.float32, device=dev)
    dec = s2.PreparedDecodePaged(qdec, kp, vp, table, seq, layd, od, ld, ws if ws.numel() else None,
                                 splits=args.splits)
    settle_clocks(dec, stream)
    for _ in range(args.warmup):
        dec()
    davg = time_loop(dec, args.steps, stream) / args.steps
    gbs = kv_bytes / (davg * 1e-3) / 1e9
    log(f"paged decode: {davg:.4f} ms per launch, {gbs:.1f} GB/s over unique active K/V")
    del kp, vp
    torch.cuda.empty_cache()
    res = {
        "workload": f"7B-shaped serving decode: 64 seqs x 1 token, context 32768, H=32 over {Hkv} K/V "
                    f"heads, D=128 bf16, window 8 + stride 16, {P}-token pages in a shuffled pool",
        "ms_per_step": round(davg, 5), "value": round(gbs, 2), "unit": "GB/s",
        "unique_kv_bytes": kv_bytes, "per_query_head_kv_bytes": Bd * per_head_blocks * blk,
        "splits": args.splits or "auto",
        "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
                     "traffic": measured_traffic("paged"), "traffic_unit": "bytes/launch",
                     "bytes_per_launch": kv_bytes, "sources": sources_hash("paged")},
    }
    return res, sel


def run_bwd(args, s2, dev, stream, qd, kd, vd, c):
    """The backward pass on the forward workload: s2_attn_bwd (plans, dQ with delta, dK/dV
    launches) with the forward's output and logsumexp, dO iid N(0,1)."""
    B, H, N, D = c["B"], c["H"], c["N"], c["D"]
    pat = s2.Pattern(H, c["W"], c["S"], c["dense"])
    nqb = N // 64
    lay = s2.s2_build_layout(pat, nqb, dev)
    lt = s2.s2_build_layout_t(pat, nqb, dev)
    o, lse = s2.s2_attn_fwd(qd, kd, vd, lay)
    dout = synth.randn_device(synth.seed_of(FWD_WORKLOAD, synth.TENSOR_DO, 0, 0), (B, H, N, D), "bf16", dev)
    dq, dk, dv = (torch.empty_like(qd) for _ in range(3))
    ws = torch.empty(s2.s2_attn_bwd_workspace(B, H, N), dtype=torch.uint8, device=dev)
    bwd = s2.PreparedBwd(qd, kd, vd, o, dout, lse, lay, lt, dq, dk, dv, ws)
    settle_clocks(bwd, stream)
    for _ in range(args.warmup):
        bwd()
    avg = time_loop(bwd, args.steps, stream) / args.steps
    tiles = B * lay.nnz
    # five 64x64xD products per active tile (S recomputed, dP, dV, dQ, dK): 2.5x the forward's
    flops = tiles * 2.5 * tile_flops(D)
    achieved = flops / (avg * 1e-3) / 1e12
    log(f"bwd: {avg:.4f} ms per call (plans + dQ + dK/dV), {achieved:.1f} TFLOP/s")
    return {
        "workload": "1.3B-shaped training backward: B=4 H=16 N=8192 D=128 bf16, window 4 + stride 8, "
                    "heads 0-1 dense; dQ, dK, dV from the forward's O and logsumexp",
        "ms_per_step": round(avg, 5), "value": round(achieved, 3), "unit": "TFLOP/s",
        "flop_per_call": flops, "flop_convention": "5 products of 64x64xD per active tile",
        "roofline": {"bound": "mfma", "kernel": "bwd_plan + bwd_dq + bwd_dkdv (one s2_attn_bwd call)",
                     "achieved": round(achieved, 3), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": measured_traffic("bwd"), "traffic_unit": "bytes/call",
                     "sources": sources_hash("bwd"), "launch_ms_avg": round(avg, 5)},
    }


def gemm_reference(dev, stream, n: int = 16384, reps: int = 8):
    """The practical bf16 matrix-core rate of this GPU under sustained load: a
    square bf16 GEMM through torch.matmul (the vendor's hipBLASLt kernels).  A
    reference beside the 2.5 PFLOP/s nominal peak, not a part of the path."""
    a = torch.randn(n, n, device=dev, dtype=torch.bfloat16)
    b = torch.randn(n, n, device=dev, dtype=torch.bfloat16)
    for _ in range(3):
        c = a @ b
    avg = time_loop(lambda: torch.matmul(a, b, out=c), reps, stream) / reps
    tf = 2.0 * n ** 3 / (avg * 1e-3) / 1e12
    log(f"gemm reference: bf16 {n}^3 in {avg:.3f} ms, {tf:.1f} TFLOP/s")
    del a, b, c
    torch.cuda.empty_cache()
    return {"kernel": f"torch.matmul bf16 {n}x{n}x{n} (hipBLASLt)", "value": round(tf, 1), "unit": "TFLOP/s",
            "ms": round(avg, 4), "frac_of_2.5_pflops": round(tf / 2500.0, 4)}


def copy_calibration(args, dev, stream):
    """A plain device copy of 1 GiB (read 1 GiB, write 1 GiB): the reference for scaling
    the FETCH_SIZE / WRITE_SIZE counters of the attention kernels."""
    n = 1 << 29  # bf16 elements = 1 GiB
    src = torch.ones(n, dtype=torch.bfloat16, device=dev)
    dst = torch.empty_like(src)
    for _ in range(args.warmup):
        dst.copy_(src)
    avg = time_loop(lambda: dst.copy_(src), args.steps, stream) / args.steps
    log(f"copy: {avg:.4f} ms per 1 GiB copy, {2 * (1 << 30) / (avg * 1e-3) / 1e9:.1f} GB/s read+write")


def fwd_inputs_device(w, dev):
    """Seeded iid N(0, 1) Q, K, V of workload w generated on the device (bulk inputs)."""
    c = synth.WORKLOADS[w]
    shape = (c["B"], c["H"], c["N"], c["D"])
    return [synth.randn_device(synth.seed_of(w, t, 0, 0), shape, c["dtype"], dev)
            for t in (synth.TENSOR_Q, synth.TENSOR_K, synth.TENSOR_V)]


def run_fwd(args, s2, dev, stream, w, q=None, k=None, v=None, cpu=None):
    """Prefill on workload w: a step is s2_build_layout + s2_attn_fwd.  Returns the
    result dict (value = active-tile flop / step time) with the forward kernel's
    roofline from event pairs around its launches in the same loop."""
    c = synth.WORKLOADS[w]
    B, H, N, D = c["B"], c["H"], c["N"], c["D"]
    if q is None:
        log(f"fwd workload {c['name']}: generating inputs on the device")
        q, k, v = fwd_inputs_device(w, dev)
    pat = s2.Pattern(H, c["W"], c["S"], c["dense"])
    nqb = N // 64
    lay = s2.s2_build_layout(pat, nqb, dev)
    out = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    tiles = B * lay.nnz
    flops = tiles * tile_flops(D)
    build = s2.PreparedLayout(pat, nqb, lay)
    fwd = s2.PreparedFwd(q, k, v, lay, out, lse)

    def step():
        build()
        fwd()

    settle_clocks(step, stream)
    steps = args.steps
    for _ in range(args.warmup):
        step()
    t0 = time.perf_counter()
    total_ms, fwd_ms = time_steps_bracketed(build, fwd, steps, stream)
    wall = time.perf_counter() - t0
    ms_step = total_ms / steps
    value = flops / (ms_step * 1e-3) / 1e12
    achieved = flops / (fwd_ms * 1e-3) / 1e12
    log(f"fwd w{w}: {ms_step:.4f} ms/step (layout+fwd), fwd kernel {fwd_ms:.4f} ms per launch, "
        f"{achieved:.1f} TFLOP/s, wall {wall:.3f} s over {steps} steps")
    bf16 = c["dtype"] == "bf16"
    kernel = f"fwd_bf16_kernel<{D},2,{2 if D == 128 else 3}>" if bf16 else f"fwd_f32_kernel<{D}>"
    res = {
        "workload": FWD_NAMES[w] + "; step = s2_build_layout + s2_attn_fwd",
        "value": round(value, 3), "unit": "TFLOP/s", "steps": steps, "ms_per_step": round(ms_step, 5),
        "B": B, "H": H, "N": N, "D": D, "W": c["W"], "S": c["S"], "dense_heads": list(c["dense"]),
        "active_tiles": tiles, "flop_per_step": flops,
        "roofline": {"bound": "mfma" if bf16 else "alu", "kernel": kernel,
                     "achieved": round(achieved, 3), "peak": PEAK_BF16_TFLOPS if bf16 else 157.3,
                     "unit": "TFLOP/s", "frac": round(achieved / (PEAK_BF16_TFLOPS if bf16 else 157.3), 4),
                     "traffic": measured_traffic(f"fwd:{w}") if bf16 else None, "traffic_unit": "bytes/launch",
                     "sources": sources_hash("fwd"), "launch_ms_avg": round(fwd_ms, 5),
                     "flop_per_launch": flops},
    }
    if cpu is not None:
        log(f"cpu baseline: oracle on a sample of workload {w}")
        res["cpu_baseline"] = cpu_baseline(q.cpu(), k.cpu(), v.cpu(), c, **cpu)
    return res


def run_tiny(args, s2, dev, stream):
    """The tiny fp32 workload: launch-bound, reported as time per step."""
    r = run_fwd(args, s2, dev, stream, 1)
    r["note"] = "launch-bound parity workload: reported as time; the fp32 path runs on the vector ALU"
    return r


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-bwd", action="store_true")
    ap.add_argument("--no-paged", action="store_true")
    ap.add_argument("--no-varlen", action="store_true")
    ap.add_argument("--no-select", action="store_true")
    ap.add_argument("--splits", type=int, default=0, help="decode splits (0 = automatic)")
    ap.add_argument("--only", choices=["fwd", "bwd", "varlen", "decode", "select", "paged", "select_paged", "copy",
                                       "gemm"],
                    default=None,
                    help="profiling runs: time one part only and print its log line")
    ap.add_argument("--workload", type=int, choices=[1, 2, 3, 4], default=HEADLINE_WORKLOAD,
                    help="with --only fwd: the forward workload to time")
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
    if args.only == "gemm":
        gemm_reference(dev, stream)
        return
    if args.only == "decode":
        args.no_cpu_baseline = True
        run_decode(args, s2, dev, stream, parts=("decode",))
        return
    if args.only == "select":
        run_decode(args, s2, dev, stream, parts=("select",))
        return
    if args.only == "paged":
        run_decode_paged(args, s2, dev, stream, parts=("paged",))
        return
    if args.only == "select_paged":
        run_decode_paged(args, s2, dev, stream, parts=("select_paged",))
        return
    if args.only == "varlen":
        run_varlen(args, s2, dev, stream)
        return
    if args.only == "fwd":
        run_fwd(args, s2, dev, stream, args.workload)
        return
    cpu = not args.no_cpu_baseline
    if args.only is None:
        head = run_fwd(args, s2, dev, stream, HEADLINE_WORKLOAD,
                       cpu=dict(budget_s=20.0, step=128) if cpu else None)
        torch.cuda.empty_cache()
        result = {
            "metric": "sparse-attn fwd effective TFLOP/s (active blocks) + decode KV GB/s, % of peak",
            "value": head["value"], "unit": "TFLOP/s",
            "n_gpus": 1, "steps": head["steps"], "warmup": args.warmup,
            "ms_per_step": head["ms_per_step"],
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
            "dtype": "bf16", "data": "synthetic",
            "config": {"workload": head["workload"],
                       **{key: head[key] for key in ("B", "H", "N", "D", "W", "S", "dense_heads",
                                                     "active_tiles", "flop_per_step")}},
            "roofline": head["roofline"],
        }
        if "cpu_baseline" in head:
            result["cpu_baseline"] = head["cpu_baseline"]
        result["fwd_7B_32K"] = run_fwd(args, s2, dev, stream, 3)
        torch.cuda.empty_cache()
        result["fwd_tiny_f32"] = run_tiny(args, s2, dev, stream)
        result["gemm_reference"] = gemm_reference(dev, stream)
        result["gemm_reference"]["headline_fwd_frac_of_gemm"] = round(head["roofline"]["achieved"] /
                                                                      result["gemm_reference"]["value"], 4)
    c = synth.WORKLOADS[FWD_WORKLOAD]
    B, H, N, D = c["B"], c["H"], c["N"], c["D"]
    log(f"fwd workload {c['name']}: generating inputs")
    q, k, v = synth.fwd_inputs(FWD_WORKLOAD, B, H, N, D, c["dtype"])
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    if args.only == "bwd":
        run_bwd(args, s2, dev, stream, qd, kd, vd, c)
        return
    result["fwd_1.3B"] = run_fwd(args, s2, dev, stream, FWD_WORKLOAD, qd, kd, vd,
                                 cpu=dict(budget_s=20.0, step=16) if cpu else None)
    if not args.no_bwd:
        result["bwd"] = run_bwd(args, s2, dev, stream, qd, kd, vd, c)
    if not args.no_varlen:
        result["fwd_varlen"] = run_varlen(args, s2, dev, stream)
    if not args.no_decode:
        del qd, kd, vd
        torch.cuda.empty_cache()
        result["decode"], sel = run_decode(args, s2, dev, stream,
                                           parts=("decode",) if args.no_select else ("decode", "select"))
        if sel is not None:
            result["decode_select"] = sel
    if not args.no_paged:
        result["decode_paged"], selp = run_decode_paged(
            args, s2, dev, stream, parts=("paged",) if args.no_select else ("paged", "select_paged"))
        if selp is not None:
            result["decode_select_paged"] = selp
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
