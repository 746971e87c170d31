"""Benchmark of the row-parallel matmul + reduce hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload prefill|decode|long_prefill]

One step is one pass of the whole path for one tensor-parallel rank, on
synthetic inputs already resident in HBM:
  1. rpl_partial               the rank's bf16 partial over its K-shard, all
                               M tokens, written as reduce-scatter chunks;
  2. rpl_w8a8_partial          the w8a8 (int8) partial of the same shape
                               (skipped for workloads without a w8a8 variant);
  3. rpl_reduce_chunk_rmsnorm  the received chunk: own chunk partial + the
                               peers' chunk partials (arrived data, produced
                               before timing) -> residual add -> RMSNorm.
The default workload is the 7B-class prefill down_proj share (M=4096,
K_full=18944 over TP=2, N=3584) with its w8a8 twin.  The JSON line reports the
step's algorithmic tera-ops per second (bf16 FLOP + int8 OP), per-kernel
times from HIP events on the launch stream, the roofline of the dominant
kernel, and the CPU oracle timed on a bounded sample of the same work.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "TFLOP/s and % of MFMA peak (prefill); HBM GB/s % peak (decode)"
PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA: 256 CU x 2.4 GHz x 4096 FLOP/clk
PEAK_I8_TOPS = 5033.2       # dense int8 MFMA
PEAK_HBM_GBS = 8000.0       # HBM3E
KERNEL_SOURCES = ["gemm_nt.h", "gemm_bf16.hip", "gemm_w8a8.hip", "reduce_rmsnorm.hip", "rpl_device.h"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "row_matmul_reduce_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def load_traffic(kernel_key: str, workload: str):
    """HBM bytes per launch from committed rocprofv3 PMC summaries, if they match these sources."""
    path = os.path.join(ROOT, "profiles", "pmc_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f).get(f"{kernel_key}@{workload}")
    if not rec or rec.get("source_sha256_16") != kernel_source_hash():
        return None
    return rec.get("hbm_bytes_per_launch")


def to_dev_bf16(a, torch):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()


def build_inputs(wl, w8, torch):
    from row_matmul_reduce_amd import synth
    t0 = time.perf_counter()
    mc = wl.m_chunk
    d = {
        "x0": to_dev_bf16(synth.x_shard(wl, 0), torch),
        "w0": to_dev_bf16(synth.w_shard(wl, 0), torch),
        "res": to_dev_bf16(synth.residual_chunk(wl), torch),
        "gam": to_dev_bf16(synth.gamma(wl), torch),
        "peer_x": [to_dev_bf16(synth.x_shard(wl, s, rows=mc), torch) for s in range(1, wl.tp)],
        "peer_w": [to_dev_bf16(synth.w_shard(wl, s), torch) for s in range(1, wl.tp)],
    }
    if w8 is not None:
        xq, sx, wq, sw = synth.w8a8_inputs(w8)
        d.update(xq=torch.from_numpy(xq).cuda(), sx=torch.from_numpy(sx).cuda(),
                 wq=torch.from_numpy(wq).cuda(), sw=torch.from_numpy(sw).cuda())
    log(f"inputs generated and uploaded in {time.perf_counter() - t0:.1f} s")
    return d


def cpu_baseline(wl, w8, budget_s: float):
    """The CPU oracle on the first R token rows of the same step (R sized to the time budget)."""
    import oracle
    from row_matmul_reduce_amd import synth
    threads = oracle.num_threads()
    mc = wl.m_chunk
    x0, w0 = synth.x_shard(wl, 0, rows=mc), synth.w_shard(wl, 0)
    peers = [(synth.x_shard(wl, s, rows=mc), synth.w_shard(wl, s)) for s in range(1, wl.tp)]
    res, gam = synth.residual_chunk(wl), synth.gamma(wl)
    if w8 is not None:
        xq, sx, wq, sw = synth.w8a8_inputs(w8, rows=mc)

    def run(rows):
        r = np.arange(rows, dtype=np.int64)
        peer_parts = [oracle.partial_rows(px, pw, mc, rows=r) for px, pw in peers]  # arrived data: untimed
        t = time.perf_counter()
        own = oracle.partial_rows(x0, w0, wl.m, rows=r, tp=wl.tp)
        if w8 is not None:
            oracle.w8a8_rows(xq, sx, wq, sw, w8.m, rows=r, tp=w8.tp)
        oracle.reduce_chunk_rmsnorm([own] + peer_parts, res[:rows], gam, wl.eps)
        return time.perf_counter() - t

    pilot_rows = 8
    tp_ = run(pilot_rows)
    rows = int(min(mc, max(pilot_rows, budget_s / max(tp_, 1e-9) * pilot_rows)))
    dt = run(rows)
    ops = 2.0 * rows * wl.n * wl.k_shard * (2 if w8 is not None else 1)
    return {"value": ops / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"first {rows} of {wl.m} token rows of the step (bf16 partial"
                      f"{' + w8a8 partial' if w8 is not None else ''} + chunk reduce/RMSNorm), "
                      f"fp64 C oracle, {dt:.1f} s"}


def time_decode(torch, rpl, steps: int, copies: int):
    """Decode o_proj partial (M=8) with the weight rotated over `copies` buffers (defeats the 256 MB MALL)."""
    from row_matmul_reduce_amd import synth
    wl = synth.WORKLOADS[2]
    x = to_dev_bf16(synth.x_shard(wl, 0), torch)
    w = to_dev_bf16(synth.w_shard(wl, 0), torch)
    ws = [w] + [w.clone() for _ in range(copies - 1)]
    out = torch.empty((wl.m_pad, wl.n), dtype=torch.bfloat16, device="cuda")
    for i in range(copies):
        rpl.rpl_partial(x, ws[i], wl.tp, out=out)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    torch.cuda.synchronize()
    for i in range(steps):
        ev[i][0].record()
        rpl.rpl_partial(x, ws[i % copies], wl.tp, out=out)
        ev[i][1].record()
    torch.cuda.synchronize()
    us = float(np.mean([a.elapsed_time(b) for a, b in ev])) * 1e3
    gbs = wl.partial_bytes() / (us * 1e-6) / 1e9
    return {"workload": wl.name, "partial_us": us, "bytes": wl.partial_bytes(), "GB/s": gbs,
            "frac_hbm": gbs / PEAK_HBM_GBS, "weight_copies_rotated": copies}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="prefill", choices=["prefill", "long_prefill", "tiny"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle work for cpu_baseline")
    ap.add_argument("--no-decode", action="store_true", help="skip the decode o_proj side measurement")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this path is single-GPU (the cross-GPU reduce-scatter is not "
              "built); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    import row_matmul_reduce_amd as rpl
    from row_matmul_reduce_amd import synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    rpl.lib()
    wid = {"prefill": 3, "long_prefill": 4, "tiny": 1}[args.workload]
    wl = synth.WORKLOADS[wid]
    w8 = synth.WORKLOADS[5] if wid == 3 else None
    log(f"workload {wl.name}: m={wl.m} k_shard={wl.k_shard} n={wl.n} tp={wl.tp}"
        f"{' + w8a8 twin' if w8 else ''}")
    d = build_inputs(wl, w8, torch)
    mc = wl.m_chunk
    dev = torch.device("cuda")
    p0 = torch.empty((wl.m_pad, wl.n), dtype=torch.bfloat16, device=dev)
    q0 = torch.empty((w8.m_pad, w8.n), dtype=torch.bfloat16, device=dev) if w8 else None
    y = torch.empty((mc, wl.n), dtype=torch.bfloat16, device=dev)
    ro = torch.empty((mc, wl.n), dtype=torch.bfloat16, device=dev)
    # the peers' chunk-0 partials: data this rank receives (produced once, before timing)
    peer_chunks = [rpl.rpl_partial(px, pw, 1) for px, pw in zip(d["peer_x"], d["peer_w"])]
    torch.cuda.synchronize()

    names = ["partial_bf16"] + (["partial_w8a8"] if w8 else []) + ["reduce_rmsnorm"]

    def step(evs=None):
        """One pass of the path; evs[k] = (start, end) HIP events around kernel k."""
        def run(k, fn):
            if evs is not None:
                evs[k][0].record()
            fn()
            if evs is not None:
                evs[k][1].record()
        run(0, lambda: rpl.rpl_partial(d["x0"], d["w0"], wl.tp, out=p0))
        if w8:
            run(1, lambda: rpl.rpl_w8a8_partial(d["xq"], d["sx"], d["wq"], d["sw"], w8.tp, out=q0))
        run(len(names) - 1, lambda: rpl.rpl_reduce_chunk_rmsnorm([p0[:mc]] + peer_chunks, d["res"], d["gam"],
                                                                  wl.eps, y=y, residual_out=ro))

    for _ in range(args.warmup):
        step()
    evs = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in names]
           for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps
    kern_us = {nm: float(np.mean([evs[i][j][0].elapsed_time(evs[i][j][1]) for i in range(args.steps)])) * 1e3
               for j, nm in enumerate(names)}

    flops_bf16 = wl.gemm_flops()
    ops_i8 = w8.gemm_flops() if w8 else 0.0
    value = (flops_bf16 + ops_i8) / (ms_per_step * 1e-3) / 1e12
    kernels = {"partial_bf16": {"us": kern_us["partial_bf16"], "flop": flops_bf16,
                                "TFLOP/s": flops_bf16 / (kern_us["partial_bf16"] * 1e-6) / 1e12}}
    kernels["partial_bf16"]["frac_bf16_peak"] = kernels["partial_bf16"]["TFLOP/s"] / PEAK_BF16_TFLOPS
    if w8:
        tops = ops_i8 / (kern_us["partial_w8a8"] * 1e-6) / 1e12
        kernels["partial_w8a8"] = {"us": kern_us["partial_w8a8"], "op": ops_i8, "TOP/s": tops,
                                   "frac_int8_peak": tops / PEAK_I8_TOPS, "frac_bf16_peak": tops / PEAK_BF16_TFLOPS}
    rb = wl.reduce_bytes()
    kernels["reduce_rmsnorm"] = {"us": kern_us["reduce_rmsnorm"], "bytes": rb,
                                 "GB/s": rb / (kern_us["reduce_rmsnorm"] * 1e-6) / 1e9}
    kernels["reduce_rmsnorm"]["frac_hbm"] = kernels["reduce_rmsnorm"]["GB/s"] / PEAK_HBM_GBS

    dom = kernels["partial_bf16"]
    roofline = {"bound": "mfma", "kernel": "partial_bf16", "achieved": dom["TFLOP/s"], "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": dom["frac_bf16_peak"],
                "traffic": load_traffic("partial_bf16", wl.name)}

    extra = {}
    if not args.no_decode:
        extra["decode"] = time_decode(torch, rpl, steps=200, copies=40)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(wl, w8, args.cpu_budget)

    line = {
        "metric": METRIC, "value": value, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_per_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16+i8" if w8 else "bf16", "data": "synthetic",
        "config": {"workload": wl.name + (" + w8a8 twin" if w8 else ""), "m_tokens": wl.m,
                   "k_full": wl.k_full, "tp": wl.tp, "k_shard": wl.k_shard, "n": wl.n, "m_chunk": mc,
                   "parallelism": f"one TP rank of {wl.tp} (peers emulated)"},
        "roofline": roofline, "cpu_baseline": cpu, "kernels": kernels, "side": extra,
        "kernel_sources_sha256_16": kernel_source_hash(),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
