"""Benchmark of the row-parallel matmul + reduce hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]
                    [--workload prefill|long_prefill|w8a8|w8a8_dynamic|decode|tiny]

One step is one pass of the path for one tensor-parallel rank, on synthetic
inputs already resident in HBM:
  1. the rank's partial over its K-shard (rpl_partial in bf16, or
     rpl_w8a8_partial for the w8a8 path), all M tokens, written as
     reduce-scatter token chunks;
  2. rpl_reduce_chunk_rmsnorm on the chunk the rank receives: its own chunk
     partial + the peers' chunk partials (data that arrives from the other
     ranks, produced before timing) -> residual add -> RMSNorm.
The w8a8_dynamic path starts one step earlier, from the bf16 activation:
rpl_quant_per_token makes the int8 codes and per-token scales that the int8
partial consumes.  A model layer runs the bf16 or the w8a8 partial, not both,
so each precision is its own path.  The default run times the bf16 prefill down_proj share
(M=4096, K_full=18944 over TP=2, N=3584) as the main step, and in the same run
the w8a8 twin, the decode o_proj share and the TP=8 long-prefill share as side
steps (w8a8 both from int8 inputs and from the bf16 activation), plus the
single-launch decode path (every shard's product + sum + residual + RMSNorm in one
kernel) for a token chunk and for all rows, the all-reduce sum, the hidden-split
epilogue and the token-row shard/gather around the exchange.  Every step cycles through several copies of its inputs (more than
twice the 256 MB MALL), so operands come from HBM as a layer's weights do.  Before the W
warmup steps, untimed steps run for half a second so that the card is at its working clock.

The JSON line reports the main step's algorithmic TFLOP/s, per-kernel times
from HIP events on the launch stream, the roofline of the dominant kernel, the
SCLK / MCLK levels sampled from sysfs while the same steps run, and the CPU
oracle timed on a bounded sample of the same work.  For the GEMM paths it also
times the partials' MFMA instruction alone on random operands (mfma_ceiling): under
the board's power cap that, not the published peak, is what the card sustains with
real data, and each partial's fraction of it is reported beside its roofline.
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
MALL_BYTES = 256 << 20
# the sources each kernel is built from (its stored HBM traffic is valid while they are unchanged)
KERNEL_SOURCES = {
    "partial_bf16": ["gemm_nt.h", "gemm_bf16.hip", "rpl_device.h"],
    "partial_w8a8": ["gemm_nt.h", "gemm_w8a8.hip", "rpl_device.h"],
    "reduce_rmsnorm": ["reduce_rmsnorm.hip", "rpl_device.h"],
    "quant_per_token": ["quant_per_token.hip", "rpl_device.h"],
    "decode_fused": ["decode_fused.hip", "rpl_device.h"],
    "reduce_variants": ["reduce_variants.hip", "rpl_device.h"],
    "token_rows": ["token_rows.hip", "rpl_device.h"],
    "read_ceiling": ["read_ceiling.hip", "rpl_device.h"],
}
# kernels that live in a shared source file
KERNEL_KEY = {"sum_partials": "reduce_variants", "slice_sumsq": "reduce_variants", "slice_apply": "reduce_variants",
              "token_rows_gather": "token_rows", "token_rows_shard": "token_rows",
              "decode_fused_chunk": "decode_fused", "decode_fused_allrows": "decode_fused"}
WORKLOAD_IDS = {"tiny": 1, "decode": 2, "prefill": 3, "long_prefill": 4, "w8a8": 5, "w8a8_dynamic": 5}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash(kernel: str) -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
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
    if not rec or rec.get("source_sha256_16") != kernel_source_hash(KERNEL_KEY.get(kernel_key, kernel_key)):
        return None
    return rec.get("hbm_bytes_per_launch")


class Path:
    """One rank's step ([quantiser +] partial + received-chunk reduce/RMSNorm) on several input sets."""

    def __init__(self, wl, torch, rpl, copies: int, dynamic: bool = False):
        from row_matmul_reduce_amd import synth
        self.wl, self.torch, self.rpl = wl, torch, rpl
        self.w8 = wl.kind == "w8a8"
        self.dyn = self.w8 and dynamic
        t0 = time.perf_counter()
        mc = wl.m_chunk
        dev = torch.device("cuda")

        def bf(a):
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

        def up(a):
            return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

        base = {"res": bf(synth.residual_chunk(wl)), "gam": bf(synth.gamma(wl))}
        if self.dyn:
            wq, sw = synth.w8a8_weight(wl, 0)
            base.update(x=bf(synth.x_shard(wl, 0)), wq=up(wq), sw=up(sw))
            peers = []
            for s in range(1, wl.tp):
                pwq, psw = synth.w8a8_weight(wl, s)
                pq, psx = rpl.rpl_quant_per_token(bf(synth.x_shard(wl, s, rows=mc)))
                peers.append(rpl.rpl_w8a8_partial(pq, psx, up(pwq), up(psw), 1))
        elif self.w8:
            xq, sx, wq, sw = synth.w8a8_inputs(wl, shard=0)
            base.update(xq=up(xq), sx=up(sx), wq=up(wq), sw=up(sw))
            peers = []
            for s in range(1, wl.tp):
                pq, psx, pwq, psw = synth.w8a8_inputs(wl, rows=mc, shard=s)
                peers.append(rpl.rpl_w8a8_partial(up(pq), up(psx), up(pwq), up(psw), 1))
        else:
            base.update(x=bf(synth.x_shard(wl, 0)), w=bf(synth.w_shard(wl, 0)))
            peers = [rpl.rpl_partial(bf(synth.x_shard(wl, s, rows=mc)), bf(synth.w_shard(wl, s)), 1)
                     for s in range(1, wl.tp)]
        base["peers"] = peers  # received chunk partials (bf16), produced before timing
        self.set_bytes = sum(t.numel() * t.element_size() for v in base.values()
                             for t in (v if isinstance(v, list) else [v]))
        if copies <= 0:
            copies = max(3, -(-(2 * MALL_BYTES + 1) // self.set_bytes) + 1)
        self.sets = [base] + [{k: ([t.clone() for t in v] if isinstance(v, list) else v.clone())
                               for k, v in base.items()} for _ in range(copies - 1)]
        self.p = torch.empty((wl.m_pad, wl.n), dtype=torch.bfloat16, device=dev)
        self.y = torch.empty((mc, wl.n), dtype=torch.bfloat16, device=dev)
        self.ro = torch.empty((mc, wl.n), dtype=torch.bfloat16, device=dev)
        if self.dyn:
            self.xq = torch.empty((wl.m, wl.k_shard), dtype=torch.int8, device=dev)
            self.sx = torch.empty((wl.m,), dtype=torch.float32, device=dev)
        self.pname = "partial_w8a8" if self.w8 else "partial_bf16"
        self.names = (["quant_per_token"] if self.dyn else []) + [self.pname, "reduce_rmsnorm"]
        self.stages = ([self.quant] if self.dyn else []) + [self.partial, self.reduce]
        torch.cuda.synchronize()
        log(f"{wl.name}: inputs ready in {time.perf_counter() - t0:.1f} s, {len(self.sets)} copies x "
            f"{self.set_bytes / 1e6:.0f} MB")

    def quant(self, d):
        self.rpl.rpl_quant_per_token(d["x"], xq=self.xq, x_scale=self.sx)

    def partial(self, d):
        if self.dyn:
            self.rpl.rpl_w8a8_partial(self.xq, self.sx, d["wq"], d["sw"], self.wl.tp, out=self.p)
        elif self.w8:
            self.rpl.rpl_w8a8_partial(d["xq"], d["sx"], d["wq"], d["sw"], self.wl.tp, out=self.p)
        else:
            self.rpl.rpl_partial(d["x"], d["w"], self.wl.tp, out=self.p)

    def reduce(self, d):
        self.rpl.rpl_reduce_chunk_rmsnorm([self.p[:self.wl.m_chunk]] + d["peers"], d["res"], d["gam"],
                                          self.wl.eps, y=self.y, residual_out=self.ro)

    def step(self, i, evs=None):
        d = self.sets[i % len(self.sets)]
        for j, fn in enumerate(self.stages):
            if evs is not None:
                evs[j][0].record()
            fn(d)
            if evs is not None:
                evs[j][1].record()

    def settle(self, seconds: float = 0.5):
        """Untimed steps for at least `seconds` before the warmup steps: from idle the card takes
        tens of milliseconds to reach its working clock, far longer than a few steps of this size."""
        t0 = time.perf_counter()
        i = 0
        while time.perf_counter() - t0 < seconds:
            for _ in range(10):
                self.step(i)
                i += 1
            self.torch.cuda.synchronize()

    def run_graphs(self, steps: int, warmup: int):
        """Small (decode) paths: the host launch cost exceeds the kernels, so time HIP graphs
        that hold `steps` back-to-back launches; each replay runs them without host gaps."""
        torch = self.torch
        self.settle()
        for i in range(max(warmup, len(self.sets))):
            self.step(i)
        torch.cuda.synchronize()

        def capture(fn):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for i in range(steps):
                    fn(self.sets[i % len(self.sets)], i)
            g.replay()
            torch.cuda.synchronize()
            return g

        def per_launch_us(g, nm, replays=5):
            # the mean per launch of one replay; over `replays` replays, their mean and median
            ts = []
            for _ in range(replays):
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record()
                g.replay()
                b.record()
                torch.cuda.synchronize()
                ts.append(a.elapsed_time(b) * 1e3 / steps)
            self.medians[nm] = float(np.median(ts))
            return float(np.mean(ts))

        g_step = capture(lambda d, i: self.step(i))
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        g_step.replay()          # exactly `steps` steps
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        self.medians = {}
        kern = {nm: per_launch_us(capture(lambda d, i, fn=fn: fn(d)), nm) for nm, fn in zip(self.names, self.stages)}
        return wall * 1e3 / steps, kern, kern[self.pname]

    def run(self, steps: int, warmup: int):
        """Time `steps` steps after the clock settles and `warmup` steps: wall ms per step (the steps alone, nothing recorded
        between their kernels), then the same number of steps again with HIP events around each
        kernel for the per-kernel means and medians (us), and the back-to-back launch period of the partial
        alone (us; includes launch gaps)."""
        torch = self.torch
        self.settle()
        for i in range(warmup):
            self.step(i)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            self.step(warmup + i)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        evs = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in self.names]
               for _ in range(steps)]
        for i in range(steps):
            self.step(warmup + steps + i, evs[i])
        torch.cuda.synchronize()
        kern = {nm: float(np.mean([evs[i][j][0].elapsed_time(evs[i][j][1]) for i in range(steps)])) * 1e3
                for j, nm in enumerate(self.names)}
        self.medians = {nm: float(np.median([evs[i][j][0].elapsed_time(evs[i][j][1]) for i in range(steps)])) * 1e3
                        for j, nm in enumerate(self.names)}
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for i in range(steps):
            self.partial(self.sets[i % len(self.sets)])
        b.record()
        torch.cuda.synchronize()
        period = a.elapsed_time(b) * 1e3 / steps
        return wall * 1e3 / steps, kern, period

    def resident_partial_us(self, launches: int = 20, rounds: int = 5):
        """The partial back to back on one input set (operands stay in the 256 MB MALL, and in L2
        where they fit: the cache-resident figure) and, alternating with it in blocks of `launches`,
        back to back over the rotated HBM-resident sets, so both see the same clock. Returns the
        medians over `rounds` blocks (us per launch): (cache_resident, hbm_resident)."""
        torch = self.torch
        for _ in range(3):
            self.partial(self.sets[0])
        torch.cuda.synchronize()

        def block(pick):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            for i in range(launches):
                self.partial(self.sets[pick(i)])
            b.record()
            torch.cuda.synchronize()
            return a.elapsed_time(b) * 1e3 / launches

        res, rot = [], []
        for _ in range(rounds):
            res.append(block(lambda i: 0))
            rot.append(block(lambda i: i % len(self.sets)))
        return float(np.median(res)), float(np.median(rot))

    def kernels_report(self, kern, period):
        wl = self.wl
        pn, rn = self.pname, "reduce_rmsnorm"
        flop, pbytes, rbytes = wl.gemm_flops(), wl.partial_bytes(), wl.reduce_bytes()
        pu = kern[pn]
        peak = PEAK_I8_TOPS if self.w8 else PEAK_BF16_TFLOPS
        rate = flop / (pu * 1e-6) / 1e12
        med = getattr(self, "medians", {})
        rep = {pn: {"us": pu, "us_median": med.get(pn), "back_to_back_period_us": period, "flop": flop,
                    ("TOP/s" if self.w8 else "TFLOP/s"): rate, "frac_mfma_peak": rate / peak,
                    "bytes": pbytes, "GB/s": pbytes / (pu * 1e-6) / 1e9}}
        if self.w8:
            rep[pn]["frac_bf16_peak_figure"] = rate / PEAK_BF16_TFLOPS
        rep[pn]["frac_hbm"] = rep[pn]["GB/s"] / PEAK_HBM_GBS
        ru = kern[rn]
        rep[rn] = {"us": ru, "us_median": med.get(rn), "bytes": rbytes, "GB/s": rbytes / (ru * 1e-6) / 1e9}
        rep[rn]["frac_hbm"] = rep[rn]["GB/s"] / PEAK_HBM_GBS
        if self.dyn:
            qu, qb = kern["quant_per_token"], wl.quant_bytes()
            rep["quant_per_token"] = {"us": qu, "us_median": med.get("quant_per_token"), "bytes": qb,
                                      "GB/s": qb / (qu * 1e-6) / 1e9,
                                      "frac_hbm": qb / (qu * 1e-6) / 1e9 / PEAK_HBM_GBS}
        return rep


def fused_decode(torch, rpl, copies: int, all_rows: bool, launches: int = 200):
    """The single-launch decode path (every shard's product + sum + residual + RMSNorm) on the
    decode o_proj workload: rank 0's token chunk (reduce-scatter form) or all rows (all-reduce
    form).  Timed by replaying a HIP graph of `launches` launches over rotated weight copies,
    next to the unfused composition on the same inputs (a bf16 partial per shard, then the
    reduce + RMSNorm), captured and replayed the same way, in alternating replays."""
    from row_matmul_reduce_amd import synth
    wl = synth.WORKLOADS[WORKLOAD_IDS["decode"]]
    rows = wl.m if all_rows else wl.m_chunk

    def bf(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()

    xs = [bf(synth.x_shard(wl, s, rows=rows)) for s in range(wl.tp)]
    ws = [bf(synth.w_shard(wl, s)) for s in range(wl.tp)]
    res = bf(np.tile(synth.residual_chunk(wl), (-(-rows // wl.m_chunk), 1))[:rows])
    gam = bf(synth.gamma(wl))
    set_bytes = sum(t.numel() * 2 for t in ws)
    if copies <= 0:
        copies = max(3, -(-(2 * MALL_BYTES + 1) // set_bytes) + 1)
    sets = [ws] + [[t.clone() for t in ws] for _ in range(copies - 1)]
    work = rpl.rpl_matmul_reduce_rmsnorm_workspace(rows, wl.n, wl.tp)
    y = torch.empty_like(res)
    ro = torch.empty_like(res)
    parts = [torch.empty((rows, wl.n), dtype=torch.bfloat16, device="cuda") for _ in range(wl.tp)]
    y2, ro2 = torch.empty_like(res), torch.empty_like(res)

    def fused(i):
        rpl.rpl_matmul_reduce_rmsnorm(xs, sets[i % len(sets)], res, gam, wl.eps, workspace=work, y=y,
                                      residual_out=ro)

    def unfused(i):
        for s in range(wl.tp):
            rpl.rpl_partial(xs[s], sets[i % len(sets)][s], 1, out=parts[s])
        rpl.rpl_reduce_chunk_rmsnorm(parts, res, gam, wl.eps, y=y2, residual_out=ro2)

    def capture(fn):
        for i in range(len(sets)):
            fn(i)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(launches):
                fn(i)
        g.replay()
        torch.cuda.synchronize()
        return g

    def replay_us(g):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        g.replay()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) * 1e3 / launches

    gf, gu = capture(fused), capture(unfused)
    tf, tu = [], []
    for _ in range(5):
        tf.append(replay_us(gf))
        tu.append(replay_us(gu))
    us, uus = float(np.median(tf)), float(np.median(tu))
    status = rpl.rpl_matmul_reduce_rmsnorm_status(work)
    nbytes = (wl.tp * wl.n * wl.k_shard * 2 + wl.tp * rows * wl.k_shard * 2 + 3 * rows * wl.n * 2 + wl.n * 2)
    return {"workload": wl.name, "rows": rows, "form": "all-reduce" if all_rows else "reduce-scatter chunk",
            "shards": wl.tp, "us": us, "bytes": nbytes, "GB/s": nbytes / (us * 1e-6) / 1e9,
            "frac_hbm": nbytes / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, "weight_sets_rotated": len(sets),
            "unfused_us": uus, "fused_over_unfused_time": us / uus,
            "unfused_what": f"rpl_partial per shard ({rows} rows each) + rpl_reduce_chunk_rmsnorm, same inputs, "
                            f"same graph replay; medians of 5 alternating replays of {launches} launches each",
            "workspace_status": status}


def plain_read_ceiling(torch, rpl, tensors, launches: int = 200):
    """What a standalone launch that only reads one of `tensors` achieves here, timed like the
    decode kernels (HIP graph of `launches` launches over the rotated copies): the library's
    plain streaming read (rpl_read_ceiling, measurement only) at several grid sizes, the best
    of them as the ceiling; torch's own row reduction of the same copies as context."""
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    grids = {}
    for grid in (224, 256, 512, 1024, 2048, 4096):
        grids[grid] = _graph_mean_us(torch, lambda i, g=grid: rpl.rpl_read_ceiling(tensors[i % len(tensors)], g, sink),
                                     len(tensors), launches)
    best = min(grids, key=grids.get)
    t_sum = _graph_mean_us(torch, lambda i: torch.sum(tensors[i % len(tensors)], dim=1, dtype=torch.float32),
                           len(tensors), launches)
    nbytes = tensors[0].numel() * tensors[0].element_size()
    return {"what": "rpl_read_ceiling (a plain grid-stride read that writes nothing) of one rotated weight copy "
                    "per launch, HIP graph replay, best grid", "grid": best, "us": grids[best], "bytes": nbytes,
            "GB/s": nbytes / (grids[best] * 1e-6) / 1e9,
            "frac_hbm": nbytes / (grids[best] * 1e-6) / 1e9 / PEAK_HBM_GBS,
            "us_by_grid": grids, "torch_row_sum_us": t_sum}


def mfma_power_ceiling(torch, rpl, launches: int = 3, iters: int = 40000):
    """The MFMA instruction of each partial alone (rpl_mfma_ceiling, measurement only: 256 workgroups of
    four waves, the engine's 128 x 128 wave tile in accumulation registers, no memory traffic) on random
    operands, i.e. the rate the board's power cap allows with real data in the operands, and for bf16 also
    on zeros (the clock without the data's power).  Event-timed medians of `launches` launches of about
    40 ms; the chip's clock and each XCD's from the shader-clock and 100 MHz tick counts of every
    workgroup (workgroup b runs on XCD b mod 8)."""
    nb = rpl.MFMA_CEILING_OPS_BYTES
    g = torch.Generator(device="cuda")
    g.manual_seed(20260607)
    ops = {"bf16_random": (0, torch.randn(nb // 2, device="cuda", generator=g).to(torch.bfloat16)),
           "bf16_zero": (0, torch.zeros(nb, dtype=torch.uint8, device="cuda")),
           "i8_random": (1, torch.randint(-127, 128, (nb,), device="cuda", dtype=torch.int8, generator=g))}
    clocks = torch.zeros(512, dtype=torch.int64, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = {"what": "rpl_mfma_ceiling: v_mfma_f32_16x16x32_bf16 / v_mfma_i32_16x16x64_i8 alone on 256 workgroups "
                   "of four waves, two alternating operand sets per lane (random normal bf16, uniform int8 in "
                   "[-127, 127], or zeros), no memory traffic; medians of %d event-timed launches of %d x 128 "
                   "MFMAs per wave" % (launches, iters)}
    for name, (kind, t) in ops.items():
        rpl.rpl_mfma_ceiling(t, kind, max(1, iters // 10), clocks, sink)
        torch.cuda.synchronize()
        runs = []
        for _ in range(launches):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            rpl.rpl_mfma_ceiling(t, kind, iters, clocks, sink)
            b.record()
            torch.cuda.synchronize()
            c = clocks.view(256, 2).cpu().double()
            xcd = [float(c[x::8, 0].sum() / c[x::8, 1].sum()) * 0.1 for x in range(8)]
            runs.append((a.elapsed_time(b) * 1e3, float(c[:, 0].sum() / c[:, 1].sum()) * 0.1, xcd))
        runs.sort(key=lambda r: r[0])
        us, ghz, xcd = runs[len(runs) // 2]
        unit = "TOP/s" if kind else "TFLOP/s"
        rate = 256 * 4 * 128 * iters * (32768 if kind else 16384) / (us * 1e-6) / 1e12
        out[name] = {"us": us, unit: rate, "frac_peak": rate / (PEAK_I8_TOPS if kind else PEAK_BF16_TFLOPS),
                     "clock_ghz": ghz, "xcd_clock_ghz": xcd, "xcd_clock_spread": max(xcd) / min(xcd) - 1}
    return out


def _graph_mean_us(torch, fn, n_sets: int, launches: int = 100):
    """Mean device time per launch of fn(i) over a replayed HIP graph of `launches` launches
    (small kernels: a Python launch costs more than the kernel, so events around single
    launches would time the host)."""
    for i in range(max(3, n_sets)):
        fn(i)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(launches):
            fn(i)
    g.replay()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    g.replay()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) * 1e3 / launches


def reduce_variants(torch, rpl, copies: int):
    """The other reduction forms on the pages' shapes, HBM-resident: the all-reduce sum of the
    prefill down_proj partials (all 4096 rows, TP=2) and the hidden-split epilogue for rank 0's
    column slice of the TP=8 long-prefill chunk (2048 rows, 640 of 5120 columns)."""
    from row_matmul_reduce_amd import synth
    rng = np.random.default_rng(0)

    def bf(shape):
        return torch.from_numpy(synth.bf16_bits(rng.standard_normal(shape, dtype=np.float32)).view(np.int16)).view(
            torch.bfloat16).cuda()

    out = {}
    wl = synth.WORKLOADS[WORKLOAD_IDS["prefill"]]
    m, n, tp = wl.m, wl.n, wl.tp
    base = [bf((m, n)) for _ in range(tp)]
    nb = tp * m * n * 2
    k = copies if copies > 0 else max(3, -(-(2 * MALL_BYTES + 1) // nb) + 1)
    sets = [base] + [[t.clone() for t in base] for _ in range(k - 1)]
    o = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
    us = _graph_mean_us(torch, lambda i: rpl.rpl_sum_partials(sets[i % len(sets)], out=o), len(sets))
    b = (tp + 1) * m * n * 2
    out["allreduce_sum"] = {"workload": wl.name, "rows": m, "shards": tp, "us": us, "bytes": b,
                            "GB/s": b / (us * 1e-6) / 1e9, "frac_hbm": b / (us * 1e-6) / 1e9 / PEAK_HBM_GBS,
                            "input_sets_rotated": len(sets)}
    del sets, base
    wl = synth.WORKLOADS[WORKLOAD_IDS["long_prefill"]]
    m, n, tp = wl.m_chunk, wl.n, wl.tp
    ns = n // tp
    base = [bf((m, n)) for _ in range(tp)] + [bf((m, n))]
    nb = (tp + 1) * m * n * 2
    k = copies if copies > 0 else max(3, -(-(2 * MALL_BYTES + 1) // nb) + 1)
    sets = [base] + [[t.clone() for t in base] for _ in range(k - 1)]
    ro = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
    y = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
    h = torch.empty((m, ns), dtype=torch.float32, device="cuda")
    ss = [torch.rand(m, dtype=torch.float32, device="cuda") * ns for _ in range(tp)]
    gam = bf((n,))

    def step1(i):
        d = sets[i % len(sets)]
        rpl.rpl_reduce_slice_sumsq([p[:, :ns] for p in d[:tp]], d[tp][:, :ns], ro[:, :ns], h=h, sumsq=ss[0])

    us1 = _graph_mean_us(torch, step1, len(sets))
    us2 = _graph_mean_us(torch, lambda i: rpl.rpl_rmsnorm_slice_apply(h, ss, n, gam[:ns], wl.eps, y[:, :ns]), 1)
    b1 = tp * m * ns * 2 + 2 * m * ns * 2 + m * ns * 4 + 4 * m
    b2 = m * ns * 4 + tp * 4 * m + ns * 2 + m * ns * 2
    out["hidden_split_slice"] = {"workload": wl.name, "rows": m, "slice_cols": ns, "shards": tp,
                                 "step1_us": us1, "step1_bytes": b1, "step1_GB/s": b1 / (us1 * 1e-6) / 1e9,
                                 "step2_us": us2, "step2_bytes": b2, "step2_GB/s": b2 / (us2 * 1e-6) / 1e9,
                                 "input_sets_rotated": len(sets)}
    return out


def _dpm_files(torch):
    """sysfs DPM tables (pp_dpm_sclk, pp_dpm_mclk) of the card the process runs on, or None."""
    import glob
    props = torch.cuda.get_device_properties(0)
    want = None
    if hasattr(props, "pci_bus_id") and hasattr(props, "pci_device_id"):
        want = f"{getattr(props, 'pci_domain_id', 0):04x}:{props.pci_bus_id:02x}:{props.pci_device_id:02x}"
    cards = []
    for dev in sorted(glob.glob("/sys/class/drm/card*/device")):
        f = os.path.join(dev, "pp_dpm_sclk")
        if os.path.exists(f) and os.access(f, os.R_OK):
            cards.append((os.path.basename(os.path.realpath(dev)), dev))
    if want is not None:
        cards = [c for c in cards if c[0].lower().startswith(want)]
    if len(cards) != 1:
        return None
    dev = cards[0][1]
    return {k: os.path.join(dev, f"pp_dpm_{k}") for k in ("sclk", "mclk")}


def _hwmon_power(dpm_sclk_path):
    """(power1_input path, power cap in W) of the card's hwmon, or (None, None) if not readable."""
    import glob
    dev = os.path.dirname(dpm_sclk_path)
    for h in sorted(glob.glob(os.path.join(dev, "hwmon", "hwmon*"))):
        p, c = os.path.join(h, "power1_input"), os.path.join(h, "power1_cap")
        if os.path.exists(p) and os.access(p, os.R_OK):
            try:
                cap = int(open(c).read()) / 1e6 if os.path.exists(c) else None
            except (OSError, ValueError):
                cap = None
            return p, cap
    return None, None


def _dpm_current_mhz(path):
    """MHz of the level marked current ('*') in a pp_dpm_* table."""
    try:
        with open(path) as f:
            for ln in f:
                if ln.rstrip().endswith("*"):
                    tok = ln.split(":", 1)[1].strip().split()[0].lower()
                    return float(tok.replace("mhz", ""))
    except (OSError, ValueError, IndexError):
        return None
    return None


def clocks_under_load(torch, step, seconds: float = 1.5):
    """SCLK, MCLK and board power while steps run back to back for `seconds`: the current DPM level
    of the card and its hwmon power reading, read from sysfs every millisecond on a host thread
    (outside the timed region; same work).  The power reading is a running average that takes a
    good part of a second to settle, so only the samples of the second half of the window count."""
    import threading
    files = _dpm_files(torch)
    if files is None:
        return None
    samples = {"sclk": [], "mclk": []}
    power_path, power_cap = _hwmon_power(files["sclk"])
    watts = []
    stop = threading.Event()

    def sample():
        while not stop.is_set():
            for k, f in files.items():
                v = _dpm_current_mhz(f)
                if v is not None:
                    samples[k].append(v)
            if power_path is not None:
                try:
                    watts.append(int(open(power_path).read()) / 1e6)
                except (OSError, ValueError):
                    pass
            time.sleep(0.001)

    th = threading.Thread(target=sample, daemon=True)
    t0 = time.perf_counter()
    th.start()
    i = 0
    while time.perf_counter() - t0 < seconds:
        for _ in range(10):
            step(i)
            i += 1
        torch.cuda.synchronize()
    stop.set()
    th.join()
    for v in list(samples.values()) + [watts]:
        del v[:len(v) // 2]  # keep the settled second half
    out = {"source": "current level of pp_dpm_sclk / pp_dpm_mclk and the hwmon power1_input, sampled every "
                     f"1 ms while {i} steps ran back to back for {seconds:.1f} s; the second half of the "
                     "samples", "card": os.path.dirname(files["sclk"])}
    for k, v in samples.items():
        out[f"{k}_mhz"] = ({"median": float(np.median(v)), "min": min(v), "max": max(v), "samples": len(v)}
                          if v else None)
    out["power_w"] = ({"median": float(np.median(watts)), "min": min(watts), "max": max(watts), "samples": len(watts)}
                      if watts else None)
    out["power_cap_w"] = power_cap
    return out


def token_rows(torch, rpl, copies: int):
    """The FlashComm1 token-row movement on the TP=8 long-prefill rows, HBM-resident: rank 0's block
    of the padded residual rows (16384 x 5120 -> 2048 x 5120) and the gather of the 8 ranks' blocks
    back to all 16384 rows."""
    from row_matmul_reduce_amd import synth
    rng = np.random.default_rng(1)

    def bf(shape):
        return torch.from_numpy(synth.bf16_bits(rng.standard_normal(shape, dtype=np.float32)).view(np.int16)).view(
            torch.bfloat16).cuda()

    wl = synth.WORKLOADS[WORKLOAD_IDS["long_prefill"]]
    m, n, tp, mc = wl.m, wl.n, wl.tp, wl.m_chunk
    base = [bf((mc, n)) for _ in range(tp)]
    nb = 2 * tp * mc * n * 2  # blocks read + rows written per gather
    k = copies if copies > 0 else max(2, -(-(2 * MALL_BYTES + 1) // nb) + 1)
    sets = [base] + [[t.clone() for t in base] for _ in range(k - 1)]
    rows = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
    us_g = _graph_mean_us(torch, lambda i: rpl.rpl_gather_rows(sets[i % len(sets)], m, out=rows), len(sets))
    del sets, base
    xs = [bf((m, n)) for _ in range(max(2, -(-(2 * MALL_BYTES + 1) // (m * n * 2)) + 1))]
    blk = torch.empty((mc, n), dtype=torch.bfloat16, device="cuda")
    us_s = _graph_mean_us(torch, lambda i: rpl.rpl_shard_rows(xs[i % len(xs)], tp, 0, out=blk), len(xs))
    bg, bs = 2 * m * n * 2, 2 * mc * n * 2
    return {"token_rows": {"workload": wl.name, "rows": m, "cols": n, "ranks": tp,
                           "gather_us": us_g, "gather_bytes": bg, "gather_GB/s": bg / (us_g * 1e-6) / 1e9,
                           "gather_frac_hbm": bg / (us_g * 1e-6) / 1e9 / PEAK_HBM_GBS,
                           "shard_us": us_s, "shard_bytes": bs, "shard_GB/s": bs / (us_s * 1e-6) / 1e9,
                           "shard_frac_hbm": bs / (us_s * 1e-6) / 1e9 / PEAK_HBM_GBS}}


def library_reference(path, torch, rounds: int = 6, block: int = 20, zero: bool = True):
    """Context only, not part of the path: the vendor GEMM on the same HBM-resident input sets --
    torch.matmul (hipBLASLt, bf16) for the bf16 partial, torch._int_mm (hipBLASLt, int8 x int8 ->
    int32, without the scales and with twice the output bytes) for the w8a8 partial.  It and the
    library's partial are timed the same way, per launch with HIP events, in alternating blocks of
    `block` launches so both see the same clock; medians over all launches.  Its result is not used
    anywhere."""
    wl = path.wl

    def vendor(d):
        if path.w8:
            torch._int_mm(d["xq"], d["wq"].t())
        else:
            torch.matmul(d["x"], d["w"].t())

    def timed(fn, sets):
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(block)]
        for i, (a, b) in enumerate(evs):
            d = sets[i % len(sets)]
            a.record()
            fn(d)
            b.record()
        torch.cuda.synchronize()
        return [a.elapsed_time(b) * 1e3 for a, b in evs]

    def compare(sets, n_rounds):
        for fn in (vendor, path.partial):
            for i in range(5):
                fn(sets[i % len(sets)])
        torch.cuda.synchronize()
        ours, theirs = [], []
        for _ in range(n_rounds):
            ours += timed(path.partial, sets)
            theirs += timed(vendor, sets)
        return float(np.median(theirs)), float(np.median(ours))

    def load_of(sets):
        # the card's clock and power while each GEMM runs back to back (outside the timed blocks)
        load = {}
        for name, fn in (("partial", path.partial), ("vendor", vendor)):
            c = clocks_under_load(torch, lambda i, fn=fn: fn(sets[i % len(sets)]))
            if c is not None:
                load[name] = {"sclk_mhz": (c["sclk_mhz"] or {}).get("median"),
                              "power_w": (c["power_w"] or {}).get("median"), "power_cap_w": c["power_cap_w"]}
        return load or None

    us, own = compare(path.sets, rounds)
    rate = wl.gemm_flops() / (us * 1e-6) / 1e12
    if path.w8:
        return {"what": "torch._int_mm (hipBLASLt) of the same int8 operands, [m,k] x [n,k]^T -> int32 (no "
                        "scales, 4-byte outputs); same input rotation; it and the library's w8a8 partial timed "
                        "per launch in alternating blocks, medians",
                "us": us, "TOP/s": rate, "frac_int8_peak": rate / PEAK_I8_TOPS,
                "partial_us_same_method": own, "partial_over_vendor_time": own / us}
    load = load_of(path.sets)
    if not zero:
        return {"what": "torch.matmul (hipBLASLt) of the same operands, [m,k] x [n,k]^T, same input rotation; it "
                        "and the library's partial timed per launch in alternating blocks, medians",
                "us": us, "TFLOP/s": rate, "frac_bf16_peak": rate / PEAK_BF16_TFLOPS,
                "partial_us_same_method": own, "partial_over_vendor_time": own / us,
                "clock_and_power_under_load": load, "zero_operands": None}
    # The same two GEMMs on all-zero operands of the same shapes (as many HBM-resident copies): the
    # operands' bits hardly toggle, so the board's power cap does not bind and the clock stays near its
    # maximum -- how fast each kernel's schedule is, apart from the power the data costs.
    zsets = [{"x": torch.zeros_like(path.sets[0]["x"]), "w": torch.zeros_like(path.sets[0]["w"])}
             for _ in range(len(path.sets))]
    zus, zown = compare(zsets, max(2, rounds // 2))
    zero = {"what": "both GEMMs on all-zero operands of the same shapes and rotation (context: the clock "
                    "without the power the data's bit activity costs)",
            "vendor_us": zus, "partial_us": zown,
            "partial_TFLOP/s": wl.gemm_flops() / (zown * 1e-6) / 1e12,
            "partial_frac_bf16_peak": wl.gemm_flops() / (zown * 1e-6) / 1e12 / PEAK_BF16_TFLOPS,
            "partial_over_vendor_time": zown / zus, "clock_and_power_under_load": load_of(zsets)}
    del zsets
    return {"what": "torch.matmul (hipBLASLt) of the same operands, [m,k] x [n,k]^T, same input rotation; it and "
                    "the library's partial timed per launch in alternating blocks, medians",
            "us": us, "TFLOP/s": rate, "frac_bf16_peak": rate / PEAK_BF16_TFLOPS,
            "partial_us_same_method": own, "partial_over_vendor_time": own / us,
            "clock_and_power_under_load": load, "zero_operands": zero}


def cpu_baseline(wl, budget_s: float, dynamic: bool = False):
    """The CPU oracle on the first R token rows of the same step (R sized to the time budget).
    For the w8a8 path the step is the int8 partial rows (preceded, for w8a8_dynamic, by the
    per-token quantiser of those rows) and the chunk reduce/RMSNorm."""
    import oracle
    from row_matmul_reduce_amd import synth
    threads = oracle.num_threads()
    mc = wl.m_chunk
    res, gam = synth.residual_chunk(wl), synth.gamma(wl)
    if wl.kind == "w8a8":
        if dynamic:
            xb = synth.x_shard(wl, 0, rows=mc)
            wq0, sw0 = synth.w8a8_weight(wl, 0)
        else:
            xq0, sx0, wq0, sw0 = synth.w8a8_inputs(wl, rows=mc, shard=0)
        peers = [synth.w8a8_inputs(wl, rows=mc, shard=s) for s in range(1, wl.tp)]

        def run(rows):
            r = np.arange(rows, dtype=np.int64)
            peer_parts = [oracle.w8a8_rows(pq, psx, pwq, psw, mc, rows=r)[0]
                          for pq, psx, pwq, psw in peers]  # arrived data: untimed
            t = time.perf_counter()
            if dynamic:
                xq, sx = oracle.quant_per_token(xb, rows)
            else:
                xq, sx = xq0[:rows], sx0[:rows]
            own = oracle.w8a8_rows(xq, sx, wq0, sw0, rows, rows=r)[0]
            oracle.reduce_chunk_rmsnorm([own] + peer_parts, res[:rows], gam, wl.eps)
            return time.perf_counter() - t
    else:
        x0, w0 = synth.x_shard(wl, 0, rows=mc), synth.w_shard(wl, 0)
        peers = [(synth.x_shard(wl, s, rows=mc), synth.w_shard(wl, s)) for s in range(1, wl.tp)]

        def run(rows):
            r = np.arange(rows, dtype=np.int64)
            peer_parts = [oracle.partial_rows(px, pw, mc, rows=r) for px, pw in peers]  # arrived data: untimed
            t = time.perf_counter()
            own = oracle.partial_rows(x0, w0, wl.m, rows=r, tp=wl.tp)
            oracle.reduce_chunk_rmsnorm([own] + peer_parts, res[:rows], gam, wl.eps)
            return time.perf_counter() - t

    pilot = min(8, mc)
    t_pilot = run(pilot)
    rows = int(min(mc, max(pilot, budget_s / max(t_pilot, 1e-9) * pilot)))
    dt = run(rows)
    reps = 1
    if rows == mc and dt < budget_s / 2:  # the whole chunk is quick (decode): repeat it to fill the budget
        reps = int(min(1000, budget_s / max(dt, 1e-6)))
        dt = sum(run(rows) for _ in range(reps)) / reps
    if wl.m_pad <= 16:  # decode: the metric is bytes moved (the weight stream dominates)
        nbytes = 2.0 * (wl.n * wl.k_shard + rows * wl.k_shard + rows * wl.n) + wl.tp * 2.0 * rows * wl.n
        value, unit = nbytes / dt / 1e9, "GB/s"
    else:
        value, unit = 2.0 * rows * wl.n * wl.k_shard / dt / 1e12, ("TOP/s" if wl.kind == "w8a8" else "TFLOP/s")
    what = "partial rows + chunk reduce/RMSNorm of those rows"
    if wl.kind == "w8a8":
        what = ("per-token quantiser, " if dynamic else "") + "int8 partial rows + chunk reduce/RMSNorm of those rows"
    return {"value": value, "unit": unit, "cores": threads, "kind": "oracle", "cpu_model": _cpu_model(),
            "sample": f"the step restricted to the first {rows} of {wl.m} token rows ({what}), "
                      f"fp64 C oracle with {threads} OpenMP threads, "
                      f"{dt * reps:.1f} s" + (f" over {reps} repeats" if reps > 1 else "")}


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


# ------------------------------------------------------------------ rocprofv3 summaries
# The profiles/ summaries come from these runs of this file under rocprofv3 (each in its own run;
# <dir> is where rocprofv3 writes), then `python bench.py --rocprof-summary <dir>`.
PROFILE_RUNS = {
    "trace": "cd /tmp && rocprofv3 --kernel-trace --stats -f csv -d <dir>/trace -o bench -- "
             "python3 /root/repo/bench.py --steps 10 --warmup 2 --no-cpu-baseline --no-zero-operands",
    "fetch": "cd /tmp && rocprofv3 --pmc FETCH_SIZE -f csv -d <dir>/fetch -o run -- "
             "python3 /root/repo/bench.py --steps 4 --warmup 1 --no-cpu-baseline --no-zero-operands",
    "write": "cd /tmp && rocprofv3 --pmc WRITE_SIZE -f csv -d <dir>/write -o run -- "
             "python3 /root/repo/bench.py --steps 4 --warmup 1 --no-cpu-baseline --no-zero-operands",
    "cal_fetch": "cd /tmp && rocprofv3 --pmc FETCH_SIZE -f csv -d <dir>/cal_fetch -o run -- "
                 "python3 /root/repo/bench.py --copy-calibration",
    "cal_write": "cd /tmp && rocprofv3 --pmc WRITE_SIZE -f csv -d <dir>/cal_write -o run -- "
                 "python3 /root/repo/bench.py --copy-calibration",
    "mfma": "cd /tmp && rocprofv3 --pmc SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CYCLES GRBM_GUI_ACTIVE GRBM_COUNT -f csv "
            "-d <dir>/mfma -o run -- python3 /root/repo/bench.py --steps 4 --warmup 1 --no-cpu-baseline --no-zero-operands",
    # memory-path and wait counters of the bf16 partials and hipBLASLt, three passes (each within the
    # per-block counter limits of one pass)
    "mem_a": "cd /tmp && rocprofv3 --pmc SQ_WAIT_INST_ANY SQ_WAIT_ANY SQ_BUSY_CYCLES SQ_WAVE_CYCLES SQ_INSTS_VMEM "
             "SQ_INSTS_LDS SQ_LDS_BANK_CONFLICT SQ_WAIT_INST_LDS -f csv -d <dir>/mem_a -o run -- "
             "python3 /root/repo/bench.py --steps 4 --warmup 1 --no-cpu-baseline --no-zero-operands",
    "mem_b": "cd /tmp && rocprofv3 --pmc TA_TA_BUSY_sum TA_ADDR_STALLED_BY_TC_CYCLES_sum TD_TD_BUSY_sum TD_TC_STALL_sum "
             "TCP_PENDING_STALL_CYCLES_sum TCP_TCC_READ_REQ_sum TCP_TOTAL_CACHE_ACCESSES_sum GRBM_GUI_ACTIVE -f csv "
             "-d <dir>/mem_b -o run -- python3 /root/repo/bench.py --steps 4 --warmup 1 --no-cpu-baseline --no-zero-operands",
    "mem_c": "cd /tmp && rocprofv3 --pmc SQ_LDS_DATA_FIFO_FULL SQ_LDS_CMD_FIFO_FULL SQ_LDS_ADDR_CONFLICT SQ_LDS_IDX_ACTIVE "
             "SQ_ACTIVE_INST_LDS SQ_INST_LEVEL_VMEM SQ_INST_CYCLES_VMEM_RD SQ_INSTS_MFMA TA_DATA_STALLED_BY_TC_CYCLES_sum "
             "TA_ADDR_STALLED_BY_TD_CYCLES_sum TD_TCP_STALL_CYCLES_sum TD_SPI_STALL_sum -f csv -d <dir>/mem_c -o run -- "
             "python3 /root/repo/bench.py --steps 4 --warmup 1 --no-cpu-baseline --no-zero-operands",
}
# The default run's phases, in order, each opened by the first dispatch whose name matches (after the
# previous phase opened): the main bf16 prefill step, the two w8a8 steps, the decode step, the
# decode plain-read ceiling, the long-prefill step, the single-launch decode path (with its
# unfused composition), then the reduce variants and the token rows.
PHASES = [("prefill", None), ("w8a8", "gemm_w8a8_wide_kernel"), ("decode", "gemm_bf16_decode_kernel"),
          ("ceiling", "read_ceiling_kernel"), ("long", "gemm_bf16_wide_kernel"), ("fused", "decode_fused_kernel"),
          ("rest", "sum_partials_kernel")]
# (profile key, workload, full kernel-name prefix after "rpl::", phase, grid: None = most dispatches,
#  "min" / "max" = smallest / largest grid, "all" = every grid)
PROFILES = [
    ("partial_bf16", "prefill_down_proj_7b", "gemm_bf16_wide_kernel<224, 3, false>", "prefill", None),
    ("reduce_rmsnorm", "prefill_down_proj_7b", "reduce_rmsnorm_kernel<", "prefill", None),
    ("partial_w8a8", "w8a8_prefill_down_proj_7b", "gemm_w8a8_wide_kernel<224, 3, false>", "w8a8", "max"),
    ("quant_per_token", "w8a8_prefill_down_proj_7b", "quant_rows_kernel<", "w8a8", "max"),
    ("partial_bf16", "decode_o_proj_7b", "gemm_bf16_decode_kernel<2>", "decode", None),
    ("reduce_rmsnorm", "decode_o_proj_7b", "reduce_rmsnorm_kernel<", "decode", None),
    ("read_ceiling", "decode_o_proj_7b", "read_ceiling_kernel", "ceiling", "all"),
    ("partial_bf16", "long_prefill_tp8_share", "gemm_bf16_wide_kernel<256, 3, false>", "long", None),
    ("reduce_rmsnorm", "long_prefill_tp8_share", "reduce_rmsnorm_kernel<", "long", None),
    ("decode_fused_chunk", "decode_o_proj_7b", "decode_fused_kernel<1, 4>", "fused", None),
    ("decode_fused_allrows", "decode_o_proj_7b", "decode_fused_kernel<1, 2>", "fused", None),
    ("sum_partials", "prefill_down_proj_7b", "sum_partials_kernel", "rest", None),
    ("slice_sumsq", "long_prefill_tp8_share", "slice_sumsq_kernel", "rest", None),
    ("slice_apply", "long_prefill_tp8_share", "slice_apply_kernel", "rest", None),
    ("token_rows_gather", "long_prefill_tp8_share", "token_rows_kernel<true>", "rest", "max"),
    ("token_rows_shard", "long_prefill_tp8_share", "token_rows_kernel<false>", "rest", "min"),
]
PROFILE_NOTES = {
    "decode_fused_chunk": "single-launch decode path on rank 0's 4-row token chunk, both shards' products",
    "decode_fused_allrows": "single-launch decode path on all 8 rows (all-reduce form), both shards' products",
    "read_ceiling": "plain streaming read of one rotated 12.85 MB weight copy per launch, at each grid the bench tries",
    "token_rows_gather": "the 8 ranks' 2048-row blocks gathered back to all 16384 rows",
    "token_rows_shard": "rank 0's 2048-row block of the 16384 rows",
    "sum_partials": "all-reduce form: both ranks' partials summed over all 4096 rows",
    "slice_sumsq": "hidden-split step 1: one rank's 640-column slice of the 2048-row chunk, 8 partials",
    "slice_apply": "hidden-split step 2: the slice normalised with the 8 ranks' sums of squares",
}


def _profile_alg_bytes(key, w):
    if key.startswith("partial"):
        return w.partial_bytes()
    if key == "reduce_rmsnorm":
        return w.reduce_bytes()
    if key == "quant_per_token":
        return w.quant_bytes()
    if key.startswith("decode_fused"):
        rows = w.m_chunk if key.endswith("chunk") else w.m
        return w.tp * w.n * w.k_shard * 2 + w.tp * rows * w.k_shard * 2 + 3 * rows * w.n * 2 + w.n * 2
    if key == "read_ceiling":
        return w.n * w.k_shard * 2
    return {"sum_partials": 88080384, "slice_sumsq": 31465472, "slice_apply": 7931136,
            "token_rows_gather": 335544320, "token_rows_shard": 41943040}[key]


def _csv_rows(d, pattern):
    import csv
    import glob
    fs = sorted(glob.glob(os.path.join(d, "**", pattern), recursive=True))
    if not fs:
        return None
    with open(fs[0]) as f:
        return list(csv.DictReader(f))


def _grid(r):
    if r.get("Grid_Size") not in (None, ""):
        return int(r["Grid_Size"])
    g = 1
    for a in ("X", "Y", "Z"):
        v = r.get(f"Grid_Size_{a}")
        g *= int(v) if v not in (None, "") else 1
    return g


def _kname(r):
    """The kernel's demangled name without the leading 'void rpl::'."""
    nm = r["Kernel_Name"]
    return nm.split("rpl::", 1)[1] if "rpl::" in nm else nm


def _select(recs, order_key):
    """{(key, workload): {grid: [rows]}} following PHASES and PROFILES."""
    recs = sorted(recs, key=lambda r: int(r[order_key]))
    phase, pi, tagged = PHASES[0][0], 0, []
    for r in recs:
        if pi + 1 < len(PHASES) and PHASES[pi + 1][1] in _kname(r):
            pi += 1
            phase = PHASES[pi][0]
        tagged.append((phase, r))
    out = {}
    for key, wname, prefix, ph, gsel in PROFILES:
        grids = {}
        for p_, r in tagged:
            if p_ == ph and _kname(r).startswith(prefix):
                grids.setdefault(_grid(r), []).append(r)
        if not grids:
            continue
        if gsel == "all":
            out[(key, wname)] = grids
            continue
        g = (min(grids) if gsel == "min" else max(grids) if gsel == "max"
             else max(grids, key=lambda k: len(grids[k])))
        out[(key, wname)] = {g: grids[g]}
    return out


def rocprof_summary(d: str):
    """Write profiles/<key>__<workload>.md, profiles/pmc_traffic.json and profiles/mfma_util__*.md from
    the rocprofv3 runs of PROFILE_RUNS found under d."""
    import statistics
    from row_matmul_reduce_amd import synth
    wls = {w.name: w for w in synth.WORKLOADS.values()}
    cmds = PROFILE_RUNS
    trace = _csv_rows(os.path.join(d, "trace"), "*kernel_trace.csv")
    stats = _csv_rows(os.path.join(d, "trace"), "*kernel_stats.csv") or []
    if trace is None:
        raise SystemExit(f"no kernel trace under {d}/trace")
    tsel = _select(trace, "Start_Timestamp")

    def counter(sub, name):
        rows = _csv_rows(os.path.join(d, sub), "*counter_collection.csv")
        return [r for r in rows if r["Counter_Name"] == name] if rows else None

    fetch, write = counter("fetch", "FETCH_SIZE"), counter("write", "WRITE_SIZE")
    cf, cw = counter("cal_fetch", "FETCH_SIZE"), counter("cal_write", "WRITE_SIZE")
    traffic, rf, wf = None, None, None
    if fetch and write and cf and cw:
        cbytes = 512 << 20
        fk = statistics.median(float(r["Counter_Value"]) for r in cf if "copy" in r["Kernel_Name"].lower())
        wk = statistics.median(float(r["Counter_Value"]) for r in cw if "copy" in r["Kernel_Name"].lower())
        rf, wf = cbytes / (fk * 1024), cbytes / (wk * 1024)
        fsel, wsel = _select(fetch, "Dispatch_Id"), _select(write, "Dispatch_Id")
        traffic = {"_about": "HBM traffic per launch from rocprofv3 --pmc FETCH_SIZE and WRITE_SIZE passes (KiB per "
                             "dispatch, median over the dispatches of the kernel at its workload), each scaled by what the "
                             "same counter reads for a plain 512 MiB device copy: bytes = FETCH_SIZE*1024*read_factor + "
                             "WRITE_SIZE*1024*write_factor.",
                   "_copy_calibration": {"bytes": cbytes, "fetch_kib": fk, "write_kib": wk, "read_factor": rf,
                                         "write_factor": wf},
                   "_commands": [cmds["fetch"], cmds["write"], cmds["cal_fetch"], cmds["cal_write"]]}
    lines_out = []
    for key, wname, prefix, ph, gsel in PROFILES:
        if (key, wname) not in tsel:
            continue
        w = wls[wname]
        src_key = KERNEL_KEY.get(key, key)
        sha = kernel_source_hash(src_key)
        ab = _profile_alg_bytes(key, w)
        md = [f"# {key} -- {wname}" + (f" ({PROFILE_NOTES[key]})" if key in PROFILE_NOTES else ""), "",
              f"Workload: m={w.m} tokens, K_full={w.k_full} over TP={w.tp} (K_shard={w.k_shard}), n={w.n}, "
              f"m_chunk={w.m_chunk}; kernel sources sha256/16 {sha}.", "",
              "Command (kernel trace + stats; the bench cycles through HBM-resident input copies), then "
              "`python bench.py --rocprof-summary <dir>`:", "", "    " + cmds["trace"], ""]
        for g, sel in sorted(tsel[(key, wname)].items()):
            durs = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in sel]
            mean, med = statistics.mean(durs), statistics.median(durs)
            if key.startswith("partial") and w.m_pad > 16:
                rate = f"{w.gemm_flops() / (mean * 1e-6) / 1e12:.1f} T{'OP' if 'w8a8' in key else 'FLOP'}/s on the mean"
            else:
                rate = f"{ab / (mean * 1e-6) / 1e9:.0f} GB/s on the mean ({ab / 1e6:.2f} MB algorithmic)"
            full = sel[0]["Kernel_Name"]
            md += [f"Kernel `{full}`, grid {g} threads: {len(sel)} dispatches in the phase; duration mean {mean:.2f} us, "
                   f"median {med:.2f} us, min {min(durs):.2f} us, max {max(durs):.2f} us; {rate}.", ""]
            lines_out.append(f"{key:22s} {wname:28s} grid {g:8d} n={len(sel):6d} mean {mean:9.2f} us median {med:9.2f}")
            st = [x for x in stats if x["Name"] == full]
            if st:
                x = st[0]
                md += ["rocprofv3 --stats row of this kernel (every dispatch of it in the run, all phases):", "",
                       '    "Name","Calls","TotalDurationNs","AverageNs","Percentage","MinNs","MaxNs","StdDev"',
                       "    " + ",".join([f'"{x["Name"]}"'] + [x[c] for c in ("Calls", "TotalDurationNs", "AverageNs",
                                                                          "Percentage", "MinNs", "MaxNs", "StdDev")]), ""]
        if traffic is not None and (key, wname) in fsel and (key, wname) in wsel and gsel != "all":
            fr = next(iter(fsel[(key, wname)].values()))
            wr = next(iter(wsel[(key, wname)].values()))
            fv = statistics.median(float(r["Counter_Value"]) for r in fr)
            wv = statistics.median(float(r["Counter_Value"]) for r in wr)
            hbm = fv * 1024 * rf + wv * 1024 * wf
            traffic[f"{key}@{wname}"] = {"source_sha256_16": sha, "sources": KERNEL_SOURCES[src_key],
                                         "kernel": fr[0]["Kernel_Name"], "dispatches": [len(fr), len(wr)],
                                         "fetch_kib": fv, "write_kib": wv, "hbm_bytes_per_launch": hbm,
                                         "algorithmic_bytes": ab, "ratio_to_algorithmic": hbm / ab}
            md += [f"HBM traffic (rocprofv3 --pmc FETCH_SIZE, then WRITE_SIZE, in separate runs of the bench; scaled by a "
                   f"512 MiB device copy, read factor {rf:.3f}, write factor {wf:.3f}):", "",
                   f"    FETCH_SIZE {fv:,.0f} KiB, WRITE_SIZE {wv:,.0f} KiB per dispatch (median of {len(fr)}) -> "
                   f"{hbm / 1e6:.2f} MB per launch vs {ab / 1e6:.2f} MB algorithmic ({hbm / ab:.2f}x)", "",
                   "    counter commands:"] + ["    " + c for c in traffic["_commands"]]
        with open(os.path.join(ROOT, "profiles", f"{key}__{wname}.md"), "w") as f:
            f.write("\n".join(md) + "\n")
    if traffic is not None:
        traffic.update(_vendor_traffic(d, wls, rf, wf))
        with open(os.path.join(ROOT, "profiles", "pmc_traffic.json"), "w") as f:
            json.dump(traffic, f, indent=1)
    print("\n".join(lines_out))
    _mfma_summary(d, cmds["mfma"])
    _memory_path_summary(d, cmds)


def _vendor_traffic(d, wls, rf, wf):
    """HBM traffic of the vendor GEMMs the bench times beside the partials (hipBLASLt's kernels, named
    Cijk_*), from the same FETCH_SIZE / WRITE_SIZE passes and copy calibration as the library's
    kernels, against the algorithmic bytes of the vendor's own problem (its int8 GEMM writes int32)."""
    import statistics
    fd, wd = _counter_dispatches(d, "fetch"), _counter_dispatches(d, "write")
    out = {}
    if not fd or not wd:
        return out
    for ph, wname, label in (("prefill", "prefill_down_proj_7b", "hipblaslt_bf16"),
                             ("w8a8", "w8a8_prefill_down_proj_7b", "hipblaslt_int8"),
                             ("long", "long_prefill_tp8_share", "hipblaslt_bf16")):
        fr = [dd for p_, dd in fd if p_ == ph and "Cijk_" in dd["r"]["Kernel_Name"] and "FETCH_SIZE" in dd]
        wr = [dd for p_, dd in wd if p_ == ph and "Cijk_" in dd["r"]["Kernel_Name"] and "WRITE_SIZE" in dd]
        if not fr or not wr:
            continue
        w = wls[wname]
        ab = (w.m * w.k_shard + w.n * w.k_shard + 4 * w.m * w.n) if label.endswith("int8") else \
            2 * (w.m * w.k_shard + w.n * w.k_shard + w.m * w.n)
        fv = statistics.median(dd["FETCH_SIZE"] for dd in fr)
        wv = statistics.median(dd["WRITE_SIZE"] for dd in wr)
        hbm = fv * 1024 * rf + wv * 1024 * wf
        out[f"{label}@{wname}"] = {"kernel": fr[0]["r"]["Kernel_Name"][:120], "dispatches": [len(fr), len(wr)],
                                   "fetch_kib": fv, "write_kib": wv, "hbm_bytes_per_launch": hbm,
                                   "algorithmic_bytes": ab, "ratio_to_algorithmic": hbm / ab,
                                   "note": "vendor GEMM on the same operands (context, not part of the path)"}
    return out


def _counter_dispatches(d, sub):
    """Per-dispatch counter dicts of one --pmc pass ({"r": first csv row, counter: value}), in dispatch
    order, each tagged with its bench phase."""
    rows = _csv_rows(os.path.join(d, sub), "*counter_collection.csv")
    if not rows:
        return None
    by = {}
    for r in rows:
        by.setdefault(int(r["Dispatch_Id"]), {"r": r})[r["Counter_Name"]] = float(r["Counter_Value"])
    phase, pi, out = PHASES[0][0], 0, []
    for _, dd in sorted(by.items()):
        if pi + 1 < len(PHASES) and PHASES[pi + 1][1] in _kname(dd["r"]):
            pi += 1
            phase = PHASES[pi][0]
        out.append((phase, dd))
    return out


def _memory_path_summary(d, cmds, out_dir=None):
    """profiles/memory_path_counters__prefill_down_proj_7b.md: per-dispatch medians of the memory-path
    and wait counters for the bf16 partial and hipBLASLt on the prefill and long-prefill shares."""
    import statistics
    passes = [(k, _counter_dispatches(d, k)) for k in ("mem_a", "mem_b", "mem_c")]
    if any(v is None for _, v in passes):
        return
    cols = [("lib:prefill", "prefill", "Cijk_"), ("lib:long", "long", "Cijk_"),
            ("ours:prefill", "prefill", "gemm_bf16_wide_kernel"), ("ours:long", "long", "gemm_bf16_wide_kernel")]

    def pick(disp, ph, key):
        return [dd for p_, dd in disp if p_ == ph and key in dd["r"]["Kernel_Name"] and
                (key == "Cijk_" or _grid(dd["r"]) == 65536)]

    out = ["# Memory-path and wait counters -- bf16 partial (four-wave engine) against hipBLASLt, prefill down_proj "
           "and long-prefill shares", "",
           "Commands (three counter passes of the same bench command, each within the per-block counter limits of "
           "one pass), then `python bench.py --rocprof-summary <dir>`:", ""]
    out += ["    " + cmds[k] for k, _ in passes]
    out += ["", "Per-dispatch medians. Columns: hipBLASLt (torch.matmul on the same operands) and the engine "
            "(`gemm_bf16_wide_kernel`, its timed calls) on the prefill share (4096 x 9472 x 3584) and the long-prefill "
            "share (16384 x 3200 x 5120). Durations are those of a kernel running alone (counter collection "
            "serialises dispatches).", "", "```"]
    waits = {}
    for k, disp in passes:
        sel = {c: pick(disp, ph, key) for c, ph, key in cols}
        names = sorted({n for v in sel.values() for dd in v for n in dd if n != "r"})
        out.append(f"== pass {k}")
        out.append(f"{'counter':40s}" + "".join(f"{c:>16s}" for c, _, _ in cols))

        def dur(v):
            if not v or not v[0]["r"].get("Start_Timestamp"):
                return float("nan")
            return statistics.median((int(x["r"]["End_Timestamp"]) - int(x["r"]["Start_Timestamp"])) / 1e3 for x in v)
        out.append(f"{'n / duration us':40s}" + "".join(f"{len(sel[c]):>7d}/{dur(sel[c]):8.1f}" for c, _, _ in cols))
        for n in names:
            vals = []
            for c, _, _ in cols:
                xs = [dd[n] for dd in sel[c] if n in dd]
                vals.append(statistics.median(xs) if xs else float("nan"))
                if n in ("SQ_WAIT_ANY", "SQ_WAVE_CYCLES"):
                    waits.setdefault(c, {})[n] = vals[-1]
            out.append(f"{n:40s}" + "".join(f"{v:16.4g}" for v in vals))
    out.append("```")
    if waits:
        out += ["", "Fraction of wave cycles spent waiting (`SQ_WAIT_ANY / SQ_WAVE_CYCLES`): " + ", ".join(
            f"{c} {w['SQ_WAIT_ANY'] / w['SQ_WAVE_CYCLES']:.1%}" for c, w in waits.items()
            if w.get("SQ_WAVE_CYCLES"))]
    with open(os.path.join(out_dir or os.path.join(ROOT, "profiles"), "memory_path_counters__prefill_down_proj_7b.md"),
              "w") as f:
        f.write("\n".join(out) + "\n")
    print("\n".join(out[-3:]))


def _mfma_summary(d, cmd):
    import statistics
    rows = _csv_rows(os.path.join(d, "mfma"), "*counter_collection.csv")
    if not rows:
        return
    by = {}
    for r in rows:
        by.setdefault(int(r["Dispatch_Id"]), {"r": r})[r["Counter_Name"]] = float(r["Counter_Value"])
    disp = [v for _, v in sorted(by.items())]
    phase, pi, groups = PHASES[0][0], 0, {}
    for dd in disp:
        r = dd["r"]
        if pi + 1 < len(PHASES) and PHASES[pi + 1][1] in _kname(r):
            pi += 1
            phase = PHASES[pi][0]
        nm = r["Kernel_Name"]
        if phase in ("prefill", "long") and "gemm_bf16_wide_kernel" in nm and _grid(r) == 65536:
            label = f"`{_kname(r).split('(')[0]}` ({'prefill' if phase == 'prefill' else 'long prefill'}, grid 65536)"
        elif phase == "w8a8" and "gemm_w8a8_wide_kernel" in nm and _grid(r) == 65536:
            label = f"`{_kname(r).split('(')[0]}` (w8a8 prefill, grid 65536)"
        elif phase in ("prefill", "long") and "Cijk_" in nm:
            label = f"hipBLASLt `{nm[:20]}...` ({'prefill' if phase == 'prefill' else 'long prefill'}, same operands, grid {_grid(r)})"
        else:
            continue
        groups.setdefault(label, []).append(dd)
    out = ["# MFMA utilisation and clock -- bf16 and w8a8 partials on the prefill shares, and hipBLASLt on the same "
           "operands", "", "Command (one counter pass; the bench cycles through HBM-resident input copies), then "
           "`python bench.py --rocprof-summary <dir>`:", "", "    " + cmd, "",
           "Per dispatch, medians over the dispatches of each kernel in its phase of the bench. "
           "`SQ_VALU_MFMA_BUSY_CYCLES` is summed over the 1024 SIMDs, `GRBM_GUI_ACTIVE` over the 8 XCDs, so the "
           "clock is `GUI_ACTIVE / 8 / duration` and the MFMA busy fraction `MFMA_BUSY / (1024 * GUI_ACTIVE / 8)`. "
           "Counter collection serialises dispatches: durations are those of a kernel running alone.", "",
           "| Kernel (workload) | Dispatches | Duration | MFMA_BUSY | GUI_ACTIVE | Clock | MFMA busy |",
           "|---|---|---|---|---|---|---|"]
    for label, ds in groups.items():
        def med(k):
            return statistics.median(x.get(k, float("nan")) for x in ds)
        r0 = ds[0]["r"]
        dur = None
        if r0.get("Start_Timestamp"):
            dur = statistics.median((int(x["r"]["End_Timestamp"]) - int(x["r"]["Start_Timestamp"])) / 1e3 for x in ds)
        busy, gui = med("SQ_VALU_MFMA_BUSY_CYCLES"), med("GRBM_GUI_ACTIVE")
        clk = f"{gui / 8 / (dur * 1e-6) / 1e9:.2f} GHz" if dur else "n/a"
        durs = f"{dur:.1f} us" if dur else "n/a"
        out.append(f"| {label} | {len(ds)} | {durs} | {busy:.4g} | {gui:.4g} | {clk} | {busy / (1024 * gui / 8):.0%} |")
    with open(os.path.join(ROOT, "profiles", "mfma_util__prefill_down_proj_7b.md"), "w") as f:
        f.write("\n".join(out) + "\n")
    print("\n".join(out[-len(groups):]))


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="prefill", choices=list(WORKLOAD_IDS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-zero-operands", action="store_true",
                    help="skip the vendor comparison's runs on all-zero operands (the profile passes use this, so "
                         "that every dispatch they summarise ran on the workload's data)")
    ap.add_argument("--cpu-budget", type=float, default=25.0, help="seconds of oracle work for cpu_baseline (the pilot estimate runs long: about half of it is spent)")
    ap.add_argument("--no-side", action="store_true",
                    help="skip the side paths (w8a8, w8a8_dynamic, decode, long prefill)")
    ap.add_argument("--copies", type=int, default=0,
                    help="input sets cycled through (0: enough to exceed twice the 256 MB MALL)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 512 MiB device-to-device copy three times (scales HBM counters)")
    ap.add_argument("--rocprof-summary", metavar="DIR",
                    help="no GPU work: write profiles/ from the rocprofv3 runs of PROFILE_RUNS under DIR")
    args = ap.parse_args()
    if args.rocprof_summary:
        rocprof_summary(args.rocprof_summary)
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this path is one tensor-parallel rank's share on one GPU (the "
              "cross-GPU reduce-scatter is not built); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    import row_matmul_reduce_amd as rpl
    from row_matmul_reduce_amd import synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    rpl.lib()
    if args.copy_calibration:
        nbytes = 512 << 20
        srcs = [torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(i) for i in range(3)]
        dst = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        for src in srcs:
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration": {"bytes_read": nbytes, "bytes_written": nbytes, "launches": 3}}))
        return
    wl = synth.WORKLOADS[WORKLOAD_IDS[args.workload]]
    path = Path(wl, torch, rpl, args.copies, dynamic=args.workload == "w8a8_dynamic")
    small = wl.m_pad <= 16
    runner = path.run_graphs if small else path.run
    ms_per_step, kern, period = runner(args.steps, args.warmup)
    kernels = path.kernels_report(kern, period)
    clocks = None if small else clocks_under_load(torch, path.step)
    if not small:
        ru, rr = path.resident_partial_us()
        rate = "TFLOP/s" if not path.w8 else "TOP/s"
        kernels[path.pname]["cache_resident"] = {
            "what": "back to back on one input set (operands resident in MALL), alternating in blocks with the "
                    "rotated HBM-resident sets; medians of 5 blocks of 20; not the headline",
            "us": ru, rate: wl.gemm_flops() / (ru * 1e-6) / 1e12, "hbm_resident_us": rr}
    pn = path.pname
    if small:  # decode: bound by the weight stream
        value, unit = (wl.partial_bytes() + wl.reduce_bytes()) / (ms_per_step * 1e-3) / 1e9, "GB/s"
        roofline = {"bound": "hbm", "kernel": pn, "achieved": kernels[pn]["GB/s"], "peak": PEAK_HBM_GBS,
                    "unit": "GB/s", "frac": kernels[pn]["frac_hbm"], "traffic": load_traffic(pn, wl.name)}
    else:
        value, unit = wl.gemm_flops() / (ms_per_step * 1e-3) / 1e12, ("TOP/s" if path.w8 else "TFLOP/s")
        peak = PEAK_I8_TOPS if path.w8 else PEAK_BF16_TFLOPS
        rate = kernels[pn]["TOP/s" if path.w8 else "TFLOP/s"]
        roofline = {"bound": "mfma", "kernel": pn, "achieved": rate, "peak": peak,
                    "unit": "TOP/s" if path.w8 else "TFLOP/s", "frac": rate / peak,
                    "traffic": load_traffic(pn, wl.name)}
    sets_used = len(path.sets)
    w8 = path.w8
    reference = None
    if not path.w8 and not small and not args.no_side:
        reference = library_reference(path, torch, zero=not args.no_zero_operands)
    del path
    torch.cuda.empty_cache()

    side = {}
    if not args.no_side and args.workload == "prefill":
        for key in ("w8a8", "w8a8_dynamic", "decode", "long_prefill"):
            swl = synth.WORKLOADS[WORKLOAD_IDS[key]]
            sp = Path(swl, torch, rpl, args.copies, dynamic=key == "w8a8_dynamic")
            if swl.m_pad <= 16:
                s_ms, s_kern, s_period = sp.run_graphs(200, 3)
            else:
                s_ms, s_kern, s_period = sp.run(10, 3)
            side[key] = {"workload": swl.name, "ms_per_step": s_ms, "input_sets_rotated": len(sp.sets),
                         "kernels": sp.kernels_report(s_kern, s_period)}
            if swl.m_pad <= 16:  # decode: the same weight copies read by a plain standalone launch
                ceil = plain_read_ceiling(torch, rpl, [d["w"] for d in sp.sets])
                kp = side[key]["kernels"][sp.pname]
                kp["plain_read_ceiling"] = ceil
                kp["frac_of_ceiling"] = ceil["us"] / kp["us"]
            if key in ("long_prefill", "w8a8"):
                side[key]["library_reference"] = library_reference(sp, torch, zero=not args.no_zero_operands)
            del sp
            torch.cuda.empty_cache()

    if not args.no_side and args.workload == "prefill":
        for key, all_rows in (("decode_fused_chunk", False), ("decode_fused_allreduce", True)):
            side[key] = fused_decode(torch, rpl, args.copies, all_rows)
            torch.cuda.empty_cache()
        side.update(reduce_variants(torch, rpl, args.copies))
        torch.cuda.empty_cache()
        side.update(token_rows(torch, rpl, args.copies))
        torch.cuda.empty_cache()

    ceiling = None
    if not small:  # the GEMM partials against what their MFMA instruction alone sustains here
        ceiling = mfma_power_ceiling(torch, rpl)
        torch.cuda.empty_cache()
        kernels[pn]["frac_of_power_limited_mfma_ceiling"] = roofline["achieved"] / ceiling[
            "i8_random" if w8 else "bf16_random"][roofline["unit"]]
        for key, ck, u in (("w8a8", "i8_random", "TOP/s"), ("w8a8_dynamic", "i8_random", "TOP/s"),
                           ("long_prefill", "bf16_random", "TFLOP/s")):
            kp = side.get(key, {}).get("kernels", {})
            for kname in ("partial_w8a8", "partial_bf16"):
                if kname in kp and u in kp[kname]:
                    kp[kname]["frac_of_power_limited_mfma_ceiling"] = kp[kname][u] / ceiling[ck][u]

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(wl, args.cpu_budget, dynamic=args.workload == "w8a8_dynamic")
        cpu["gpu_over_cpu"] = value / cpu["value"] if cpu["unit"] == unit else None

    line = {
        "metric": METRIC, "value": value, "unit": unit, "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_per_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "i8" if wl.kind == "w8a8" else "bf16", "data": "synthetic",
        "config": {"workload": wl.name, "m_tokens": wl.m, "k_full": wl.k_full, "tp": wl.tp, "k_shard": wl.k_shard,
                   "n": wl.n, "m_chunk": wl.m_chunk, "parallelism": f"one TP rank of {wl.tp} (peers emulated)",
                   "input_sets_rotated": sets_used},
        "roofline": roofline, "cpu_baseline": cpu, "kernels": kernels, "clocks": clocks, "side": side,
        "library_reference": reference, "mfma_ceiling": ceiling,
        "kernel_sources_sha256_16": {k: kernel_source_hash(k) for k in KERNEL_SOURCES},
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
