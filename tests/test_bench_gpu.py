"""bench.py end to end on the GPU, shortened: one JSON line with the fields its contract names,
and the roofline and CPU-baseline objects filled in consistently."""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_json_line():
    print("[bench] bench.py --steps 3 --warmup 1 --no-side --cpu-budget 0.5", flush=True)
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--steps", "3", "--warmup", "1",
                        "--no-side", "--cpu-budget", "0.5"], capture_output=True, text=True, timeout=110)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [ln for ln in r.stdout.splitlines() if ln.strip()]
    assert len(lines) == 1, r.stdout
    d = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
                "scaling", "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline"):
        assert key in d, key
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["warmup"] == 1
    assert d["unit"] == "TFLOP/s" and d["value"] > 0 and d["ms_per_step"] > 0 and d["higher_is_better"] is True
    assert d["dtype"] == "bf16" and d["data"] == "synthetic" and d["config"]["workload"] == "prefill_down_proj_7b"
    rf = d["roofline"]
    assert rf["bound"] == "mfma" and rf["unit"] == "TFLOP/s" and rf["peak"] == pytest.approx(2516.6)
    assert rf["frac"] == pytest.approx(rf["achieved"] / rf["peak"]) and 0 < rf["frac"] < 1
    assert rf["traffic"] is None or rf["traffic"] > 0
    cb = d["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["unit"] == "TFLOP/s" and cb["value"] > 0 and cb["cores"] >= 1
    # the whole step (partial + reduce) cannot run faster than its partial alone
    part = d["kernels"]["partial_bf16"]
    assert d["value"] <= part["TFLOP/s"] * 1.05
    # the MFMA instruction alone: below the dense peak, and the partial below it
    mc = d["mfma_ceiling"]
    for name, unit in (("bf16_random", "TFLOP/s"), ("bf16_zero", "TFLOP/s"), ("i8_random", "TOP/s")):
        e = mc[name]
        assert 0 < e["frac_peak"] <= 1.0 and e[unit] > 0, (name, e)
        assert 0.5 < e["clock_ghz"] < 3.0 and len(e["xcd_clock_ghz"]) == 8, (name, e)
        assert all(0.5 < c < 3.0 for c in e["xcd_clock_ghz"]) and e["xcd_clock_spread"] >= 0
    assert 0 < part["frac_of_power_limited_mfma_ceiling"] < 1.05


def test_mfma_ceiling_helper():
    """The MFMA measurement helper on both instructions: every workgroup reports its loop's shader-clock
    and 100 MHz ticks, and the clock they give lies in the card's range."""
    import torch
    import row_matmul_reduce_amd as rpl
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    nb = rpl.MFMA_CEILING_OPS_BYTES
    ops = torch.randint(-127, 128, (nb,), dtype=torch.int8, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    for kind in (0, 1):
        print(f"[mfma_ceiling] kind={kind} iters=200", flush=True)
        clocks = torch.zeros(512, dtype=torch.int64, device="cuda")
        rpl.rpl_mfma_ceiling(ops, kind, 200, clocks, sink)
        torch.cuda.synchronize()
        c = clocks.view(256, 2).cpu()
        assert bool((c > 0).all()), "every workgroup wrote its ticks"
        ghz = c[:, 0].double() / c[:, 1].double() * 0.1
        assert bool(((ghz > 0.3) & (ghz < 3.0)).all()), ghz
    with pytest.raises(rpl.RplError):
        rpl.rpl_mfma_ceiling(ops[:nb - 16], 0, 10, clocks, sink)
