"""Host-side logic of bench.py that runs without a GPU: the one-GPU guard, the CPU oracle
baseline's fields and units, and the stored HBM traffic being tied to the kernel sources."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from row_matmul_reduce_amd import synth  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


@pytest.mark.parametrize("wid, unit, dynamic", [(1, "TFLOP/s", False), (2, "GB/s", False), (5, "TOP/s", False),
                                                (5, "TOP/s", True)])
def test_cpu_baseline_fields(wid, unit, dynamic):
    wl = synth.WORKLOADS[wid]
    cb = bench.cpu_baseline(wl, 0.2, dynamic=dynamic)
    assert cb["kind"] == "oracle" and cb["unit"] == unit
    assert ("quantiser" in cb["sample"]) == dynamic
    assert cb["value"] > 0 and cb["cores"] >= 1
    assert isinstance(cb["cpu_model"], str) and cb["cpu_model"]
    assert f"of {wl.m} token rows" in cb["sample"]


def test_stored_traffic_follows_the_sources():
    with open(os.path.join(ROOT, "profiles", "pmc_traffic.json")) as f:
        stored = json.load(f)
    keys = [k for k in stored if not k.startswith("_")]
    assert keys, "no stored traffic records"
    for key in keys:
        kernel, workload = key.split("@")
        rec = stored[key]
        current = bench.kernel_source_hash(bench.KERNEL_KEY.get(kernel, kernel))
        got = bench.load_traffic(kernel, workload)
        if rec["source_sha256_16"] == current:
            assert got == rec["hbm_bytes_per_launch"] and got > 0
        else:
            assert got is None


def test_kernel_sources_exist():
    for files in bench.KERNEL_SOURCES.values():
        for f in files:
            assert os.path.exists(os.path.join(ROOT, "row_matmul_reduce_amd", "csrc", f)), f
