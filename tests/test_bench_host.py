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
    # the vendor GEMMs' records (context only) carry no library sources
    vendor = [k for k in keys if k.startswith("hipblaslt_")]
    assert all("source_sha256_16" not in stored[k] and stored[k]["hbm_bytes_per_launch"] > 0 for k in vendor)
    for key in (k for k in keys if k not in vendor):
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


def test_rocprof_phase_selection():
    """The profile summariser splits the bench's dispatches into its phases by the first kernel of
    each phase and picks each profile's kernel by its full name (template arguments included):
    the decode step's rank partial is the 8-row kernel, not the peer chunk's 4-row one."""
    names = ["gemm_bf16_wide_kernel<224, 3, false>(x)", "reduce_rmsnorm_kernel<7, 1, 1, true>(x)",
             "gemm_w8a8_wide_kernel<224, 3, false>(x)", "quant_rows_kernel<4, 1, 1>(x)",
             "gemm_bf16_decode_kernel<4>(x)", "gemm_bf16_decode_kernel<2>(x)", "gemm_bf16_decode_kernel<2>(x)",
             "reduce_rmsnorm_kernel<2, 8, 1, false>(x)", "read_ceiling_kernel(x)", "read_ceiling_kernel(x)",
             "gemm_bf16_wide_kernel<256, 3, false>(x)", "reduce_rmsnorm_kernel<3, 4, 1, true>(x)",
             "decode_fused_kernel<1, 4>(x)", "gemm_bf16_decode_kernel<4>(x)", "decode_fused_kernel<1, 2>(x)",
             "sum_partials_kernel(x)", "token_rows_kernel<true>(x)", "token_rows_kernel<false>(x)"]
    grids = [65536, 2048, 65536, 1024, 57344, 57344, 57344, 1024, 65536, 131072, 65536, 512, 115712, 57344,
             115712, 4096, 8192, 4096]
    recs = [{"Kernel_Name": "void rpl::" + n, "Grid_Size": str(g), "Start_Timestamp": str(i)}
            for i, (n, g) in enumerate(zip(names, grids))]
    sel = bench._select(recs, "Start_Timestamp")
    dec = sel[("partial_bf16", "decode_o_proj_7b")]
    assert list(dec) == [57344] and len(dec[57344]) == 2 and all("<2>" in r["Kernel_Name"] for r in dec[57344])
    assert list(sel[("partial_bf16", "prefill_down_proj_7b")][65536])[0]["Start_Timestamp"] == "0"
    assert sel[("partial_bf16", "long_prefill_tp8_share")][65536][0]["Start_Timestamp"] == "10"
    assert "<3, 4, 1, true>" in sel[("reduce_rmsnorm", "long_prefill_tp8_share")][512][0]["Kernel_Name"]
    assert sorted(sel[("read_ceiling", "decode_o_proj_7b")]) == [65536, 131072]
    assert "<1, 4>" in sel[("decode_fused_chunk", "decode_o_proj_7b")][115712][0]["Kernel_Name"]
    assert list(sel[("token_rows_gather", "long_prefill_tp8_share")]) == [8192]
    assert list(sel[("token_rows_shard", "long_prefill_tp8_share")]) == [4096]
    assert "<false>" in sel[("token_rows_shard", "long_prefill_tp8_share")][4096][0]["Kernel_Name"]


def test_memory_path_summary(tmp_path):
    """The memory-path counter summary takes each pass's per-dispatch rows, splits them into the bench's
    phases and reports medians for hipBLASLt and the engine on both prefill shares."""
    import csv
    names = [("gemm_bf16_wide_kernel<224, 3, false>(x)", 65536), ("Cijk_lib_prefill", 57344),
             ("gemm_w8a8_wide_kernel<224, 3, false>(x)", 65536), ("gemm_bf16_decode_kernel<2>(x)", 57344),
             ("read_ceiling_kernel(x)", 65536), ("gemm_bf16_wide_kernel<256, 3, false>(x)", 65536),
             ("Cijk_lib_long", 65536)]
    counters = {"mem_a": ["SQ_WAIT_ANY", "SQ_WAVE_CYCLES"], "mem_b": ["TA_TA_BUSY_sum"],
                "mem_c": ["TA_DATA_STALLED_BY_TC_CYCLES_sum"]}
    for sub, cs in counters.items():
        os.makedirs(tmp_path / sub)
        with open(tmp_path / sub / "run_counter_collection.csv", "w", newline="") as f:
            w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Grid_Size", "Counter_Name",
                                              "Counter_Value", "Start_Timestamp", "End_Timestamp"])
            w.writeheader()
            for i, (nm, g) in enumerate(names):
                for j, c in enumerate(cs):
                    kn = nm if nm.startswith("Cijk") else "void rpl::" + nm
                    w.writerow({"Dispatch_Id": i, "Kernel_Name": kn, "Grid_Size": g, "Counter_Name": c,
                                "Counter_Value": 10 * (i + 1) + j, "Start_Timestamp": 1000 * i,
                                "End_Timestamp": 1000 * i + 500})
    cmds = {k: f"cmd {k}" for k in counters}
    bench._memory_path_summary(str(tmp_path), cmds, out_dir=str(tmp_path))
    text = (tmp_path / "memory_path_counters__prefill_down_proj_7b.md").read_text()
    row = next(ln for ln in text.splitlines() if ln.startswith("SQ_WAIT_ANY"))
    # columns: lib prefill (dispatch 1), lib long (6), ours prefill (0), ours long (5)
    assert [float(v) for v in row.split()[1:]] == [20.0, 70.0, 10.0, 60.0]
    assert "cmd mem_b" in text and f"ours:long {60 / 61:.1%}" in text


def test_vendor_traffic(tmp_path):
    """The vendor GEMMs' HBM traffic comes from the same FETCH_SIZE / WRITE_SIZE passes, picked by phase,
    scaled by the copy calibration and set against the vendor problem's own algorithmic bytes."""
    import csv
    from row_matmul_reduce_amd import synth
    names = [("gemm_bf16_wide_kernel<224, 3, false>(x)", 65536), ("Cijk_lib_prefill", 57344),
             ("gemm_w8a8_wide_kernel<224, 3, false>(x)", 65536), ("Cijk_lib_int8", 57344),
             ("gemm_bf16_decode_kernel<2>(x)", 57344), ("read_ceiling_kernel(x)", 65536),
             ("gemm_bf16_wide_kernel<256, 3, false>(x)", 65536), ("Cijk_lib_long", 65536)]
    for sub, c in (("fetch", "FETCH_SIZE"), ("write", "WRITE_SIZE")):
        os.makedirs(tmp_path / sub)
        with open(tmp_path / sub / "run_counter_collection.csv", "w", newline="") as f:
            w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Grid_Size", "Counter_Name",
                                              "Counter_Value"])
            w.writeheader()
            for i, (nm, g) in enumerate(names):
                kn = nm if nm.startswith("Cijk") else "void rpl::" + nm
                w.writerow({"Dispatch_Id": i, "Kernel_Name": kn, "Grid_Size": g, "Counter_Name": c,
                            "Counter_Value": 1000 * (i + 1) if c == "FETCH_SIZE" else 100 * (i + 1)})
    wls = {wl.name: wl for wl in synth.WORKLOADS.values()}
    got = bench._vendor_traffic(str(tmp_path), wls, 2.0, 1.0)
    assert sorted(got) == ["hipblaslt_bf16@long_prefill_tp8_share", "hipblaslt_bf16@prefill_down_proj_7b",
                           "hipblaslt_int8@w8a8_prefill_down_proj_7b"]
    e = got["hipblaslt_int8@w8a8_prefill_down_proj_7b"]  # dispatch 3
    assert e["hbm_bytes_per_launch"] == 4000 * 1024 * 2.0 + 400 * 1024 * 1.0
    wl = wls["w8a8_prefill_down_proj_7b"]
    assert e["algorithmic_bytes"] == wl.m * wl.k_shard + wl.n * wl.k_shard + 4 * wl.m * wl.n
    assert got["hipblaslt_bf16@long_prefill_tp8_share"]["fetch_kib"] == 8000
