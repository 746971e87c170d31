"""Helpers shared by the GPU parity tests: host <-> device transfers of bf16
bit patterns and the element-wise tolerance check."""
from __future__ import annotations

import sys

import numpy as np

from row_matmul_reduce_amd import synth

# bf16 outputs: |gpu - oracle| <= ATOL + RTOL * |oracle| per element (max relative
# error 1e-2 and max absolute error 2e-2, combined so that a legitimate one-ulp
# bf16 disagreement -- fp32 vs fp64 sums straddling a rounding boundary -- passes
# at any magnitude; one bf16 ulp is at most 2^-7 of the value).
ATOL, RTOL = 2e-2, 1e-2
# w8a8 dequantised outputs: within 1e-3 relative (bit-exact under the fixed fp32 order).
W8A8_RTOL = 1e-3


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev_bf16(a: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()


def dev(a: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host_bf16(t) -> np.ndarray:
    import torch
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def f64(b: np.ndarray) -> np.ndarray:
    return synth.bf16_decode(b).astype(np.float64)


def assert_bf16_close(got: np.ndarray, want: np.ndarray, what: str, atol=ATOL, rtol=RTOL):
    g, o = f64(got), f64(want)
    assert g.shape == o.shape, (what, g.shape, o.shape)
    both_nan = np.isnan(g) & np.isnan(o)
    err = np.where(both_nan, 0.0, np.abs(g - o))
    bound = atol + rtol * np.abs(o)
    bad = ~(err <= bound)
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} elements out of tolerance, "
                             f"max abs err {np.nanmax(err):.4g}; first {[tuple(i) for i in idx]}: "
                             f"gpu {[g[tuple(i)] for i in idx]} oracle {[o[tuple(i)] for i in idx]}")
    return float(np.max(err)) if err.size else 0.0


def assert_rel(got: np.ndarray, want: np.ndarray, what: str, rtol=W8A8_RTOL):
    g, o = f64(got), f64(want)
    bad = ~(np.abs(g - o) <= rtol * np.abs(o))
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError(f"{what}: {int(bad.sum())} elements beyond {rtol} relative; first "
                             f"{[tuple(i) for i in idx]} gpu {[g[tuple(i)] for i in idx]} "
                             f"oracle {[o[tuple(i)] for i in idx]}")
