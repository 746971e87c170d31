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


def bf16_ulp(b: np.ndarray) -> np.ndarray:
    """One bf16 ulp at each value's magnitude: the quantum of its binade (2^(e-7) for |v| in
    [2^e, 2^(e+1)), the subnormal quantum 2^-133 below 2^-126 and at zero)."""
    v = np.abs(f64(b))
    e = np.floor(np.log2(np.where(v > 0, v, 1.0)))
    q = np.ldexp(1.0, (np.maximum(e, -126) - 7).astype(np.int64))
    return np.where(v > 0, q, 2.0 ** -133)


def assert_sum_close(got: np.ndarray, want: np.ndarray, parts, what: str, scale=1.0, atol=ATOL, rtol=RTOL):
    """The bf16 rule for an output that sums tp bf16 partials computed on each side: each
    partial is itself a bf16 value that may legitimately differ from the oracle's by one ulp
    (fp32 against fp64 accumulation, rule above), and the sum carries those differences
    undamped, so where the partials cancel the difference can exceed the rule relative to the
    small sum.  The bound adds one ulp of each oracle partial, times `scale` (the output's
    derivative with respect to the sum: 1 for residual_out, |gamma| / rms for y):
    |g - o| <= atol + rtol |o| + scale * sum_s ulp(P_s)."""
    g, o = f64(got), f64(want)
    assert g.shape == o.shape, (what, g.shape, o.shape)
    slack = np.zeros(o.shape)
    for p in parts:
        slack += bf16_ulp(p)
    both_nan = np.isnan(g) & np.isnan(o)
    err = np.where(both_nan, 0.0, np.abs(g - o))
    bound = atol + rtol * np.abs(o) + scale * slack
    bad = ~(err <= bound)
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} elements out of tolerance, "
                             f"max abs err {np.nanmax(err):.4g}; first {[tuple(i) for i in idx]}: "
                             f"gpu {[g[tuple(i)] for i in idx]} oracle {[o[tuple(i)] for i in idx]}")
    return int((err > atol + rtol * np.abs(o)).sum())


def y_scale(residual_out: np.ndarray, gamma: np.ndarray, eps: float) -> np.ndarray:
    """|gamma| / rms per element, the factor by which a difference in the sum h reaches y,
    from the oracle's residual_out (h rounded to bf16: its rms is within 2^-8 of h's, hence
    the margin)."""
    h = f64(residual_out)
    rms = np.sqrt(np.mean(h * h, axis=1, keepdims=True) + eps)
    return 1.01 * np.abs(f64(gamma))[None, :] / rms
