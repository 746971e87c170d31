"""Seeded synthetic inputs for the row-parallel matmul + reduce path.

This module only draws and encodes random inputs.  It holds none of the
method's arithmetic (no products, sums, norms or dequantisation); the CPU
oracle and the HIP path both consume the bytes it returns.

Every tensor comes from its own numpy stream ``default_rng([seed, workload,
tensor, shard])`` with the tensor ids below, drawn row-major in fp32 and, for
bf16 tensors, rounded to bfloat16 (nearest, ties to even).  Because draws are
row-major, the first ``r`` rows of a shard drawn alone equal the first ``r``
rows of the full draw -- so the other ranks' token chunk 0 needs only their
first ``m_chunk`` rows.

The five named workloads are one tensor-parallel rank's share of the
RowParallelLinear layers that the pages discuss (a 7B-class o_proj at decode
and down_proj at prefill, a TP=8 long-prefill share, and a w8a8_dynamic
quantised variant).  The pages measure end-to-end on serving benchmarks that
are not available; these synthetic tensors of the same shapes stand in for them.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

T_X, T_W, T_RESID, T_GAMMA, T_WSCALE, T_XFP = 0, 1, 2, 3, 4, 5
DEFAULT_SEED = 0
DEFAULT_EPS = 1e-6


@dataclass(frozen=True)
class Workload:
    """One TP rank's share: X_s [m, k_shard], W_s [n, k_shard]; reduce of chunk 0."""

    wid: int
    name: str
    m: int
    k_full: int
    tp: int
    n: int
    kind: str = "bf16"          # "bf16" or "w8a8"
    x_dist: str = "normal"      # normal | normal_over_sqrtk | silu
    w_std: float = 0.02         # for bf16 W; "sqrtk" handled by x_dist normal_over_sqrtk
    w_over_sqrtk: bool = False
    eps: float = DEFAULT_EPS
    seed: int = DEFAULT_SEED

    @property
    def k_shard(self) -> int:
        return self.k_full // self.tp

    @property
    def m_pad(self) -> int:
        return -(-self.m // self.tp) * self.tp

    @property
    def m_chunk(self) -> int:
        return self.m_pad // self.tp

    def gemm_flops(self) -> float:
        """Algorithmic FLOP (or integer OP) count of the rank's partial."""
        return 2.0 * self.m * self.k_shard * self.n

    def partial_bytes(self) -> int:
        """Algorithmic HBM bytes of the rank's partial (each operand once)."""
        if self.kind == "w8a8":
            return (self.m * self.k_shard + self.n * self.k_shard + 4 * self.m + 4 * self.n
                    + 2 * self.m_pad * self.n)
        return 2 * (self.m * self.k_shard + self.n * self.k_shard + self.m_pad * self.n)

    def quant_bytes(self) -> int:
        """Algorithmic HBM bytes of the per-token quantiser of the rank's activation."""
        return 3 * self.m * self.k_shard + 4 * self.m

    def reduce_bytes(self) -> int:
        """Algorithmic HBM bytes of the chunk reduce + residual + RMSNorm."""
        mc, n = self.m_chunk, self.n
        return 2 * (self.tp * mc * n + mc * n + n + 2 * mc * n)

    def describe(self) -> dict:
        return {"workload": self.name, "m": self.m, "k_full": self.k_full, "tp": self.tp,
                "k_shard": self.k_shard, "n": self.n, "m_chunk": self.m_chunk,
                "kind": self.kind, "seed": self.seed}


WORKLOADS = {
    1: Workload(1, "tiny", m=64, k_full=512, tp=2, n=512, x_dist="normal_over_sqrtk",
                w_over_sqrtk=True),
    2: Workload(2, "decode_o_proj_7b", m=8, k_full=3584, tp=2, n=3584),
    3: Workload(3, "prefill_down_proj_7b", m=4096, k_full=18944, tp=2, n=3584, x_dist="silu"),
    4: Workload(4, "long_prefill_tp8_share", m=16384, k_full=25600, tp=8, n=5120),
    5: Workload(5, "w8a8_prefill_down_proj_7b", m=4096, k_full=18944, tp=2, n=3584, kind="w8a8"),
}


def custom(m: int, n: int, k_full: int, tp: int, seed: int = 1, kind: str = "bf16",
           x_dist: str = "normal_over_sqrtk", w_over_sqrtk: bool = True, wid: int = 99,
           eps: float = DEFAULT_EPS) -> Workload:
    """A workload of arbitrary shape (for ragged/edge-case parity tests)."""
    if k_full % tp:
        raise ValueError("k_full must split evenly over tp")
    return Workload(wid, f"custom_m{m}_n{n}_k{k_full}_tp{tp}", m=m, k_full=k_full, tp=tp, n=n,
                    kind=kind, x_dist=x_dist, w_over_sqrtk=w_over_sqrtk, eps=eps, seed=seed)


# ------------------------------------------------------------------ encoding
def bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp32 -> bfloat16 bit patterns, round to nearest, ties to even (finite input)."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    if not np.all(np.isfinite(a)):
        raise ValueError("synthetic inputs must be finite")
    u = a.view(np.uint32).astype(np.uint64)
    bias = ((u >> 16) & 1) + 0x7FFF
    return ((u + bias) >> 16).astype(np.uint16)


def bf16_decode(b: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> float32 (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _rng(wl: Workload, tensor: int, shard: int = 0) -> np.random.Generator:
    return np.random.default_rng([wl.seed, wl.wid, tensor, shard])


# ------------------------------------------------------------------ bf16 path
def x_shard(wl: Workload, s: int, rows: int | None = None) -> np.ndarray:
    """Rank s's activation shard X_s [rows, k_shard] as bf16 bits (default rows = m)."""
    r = wl.m if rows is None else min(rows, wl.m)
    z = _rng(wl, T_X, s).standard_normal((r, wl.k_shard), dtype=np.float32)
    if wl.x_dist == "normal":
        v = z
    elif wl.x_dist == "normal_over_sqrtk":
        v = z / np.float32(np.sqrt(wl.k_full))
    elif wl.x_dist == "silu":
        # a SiLU-shaped activation distribution: z * sigmoid(z)
        v = z / (np.float32(1.0) + np.exp(-z))
    else:
        raise ValueError(wl.x_dist)
    return bf16_bits(v)


def w_shard(wl: Workload, s: int) -> np.ndarray:
    """Rank s's weight shard W_s [n, k_shard] (nn.Linear layout) as bf16 bits."""
    z = _rng(wl, T_W, s).standard_normal((wl.n, wl.k_shard), dtype=np.float32)
    if wl.w_over_sqrtk:
        v = z / np.float32(np.sqrt(wl.k_full))
    else:
        v = z * np.float32(wl.w_std)
    return bf16_bits(v)


def residual_chunk(wl: Workload) -> np.ndarray:
    """The receiving rank's residual chunk [m_chunk, n], bf16 N(0,1)."""
    z = _rng(wl, T_RESID, 0).standard_normal((wl.m_chunk, wl.n), dtype=np.float32)
    return bf16_bits(z)


def gamma(wl: Workload) -> np.ndarray:
    """RMSNorm weight [n], bf16 U(0.5, 1.5)."""
    g = _rng(wl, T_GAMMA, 0).uniform(0.5, 1.5, wl.n).astype(np.float32)
    return bf16_bits(g)


# ------------------------------------------------------------------ w8a8 path
def w8a8_inputs(wl: Workload, rows: int | None = None, shard: int = 0):
    """int8 activations with a per-token fp32 scale, int8 weights with a
    per-channel fp32 scale.

    The activations are synthesised as a per-token symmetric int8 encoding of
    N(0,1) data: scale = row absmax / 127 (fp32), code = round-half-even of
    x / scale clamped to [-127, 127].  This is how the int8 tensor and its scale
    are made, not a step of the path (the path consumes codes and scales).
    Returns (xq [r, k] int8, sx [r] fp32, wq [n, k] int8, sw [n] fp32) of rank `shard`.
    """
    r = wl.m if rows is None else min(rows, wl.m)
    xf = _rng(wl, T_XFP, shard).standard_normal((r, wl.k_shard), dtype=np.float32)
    absmax = np.max(np.abs(xf), axis=1)
    sx = (absmax / np.float32(127.0)).astype(np.float32)
    live = sx > 0  # an all-zero row (never drawn from N(0,1)) keeps scale 0 and codes 0
    q = np.rint(xf / np.where(live, sx, np.float32(1.0))[:, None]) * live[:, None]
    xq = np.clip(q, -127, 127).astype(np.int8)
    wq, sw = w8a8_weight(wl, shard)
    return np.ascontiguousarray(xq), sx, wq, sw


def w8a8_weight(wl: Workload, shard: int = 0):
    """Rank `shard`'s int8 weight [n, k_shard] (uniform over -127..127) and its
    per-channel fp32 scale [n] ~ U(1e-3, 1e-2)."""
    wq = _rng(wl, T_W, shard).integers(-127, 128, (wl.n, wl.k_shard), dtype=np.int8)
    sw = _rng(wl, T_WSCALE, shard).uniform(1e-3, 1e-2, wl.n).astype(np.float32)
    return np.ascontiguousarray(wq), sw


def quant_test_rows(m: int, k: int, seed: int) -> np.ndarray:
    """bf16 rows [m, k] for the per-token quantiser: N(0,1) rows scaled by
    10^U(-30, 30), with special rows cycled in: all zero, bf16-subnormal
    magnitudes, near the bf16 maximum, half-integers up to 126.5 with absmax
    127 (exact ties), a single non-zero element, a constant row, a run of
    consecutive bf16 codes (every value of the run), and small-significand
    values under a small-significand absmax (many quotients at or next to
    half-integers)."""
    rng = np.random.default_rng([seed, 7])
    z = rng.standard_normal((m, k), dtype=np.float32)
    mag = (10.0 ** rng.uniform(-30, 30, (m, 1))).astype(np.float32)
    v = z * mag
    for r in range(m):
        kind = r % 9
        if kind == 1:
            v[r] = 0.0
        elif kind == 2:
            v[r] = z[r] * np.float32(2.0 ** -130)
        elif kind == 3:
            v[r] = np.clip(z[r], -1.5, 1.5) * np.float32(2.0e38)
        elif kind == 4:
            v[r] = rng.integers(-127, 127, k).astype(np.float32) + np.float32(0.5)
            v[r, rng.integers(0, k)] = -127.0
        elif kind == 5:
            v[r] = 0.0
            v[r, rng.integers(0, k)] = z[r, 0]
        elif kind == 6:
            v[r] = np.float32(-0.375)
    b = bf16_bits(v)
    for r in range(7, m, 9):
        # every bf16 value of a run of consecutive codes below a random start, signs alternating
        start = int(bf16_bits(np.abs(v[r, :1]))[0])
        run = np.maximum(start - np.arange(k), 0).astype(np.uint16)
        run[1::2] |= np.uint16(0x8000)
        b[r] = run
    for r in range(8, m, 9):
        # small-significand values: absmax c * 2^e (c odd, 1..15), elements (odd j) * 2^(e - q)
        e = int(rng.integers(-40, 40))
        c = float(rng.choice([1, 3, 5, 7, 9, 11, 13, 15]))
        j = rng.integers(0, 128, k) * 2 + 1
        q = rng.integers(4, 12, k)
        row = (j * np.exp2(e - q.astype(np.float64))).astype(np.float32)
        row = np.minimum(row, np.float32(c * 2.0 ** e)) * np.where(rng.random(k) < 0.5, -1, 1).astype(np.float32)
        row[int(rng.integers(0, k))] = np.float32(c * 2.0 ** e)
        b[r] = bf16_bits(row)
    return b
