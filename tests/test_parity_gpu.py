"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Same seeded inputs on both sides.  bf16 outputs must satisfy
|gpu - oracle| <= 2e-2 + 1e-2 |oracle| element-wise; integer-valued cases must
be bit-exact; w8a8 int32 accumulators must be bit-exact and their dequantised
bf16 outputs within 1e-3 relative.  Small shapes are compared in full (several
tiles plus ragged tails); the full-size workloads run in the same launch
configuration as bench.py and are compared element by element too (the oracle's
products of a workload are computed once per session and shared by the tests
that need them).
"""
import numpy as np
import pytest

import oracle
import row_matmul_reduce_amd as rpl
from row_matmul_reduce_amd import synth
from gpu_util import (assert_bf16_close, assert_rel, assert_sum_close, dev, dev_bf16, f64, host_bf16, say,
                      y_scale)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    rpl.lib()


def shards(x_full, w_full, tp):
    ks = x_full.shape[1] // tp
    return [(np.ascontiguousarray(x_full[:, s * ks:(s + 1) * ks]),
             np.ascontiguousarray(w_full[:, s * ks:(s + 1) * ks])) for s in range(tp)]


# (m, n, k_full, tp): ragged m, n, K; pad rows; both kernels; full and partial tiles
SMALL_SHAPES = [
    (64, 512, 512, 2),     # the tiny workload's shape
    (5, 24, 32, 2),        # m not divisible by tp: one zero pad row (decode kernel)
    (3, 40, 64, 4),        # decode kernel, ragged column tile
    (16, 264, 2048, 2),    # decode kernel at m_pad = 16, K split over every wave
    (4, 136, 4000, 2),     # decode kernel, m_pad = 4: four K steps per activation load, K tail
    (7, 72, 2608, 2),      # decode kernel, m_pad = 8: two K steps per activation load, K tail
    (2, 24, 1040, 1),      # decode kernel, m_pad = 2, 32.5 K steps
    (8, 3584, 3584, 2),    # decode o_proj shape
    (8, 3576, 3584, 2),    # decode kernel, the last 16-column block 8 wide
    (6, 5120, 2048, 2),    # decode kernel, 320 workgroups (more than the CUs)
    (3, 4104, 512, 1),     # decode kernel, the last 16-column block 8 wide, m_pad = 3
    (17, 64, 128, 8),      # tile kernel with bounds checks, m_pad = 24, a single K step
    (300, 520, 656, 2),    # ragged m, n and K (k_shard = 328)
    (257, 264, 288, 4),    # m_pad = 260: one row past a 256-row tile
    (512, 448, 256, 2),    # whole 256 x 224 tiles (no bounds checks)
    (512, 512, 512, 4),    # 2 x 3 tiles of 256 x 224, the last tile column 64 wide
    (4100, 4104, 272, 2),  # 17 x 19 = 323 tiles > 256 workgroups: some run two; ragged m, n, K; 3 K steps
    (8192, 3584, 128, 2),  # 512 tiles of 256 x 224: every workgroup runs two tiles of one K step
    (4100, 4480, 256, 2),  # 17 x 20 = 340 tiles, some workgroups run two; 2 K steps per tile
    (9211, 1784, 512, 2),  # 36 x 7 = 252 tiles of 256 x 256 (one round, where 256 x 224 needs two):
                           # the 256-wide engine with ragged rows and columns
]


@pytest.mark.parametrize("m,n,k_full,tp", SMALL_SHAPES)
def test_partial_small(m, n, k_full, tp):
    say(f"[partial] m={m} n={n} k_full={k_full} tp={tp}")
    wl = synth.custom(m, n, k_full, tp, seed=m + n)
    x_full = np.concatenate([synth.x_shard(wl, s) for s in range(tp)], axis=1)
    w_full = np.concatenate([synth.w_shard(wl, s) for s in range(tp)], axis=1)
    xd, wd = dev_bf16(x_full), dev_bf16(w_full)
    ks = wl.k_shard
    for s, (xs, ws) in enumerate(shards(x_full, w_full, tp)):
        want = oracle.partial_rows(xs, ws, m, tp=tp)
        got = host_bf16(rpl.rpl_partial(dev_bf16(xs), dev_bf16(ws), tp))
        assert_bf16_close(got, want, f"shard {s} contiguous")
        # the same shard as strided column views of the unsharded tensors (ld = k_full)
        got_v = host_bf16(rpl.rpl_partial(xd[:, s * ks:(s + 1) * ks], wd[:, s * ks:(s + 1) * ks], tp))
        assert np.array_equal(got_v, got), "strided views must give the same bits"
        assert np.all(got[m:] == 0), "pad rows must be zero"


@pytest.mark.parametrize("m,n,k", [(8, 64, 64), (13, 48, 96), (3, 40, 1000), (7, 56, 2056), (300, 264, 272),
                                   (512, 512, 256)])
def test_partial_exact_cases(m, n, k):
    say(f"[exact] m={m} n={n} k={k}")
    rng = np.random.default_rng(m * n)
    # one-hot activation rows pick weight columns exactly
    cols = rng.integers(0, k, m)
    xo = np.zeros((m, k), np.float32)
    xo[np.arange(m), cols] = 1.0
    w = synth.bf16_bits(rng.standard_normal((n, k)).astype(np.float32))
    got = host_bf16(rpl.rpl_partial(dev_bf16(synth.bf16_bits(xo)), dev_bf16(w), 1))
    assert np.array_equal(got, w[:, cols].T)
    # small integers: every partial sum is an integer below 2^24, exact in fp32 in any order
    xi = rng.integers(-2, 3, (m, k)).astype(np.float32)
    wi = rng.integers(-2, 3, (n, k)).astype(np.float32)
    got = host_bf16(rpl.rpl_partial(dev_bf16(synth.bf16_bits(xi)), dev_bf16(synth.bf16_bits(wi)), 1))
    want = oracle.partial_rows(synth.bf16_bits(xi), synth.bf16_bits(wi), m)
    assert np.array_equal(got, want)


# oracle products of the full-size workloads, computed once per session
_ORACLE = {}


def oracle_rank_partial(wl):
    """The oracle's rank-0 partial of a workload, all M_pad rows."""
    key = ("rank", wl.name)
    if key not in _ORACLE:
        say(f"  oracle: rank partial of {wl.name} ({wl.m} x {wl.n} x {wl.k_shard})")
        _ORACLE[key] = oracle.partial_rows(synth.x_shard(wl, 0), synth.w_shard(wl, 0), wl.m, tp=wl.tp)
    return _ORACLE[key]


def oracle_peer_chunk(wl, s):
    """The oracle's chunk-0 partial of peer shard s (its first m_chunk rows)."""
    key = ("peer", wl.name, s)
    if key not in _ORACLE:
        say(f"  oracle: peer {s} chunk partial of {wl.name}")
        _ORACLE[key] = oracle.partial_rows(synth.x_shard(wl, s, rows=wl.m_chunk), synth.w_shard(wl, s),
                                           wl.m_chunk)
    return _ORACLE[key]


@pytest.mark.parametrize("wid", [2, 3, 4])
def test_partial_full_size(wid):
    """Every output element of the rank partial at the workload's full size."""
    wl = synth.WORKLOADS[wid]
    say(f"[partial full] {wl.name}")
    x, w = synth.x_shard(wl, 0), synth.w_shard(wl, 0)
    out = rpl.rpl_partial(dev_bf16(x), dev_bf16(w), wl.tp)
    got = host_bf16(out)
    assert got.shape == (wl.m_pad, wl.n)
    want = oracle_rank_partial(wl)
    err = assert_bf16_close(got, want, f"{wl.name} all elements")
    say(f"  max abs err {err:.3g} over {got.size} elements")
    assert np.all(np.isfinite(f64(got)))


def test_partial_deterministic():
    wl = synth.WORKLOADS[3]
    x, w = dev_bf16(synth.x_shard(wl, 0)), dev_bf16(synth.w_shard(wl, 0))
    a = host_bf16(rpl.rpl_partial(x, w, wl.tp))
    b = host_bf16(rpl.rpl_partial(x, w, wl.tp))
    assert np.array_equal(a, b)


def test_empty_batch():
    import torch
    w = torch.zeros(64, 32, dtype=torch.bfloat16, device="cuda")
    x = torch.zeros(0, 32, dtype=torch.bfloat16, device="cuda")
    out = rpl.rpl_partial(x, w, 2)
    assert tuple(out.shape) == (0, 64)


# ---------------------------------------------------------------------- reduce
# (tp, m_chunk, n): up to 511 rows each row is spread over 8 waves (1-4 chunks per lane); from 512
# rows one wave per row (1-8 chunks per lane) or, above 4096 columns, 4 waves per row
REDUCE_SHAPES = [(1, 3, 8), (2, 5, 64), (3, 7, 3584), (8, 33, 5120), (16, 2, 8192), (2, 4, 8200),
                 (4, 3, 16384), (2, 1, 520), (8, 130, 1024), (2, 511, 3584),
                 (2, 512, 64), (3, 600, 1032), (2, 517, 2056), (2, 520, 4096), (4, 700, 4104), (2, 513, 16384)]


@pytest.mark.parametrize("tp,mc,n", REDUCE_SHAPES)
def test_reduce_on_oracle_partials(tp, mc, n):
    say(f"[reduce] tp={tp} m_chunk={mc} n={n}")
    rng = np.random.default_rng(tp * 1000 + n)
    parts = [synth.bf16_bits(rng.standard_normal((mc, n)).astype(np.float32) * 1.3) for _ in range(tp)]
    res = synth.bf16_bits(rng.standard_normal((mc, n)).astype(np.float32))
    gam = synth.bf16_bits(rng.uniform(0.5, 1.5, n).astype(np.float32))
    y, ro = rpl.rpl_reduce_chunk_rmsnorm([dev_bf16(p) for p in parts], dev_bf16(res), dev_bf16(gam), 1e-6)
    wy, wro = oracle.reduce_chunk_rmsnorm(parts, res, gam, 1e-6)
    assert_bf16_close(host_bf16(ro), wro, "residual_out")
    assert_bf16_close(host_bf16(y), wy, "y")


def test_reduce_integer_partials_exact_and_inplace():
    import torch
    rng = np.random.default_rng(5)
    tp, mc, n = 8, 9, 3584
    ints = [rng.integers(-40, 41, (mc, n)).astype(np.float32) for _ in range(tp)]
    ri = rng.integers(-40, 41, (mc, n)).astype(np.float32)
    parts = [synth.bf16_bits(a) for a in ints]
    res = synth.bf16_bits(ri)
    gam = synth.bf16_bits(rng.uniform(0.5, 1.5, n).astype(np.float32))
    rd = dev_bf16(res)
    y = torch.empty_like(rd)
    rpl.rpl_reduce_chunk_rmsnorm([dev_bf16(p) for p in parts], rd, dev_bf16(gam), 1e-6, y=y, residual_out=rd)
    wy, wro = oracle.reduce_chunk_rmsnorm(parts, res, gam, 1e-6)
    assert np.array_equal(host_bf16(rd), wro), "integer sums are exact; residual updated in place"
    assert_bf16_close(host_bf16(y), wy, "y")


def test_reduce_zero_row_and_unit_rms():
    rng = np.random.default_rng(9)
    mc, n = 4, 512
    p = synth.bf16_bits(rng.standard_normal((mc, n)).astype(np.float32))
    p[2] = 0
    res = synth.bf16_bits(rng.standard_normal((mc, n)).astype(np.float32))
    res[2] = 0
    ones = synth.bf16_bits(np.ones(n, np.float32))
    y, ro = rpl.rpl_reduce_chunk_rmsnorm([dev_bf16(p)], dev_bf16(res), dev_bf16(ones), 0.0)
    yh = f64(host_bf16(y))
    assert np.all(np.isnan(yh[2])) or np.all(yh[2] == 0)  # 0/0 with eps = 0
    rms = np.sqrt(np.mean(yh[[0, 1, 3]] ** 2, axis=1))
    assert np.all(np.abs(rms - 1.0) < 2.0 ** -7)
    y2, _ = rpl.rpl_reduce_chunk_rmsnorm([dev_bf16(p)], dev_bf16(res), dev_bf16(ones), 1e-6)
    assert np.all(f64(host_bf16(y2))[2] == 0)


@pytest.mark.parametrize("wid", [1, 2, 3, 4])
def test_received_chunk_end_to_end(wid):
    """Rank 0's step: own partial + every peer's chunk-0 partial -> reduce + RMSNorm, every
    element.  Stage by stage against the oracle: each partial (bf16 rule), then the reduce and
    RMSNorm on the very partials the GPU produced (bf16 rule); and end to end against the
    oracle's own partials, where the bound adds one bf16 ulp per summed partial (two sides'
    partials may each differ by one ulp, and the sum keeps those differences)."""
    wl = synth.WORKLOADS[wid]
    say(f"[end-to-end] {wl.name}")
    mc = wl.m_chunk
    xs = [synth.x_shard(wl, 0)] + [synth.x_shard(wl, s, rows=mc) for s in range(1, wl.tp)]
    ws = [synth.w_shard(wl, s) for s in range(wl.tp)]
    res, gam = synth.residual_chunk(wl), synth.gamma(wl)
    own = rpl.rpl_partial(dev_bf16(xs[0]), dev_bf16(ws[0]), wl.tp)
    chunks = [own[:mc]] + [rpl.rpl_partial(dev_bf16(xs[s]), dev_bf16(ws[s]), 1) for s in range(1, wl.tp)]
    y, ro = rpl.rpl_reduce_chunk_rmsnorm(chunks, dev_bf16(res), dev_bf16(gam), wl.eps)
    if mc <= 64:
        o_parts = [oracle.partial_rows(xs[s], ws[s], wl.m if s == 0 else mc, rows=np.arange(mc),
                                       tp=wl.tp if s == 0 else 1) for s in range(wl.tp)]
    else:  # every row of the chunk, from the session's oracle products
        o_parts = [np.ascontiguousarray(oracle_rank_partial(wl)[:mc])]
        o_parts += [oracle_peer_chunk(wl, s) for s in range(1, wl.tp)]
    g_parts = [host_bf16(c) for c in chunks]
    for s in range(wl.tp):
        assert_bf16_close(g_parts[s], o_parts[s], f"{wl.name} shard {s} chunk partial")
    gy, gro = host_bf16(y), host_bf16(ro)
    # the reduce + RMSNorm on the GPU's own partials
    wy_g, wro_g = oracle.reduce_chunk_rmsnorm(g_parts, res, gam, wl.eps)
    e1 = assert_bf16_close(gro, wro_g, f"{wl.name} residual_out on the GPU partials")
    e2 = assert_bf16_close(gy, wy_g, f"{wl.name} y on the GPU partials")
    # end to end against the oracle's partials
    wy, wro = oracle.reduce_chunk_rmsnorm(o_parts, res, gam, wl.eps)
    n1 = assert_sum_close(gro, wro, o_parts, f"{wl.name} residual_out end to end")
    n2 = assert_sum_close(gy, wy, o_parts, f"{wl.name} y end to end", scale=y_scale(wro, gam, wl.eps))
    say(f"  max abs err on the GPU partials: residual_out {e1:.3g} y {e2:.3g}; end to end {n1} + {n2} of "
        f"{gro.size} elements need the per-partial ulp term, all rows")


def test_partial_row_stride_at_the_limit():
    """Row strides just under the 8 MiB the tile engine's 32-bit buffer offsets allow
    (255 rows x stride must stay below 2^31 bytes): a 256-row tile's last rows are read."""
    import torch
    m, n, k = 300, 264, 64
    ldx = (1 << 22) - 8                      # elements: 8 MiB - 16 bytes per row
    rng = np.random.default_rng(21)
    x = synth.bf16_bits(rng.standard_normal((m, k), dtype=np.float32) / np.float32(8.0))
    w = synth.bf16_bits(rng.standard_normal((n, k), dtype=np.float32) / np.float32(8.0))
    say(f"[partial ld limit] m={m} ldx={ldx}")
    big = torch.zeros((m, ldx), dtype=torch.bfloat16, device="cuda")
    big[:, :k] = dev_bf16(x)
    out = rpl.rpl_partial(big[:, :k], dev_bf16(w), 2)
    assert_bf16_close(host_bf16(out)[:m], oracle.partial_rows(x, w, m), "partial at the stride limit")
    del big
    xq = rng.integers(-127, 128, (m, 64), dtype=np.int8)
    wq = rng.integers(-127, 128, (n, 64), dtype=np.int8)
    sx = rng.uniform(1e-3, 2e-2, m).astype(np.float32)
    sw = rng.uniform(1e-3, 1e-2, n).astype(np.float32)
    bq = torch.zeros((m, (1 << 23) - 16), dtype=torch.int8, device="cuda")
    bq[:, :64] = dev(xq)
    _, acc = rpl.rpl_w8a8_partial(bq[:, :64], dev(sx), dev(wq), dev(sw), 2, want_acc=True)
    _, wacc = oracle.w8a8_rows(xq, sx, wq, sw, m, tp=2)
    assert np.array_equal(acc.cpu().numpy(), wacc)


# ------------------------------------------------------------------------ w8a8
# the last two run more tiles than workgroups, so the scale staging alternates between its two LDS
# areas (two tiles of two K steps; three tiles of one K step)
W8A8_SHAPES = [(64, 512, 256, 2), (5, 24, 32, 2), (17, 40, 64, 8), (300, 520, 672, 2), (257, 264, 272, 4),
               (512, 448, 256, 2), (512, 512, 512, 4), (4100, 4104, 160, 2), (8192, 5376, 48, 2)]


def _w8a8_inputs(m, n, k, seed):
    rng = np.random.default_rng(seed)
    xq = rng.integers(-127, 128, (m, k), dtype=np.int8)
    wq = rng.integers(-127, 128, (n, k), dtype=np.int8)
    sx = rng.uniform(1e-3, 2e-2, m).astype(np.float32)
    sw = rng.uniform(1e-3, 1e-2, n).astype(np.float32)
    return xq, sx, wq, sw


@pytest.mark.parametrize("m,n,k,tp", W8A8_SHAPES)
def test_w8a8_small(m, n, k, tp):
    say(f"[w8a8] m={m} n={n} k={k} tp={tp}")
    xq, sx, wq, sw = _w8a8_inputs(m, n, k, m + n + k)
    out, acc = rpl.rpl_w8a8_partial(dev(xq), dev(sx), dev(wq), dev(sw), tp, want_acc=True)
    wout, wacc = oracle.w8a8_rows(xq, sx, wq, sw, m, tp=tp)
    assert np.array_equal(acc.cpu().numpy(), wacc), "int32 accumulators must be bit-exact"
    assert_rel(host_bf16(out), wout, "dequantised output")
    # without the accumulator store the output is identical
    out2 = rpl.rpl_w8a8_partial(dev(xq), dev(sx), dev(wq), dev(sw), tp)
    assert np.array_equal(host_bf16(out2), host_bf16(out))


def test_w8a8_near_int32_limit():
    m, n, k = 32, 16, 131056
    xq = np.full((m, k), 127, np.int8)
    xq[1::2] = -127
    wq = np.full((n, k), 127, np.int8)
    sx = np.full(m, 1e-3, np.float32)
    sw = np.full(n, 1e-3, np.float32)
    out, acc = rpl.rpl_w8a8_partial(dev(xq), dev(sx), dev(wq), dev(sw), 1, want_acc=True)
    wout, wacc = oracle.w8a8_rows(xq, sx, wq, sw, m)
    assert int(np.abs(wacc).max()) == 127 * 127 * k
    assert np.array_equal(acc.cpu().numpy(), wacc)
    assert_rel(host_bf16(out), wout, "dequantised output")


def test_w8a8_full_size():
    """Every int32 accumulator and every dequantised output of the w8a8 workload."""
    wl = synth.WORKLOADS[5]
    say(f"[w8a8 full] {wl.name}")
    xq, sx, wq, sw = synth.w8a8_inputs(wl)
    out, acc = rpl.rpl_w8a8_partial(dev(xq), dev(sx), dev(wq), dev(sw), wl.tp, want_acc=True)
    say(f"  oracle: w8a8 rank partial of {wl.name}")
    wout, wacc = oracle.w8a8_rows(xq, sx, wq, sw, wl.m, tp=wl.tp)
    assert np.array_equal(acc.cpu().numpy(), wacc), "int32 accumulators must be bit-exact"
    assert_rel(host_bf16(out), wout, "dequantised output")
    assert np.array_equal(host_bf16(out), wout), "dequantised output bit-exact under the pinned fp32 order"
    # the timed configuration (no accumulator store) gives the same output bits
    out2 = rpl.rpl_w8a8_partial(dev(xq), dev(sx), dev(wq), dev(sw), wl.tp)
    assert np.array_equal(host_bf16(out2), host_bf16(out))
