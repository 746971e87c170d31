"""GPU parity of the single-launch decode path (rpl_matmul_reduce_rmsnorm)
through the C ABI, against the CPU oracle's unfused composition: a bf16
partial per shard (oracle.partial_rows), then the sum of the partials,
residual add and RMSNorm (oracle.reduce_chunk_rmsnorm).  Outputs follow the
bf16 rule |gpu - oracle| <= 2e-2 + 1e-2 |oracle|, plus one bf16 ulp of each
summed partial (each shard's product is a bf16 value that may differ from the
oracle's by one ulp; the sum keeps that difference); repeated calls on one
workspace must give identical bits and leave its status word at zero.
"""
import numpy as np
import pytest

import oracle
import row_matmul_reduce_amd as rpl
from row_matmul_reduce_amd import synth
from gpu_util import assert_bf16_close, assert_sum_close, dev_bf16, host_bf16, say, y_scale

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    rpl.lib()


def _oracle_step(xs, ws, m, residual, gamma, eps):
    """Unfused composition on the CPU: per-shard bf16 partials of the m rows (rows past the
    given activation rows are padding), then sum + residual + RMSNorm.  Returns (y,
    residual_out, partials)."""
    parts = []
    for x, w in zip(xs, ws):
        xpad = np.zeros((m, w.shape[1]), dtype=np.uint16)
        xpad[: x.shape[0]] = x
        parts.append(oracle.partial_rows(xpad, w, m))
    y, ro = oracle.reduce_chunk_rmsnorm(parts, residual, gamma, eps)
    return y, ro, parts


def _check_step(y, ro, want, gamma, eps, what=""):
    """The single-launch outputs against the oracle's composition.  Each shard's product is
    rounded to bf16 inside the launch, as on the wire; those products may each differ from the
    oracle's by one bf16 ulp, so the bound adds one ulp per summed partial (see
    gpu_util.assert_sum_close)."""
    wy, wro, parts = want
    assert_sum_close(host_bf16(ro), wro, parts, f"{what} residual_out")
    assert_sum_close(host_bf16(y), wy, parts, f"{what} y", scale=y_scale(wro, gamma, eps))
    return assert_bf16_close_max(host_bf16(ro), wro), assert_bf16_close_max(host_bf16(y), wy)


def assert_bf16_close_max(got, want):
    from gpu_util import f64
    return float(np.max(np.abs(f64(got) - f64(want)))) if got.size else 0.0


def _inputs(m, m_valid, n, k, tp, seed):
    wl = synth.custom(m=max(m_valid, 1), n=n, k_full=k * tp, tp=tp, seed=seed)
    xs = [synth.x_shard(wl, s)[:m_valid] for s in range(tp)]
    ws = [synth.w_shard(wl, s) for s in range(tp)]
    rng = np.random.default_rng([seed, 5])
    res = synth.bf16_bits(rng.standard_normal((m, n), dtype=np.float32))
    gam = synth.bf16_bits(rng.uniform(0.5, 1.5, n).astype(np.float32))
    return xs, ws, res, gam


# (m, m_valid, n, k, tp): one to four 16-row blocks and every activation packing (1-4, 5-8 and
# 9-16 rows), padding rows, ragged K steps, one to sixteen shards, rows from 8 to 8192 wide
# (the epilogue's threads own one to four quads of columns), the 910C operator's case (40 rows,
# hidden 2048, TP=2), and more
# (column block, shard) items than the launch has product workgroups, so each computes several
# (8 x 320 and 2 x 512 items, the widest rows 8192), with a half column block at the end
# (n % 16 == 8)
FUSED_SHAPES = [(1, 1, 8, 8, 1), (4, 4, 264, 1000, 2), (5, 3, 520, 328, 3), (12, 12, 200, 1064, 2),
                (16, 16, 512, 512, 2), (17, 17, 1024, 256, 4), (40, 40, 2048, 1024, 2), (64, 60, 136, 72, 8),
                (33, 0, 64, 64, 2), (4, 4, 72, 64, 16), (8, 8, 5120, 256, 8), (40, 37, 8192, 96, 2),
                (3, 3, 4104, 512, 3)]


@pytest.mark.parametrize("m,m_valid,n,k,tp", FUSED_SHAPES)
def test_fused_shapes(m, m_valid, n, k, tp):
    say(f"[fused] m={m} m_valid={m_valid} n={n} k={k} tp={tp}")
    xs, ws, res, gam = _inputs(m, m_valid, n, k, tp, seed=m + n + k + tp)
    eps = 1e-6
    y, ro = rpl.rpl_matmul_reduce_rmsnorm([dev_bf16(x) for x in xs], [dev_bf16(w) for w in ws], dev_bf16(res),
                                          dev_bf16(gam), eps)
    e1, e2 = _check_step(y, ro, _oracle_step(xs, ws, m, res, gam, eps), gam, eps)
    say(f"  max abs err residual_out {e1:.3g} y {e2:.3g}")


def test_fused_workspace_reuse_and_in_place():
    import torch
    m, n, k, tp = 8, 512, 256, 2
    xs, ws, res, gam = _inputs(m, m, n, k, tp, seed=3)
    dx, dw, dg = [dev_bf16(x) for x in xs], [dev_bf16(w) for w in ws], dev_bf16(gam)
    work = rpl.rpl_matmul_reduce_rmsnorm_workspace(m, n, tp)
    outs = []
    for _ in range(3):
        y, ro = rpl.rpl_matmul_reduce_rmsnorm(dx, dw, dev_bf16(res), dg, 1e-6, workspace=work)
        torch.cuda.synchronize()
        assert rpl.rpl_matmul_reduce_rmsnorm_status(work) == 0
        outs.append((host_bf16(y), host_bf16(ro)))
    for y, ro in outs[1:]:
        assert np.array_equal(y, outs[0][0]) and np.array_equal(ro, outs[0][1])
    # every call advances every workgroup's call count by one (the tag's source), whatever the grid
    counts = work[256:256 + 4 * 1024].view(torch.int32)
    assert bool((counts == 3).all())
    # residual_out may be the residual buffer itself
    r_in = dev_bf16(res)
    y2, ro2 = rpl.rpl_matmul_reduce_rmsnorm(dx, dw, r_in, dg, 1e-6, workspace=work, residual_out=r_in)
    assert ro2.data_ptr() == r_in.data_ptr()
    assert np.array_equal(host_bf16(r_in), outs[0][1]) and np.array_equal(host_bf16(y2), outs[0][0])


def test_fused_one_workspace_across_shapes():
    """Calls of different row counts, widths and shard counts share one workspace (sized for the
    largest): slots a call does not write keep older tags, which no later call may take."""
    import torch
    work = rpl.rpl_matmul_reduce_rmsnorm_workspace(16, 1024, 4)
    for i, (m, n, k, tp) in enumerate([(16, 1024, 256, 4), (4, 1024, 256, 2), (16, 1024, 128, 4), (9, 512, 64, 3),
                                       (16, 1024, 256, 4), (1, 8, 8, 1), (16, 1024, 64, 2)]):
        say(f"[fused shared workspace] call {i}: m={m} n={n} k={k} tp={tp}")
        xs, ws, res, gam = _inputs(m, m, n, k, tp, seed=40 + i)
        y, ro = rpl.rpl_matmul_reduce_rmsnorm([dev_bf16(x) for x in xs], [dev_bf16(w) for w in ws], dev_bf16(res),
                                              dev_bf16(gam), 1e-6, workspace=work)
        _check_step(y, ro, _oracle_step(xs, ws, m, res, gam, 1e-6), gam, 1e-6, f"call {i}")
    torch.cuda.synchronize()
    assert rpl.rpl_matmul_reduce_rmsnorm_status(work) == 0


def test_fused_wait_bound_reported():
    """A wait bound set from the host to a single re-read (no spin needed to test it): a workgroup
    that finds another's slot not yet written gives up, raises the status word and writes NaN to
    its y columns (and, if it was waiting for a product, hands on a NaN sum of squares, so every
    y that would depend on it is NaN as well); a y that is not NaN is right, the kernel exits
    normally, and after the bound is lifted the same workspace gives the full result again."""
    import torch
    m, n, k, tp = 4, 3584, 1792, 2
    xs, ws, res, gam = _inputs(m, m, n, k, tp, seed=8)
    dx, dw, dr, dg = [dev_bf16(x) for x in xs], [dev_bf16(w) for w in ws], dev_bf16(res), dev_bf16(gam)
    work = rpl.rpl_matmul_reduce_rmsnorm_workspace(m, n, tp)
    want = _oracle_step(xs, ws, m, res, gam, 1e-6)
    wy, wro, wparts = want
    rpl.rpl_matmul_reduce_rmsnorm_set_poll_bound(work, 1)
    y, ro = rpl.rpl_matmul_reduce_rmsnorm(dx, dw, dr, dg, 1e-6, workspace=work)
    torch.cuda.synchronize()
    status = rpl.rpl_matmul_reduce_rmsnorm_status(work)
    yh = host_bf16(y)
    nan_cols = np.isnan(synth.bf16_decode(yh)).any(axis=0)
    say(f"  bound of one re-read: status {status}, {int(nan_cols.sum())} of {n} columns NaN")
    if status == 0:
        assert not nan_cols.any()
    else:
        assert nan_cols.any()
    assert_sum_close(yh[:, ~nan_cols], wy[:, ~nan_cols], [p[:, ~nan_cols] for p in wparts],
                     "y outside the given-up columns", scale=y_scale(wro, gam, 1e-6)[:, ~nan_cols])
    rpl.rpl_matmul_reduce_rmsnorm_set_poll_bound(work, 0)
    work[8:12].zero_()
    y, ro = rpl.rpl_matmul_reduce_rmsnorm(dx, dw, dr, dg, 1e-6, workspace=work)
    torch.cuda.synchronize()
    assert rpl.rpl_matmul_reduce_rmsnorm_status(work) == 0
    _check_step(y, ro, want, gam, 1e-6, "after the bound is lifted")


def test_fused_equals_unfused_library_path():
    """Same rows through rpl_partial per shard + rpl_reduce_chunk_rmsnorm.  Both round each
    shard's product to bf16 and sum in fp32, but they split K over different numbers of waves,
    so single bf16 ulps may differ: compared with the bf16 rule."""
    m, n, k, tp = 16, 1024, 512, 4
    xs, ws, res, gam = _inputs(m, m, n, k, tp, seed=9)
    dx, dw = [dev_bf16(x) for x in xs], [dev_bf16(w) for w in ws]
    y, ro = rpl.rpl_matmul_reduce_rmsnorm(dx, dw, dev_bf16(res), dev_bf16(gam), 1e-6)
    parts = [rpl.rpl_partial(x, w, 1) for x, w in zip(dx, dw)]
    y2, ro2 = rpl.rpl_reduce_chunk_rmsnorm(parts, dev_bf16(res), dev_bf16(gam), 1e-6)
    assert_bf16_close(host_bf16(ro), host_bf16(ro2), "residual_out vs unfused")
    assert_bf16_close(host_bf16(y), host_bf16(y2), "y vs unfused")


@pytest.mark.parametrize("chunked", [True, False])
def test_fused_decode_workload(chunked):
    """The decode o_proj share: rank 0's token chunk (reduce-scatter form) or all rows
    (all-reduce form), both TP shards' products in the one launch."""
    wl = synth.WORKLOADS[2]
    rows = wl.m_chunk if chunked else wl.m
    say(f"[fused decode] {wl.name} rows={rows}")
    xs = [synth.x_shard(wl, s, rows=rows) for s in range(wl.tp)]
    ws = [synth.w_shard(wl, s) for s in range(wl.tp)]
    rng = np.random.default_rng([wl.seed, 77])
    res = synth.residual_chunk(wl) if chunked else synth.bf16_bits(
        rng.standard_normal((rows, wl.n), dtype=np.float32))
    gam = synth.gamma(wl)
    y, ro = rpl.rpl_matmul_reduce_rmsnorm([dev_bf16(x) for x in xs], [dev_bf16(w) for w in ws], dev_bf16(res),
                                          dev_bf16(gam), wl.eps)
    e1, e2 = _check_step(y, ro, _oracle_step(xs, ws, rows, res, gam, wl.eps), gam, wl.eps)
    say(f"  max abs err residual_out {e1:.3g} y {e2:.3g}")
