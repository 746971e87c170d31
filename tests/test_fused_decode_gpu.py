"""GPU parity of the single-launch decode path (rpl_matmul_reduce_rmsnorm)
through the C ABI, against the CPU oracle's unfused composition: a bf16
partial per shard (oracle.partial_rows), then the sum of the partials,
residual add and RMSNorm (oracle.reduce_chunk_rmsnorm).  Outputs follow the
bf16 rule |gpu - oracle| <= 2e-2 + 1e-2 |oracle|; repeated calls on one
workspace must give identical bits and leave its counter at zero.
"""
import numpy as np
import pytest

import oracle
import row_matmul_reduce_amd as rpl
from row_matmul_reduce_amd import synth
from gpu_util import assert_bf16_close, dev_bf16, host_bf16, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    rpl.lib()


def _oracle_step(xs, ws, m, residual, gamma, eps):
    """Unfused composition on the CPU: per-shard bf16 partials of the m rows (rows past the
    given activation rows are padding), then sum + residual + RMSNorm."""
    parts = []
    for x, w in zip(xs, ws):
        xpad = np.zeros((m, w.shape[1]), dtype=np.uint16)
        xpad[: x.shape[0]] = x
        parts.append(oracle.partial_rows(xpad, w, m))
    return oracle.reduce_chunk_rmsnorm(parts, residual, gamma, eps)


def _inputs(m, m_valid, n, k, tp, seed):
    wl = synth.custom(m=max(m_valid, 1), n=n, k_full=k * tp, tp=tp, seed=seed)
    xs = [synth.x_shard(wl, s)[:m_valid] for s in range(tp)]
    ws = [synth.w_shard(wl, s) for s in range(tp)]
    rng = np.random.default_rng([seed, 5])
    res = synth.bf16_bits(rng.standard_normal((m, n), dtype=np.float32))
    gam = synth.bf16_bits(rng.uniform(0.5, 1.5, n).astype(np.float32))
    return xs, ws, res, gam


# (m, m_valid, n, k, tp): one to four 16-row blocks, padding rows, ragged K steps,
# one to eight shards, the 910C operator's case (40 rows, hidden 2048, TP=2)
FUSED_SHAPES = [(1, 1, 8, 8, 1), (4, 4, 264, 1000, 2), (5, 3, 520, 328, 3), (16, 16, 512, 512, 2),
                (17, 17, 1024, 256, 4), (40, 40, 2048, 1024, 2), (64, 60, 136, 72, 8), (33, 0, 64, 64, 2)]


@pytest.mark.parametrize("m,m_valid,n,k,tp", FUSED_SHAPES)
def test_fused_shapes(m, m_valid, n, k, tp):
    say(f"[fused] m={m} m_valid={m_valid} n={n} k={k} tp={tp}")
    xs, ws, res, gam = _inputs(m, m_valid, n, k, tp, seed=m + n + k + tp)
    eps = 1e-6
    y, ro = rpl.rpl_matmul_reduce_rmsnorm([dev_bf16(x) for x in xs], [dev_bf16(w) for w in ws], dev_bf16(res),
                                          dev_bf16(gam), eps)
    wy, wro = _oracle_step(xs, ws, m, res, gam, eps)
    e1 = assert_bf16_close(host_bf16(ro), wro, "residual_out")
    e2 = assert_bf16_close(host_bf16(y), wy, "y")
    say(f"  max abs err residual_out {e1:.3g} y {e2:.3g}")


def test_fused_workspace_reuse_and_in_place():
    import torch
    m, n, k, tp = 8, 512, 256, 2
    xs, ws, res, gam = _inputs(m, m, n, k, tp, seed=3)
    dx, dw, dg = [dev_bf16(x) for x in xs], [dev_bf16(w) for w in ws], dev_bf16(gam)
    work = rpl.rpl_matmul_reduce_rmsnorm_workspace(m, n)
    outs = []
    for _ in range(3):
        y, ro = rpl.rpl_matmul_reduce_rmsnorm(dx, dw, dev_bf16(res), dg, 1e-6, workspace=work)
        torch.cuda.synchronize()
        assert int(work[:4].view(torch.int32).item()) == 0, "completion counter not reset"
        outs.append((host_bf16(y), host_bf16(ro)))
    for y, ro in outs[1:]:
        assert np.array_equal(y, outs[0][0]) and np.array_equal(ro, outs[0][1])
    # residual_out may be the residual buffer itself
    r_in = dev_bf16(res)
    y2, ro2 = rpl.rpl_matmul_reduce_rmsnorm(dx, dw, r_in, dg, 1e-6, workspace=work, residual_out=r_in)
    assert ro2.data_ptr() == r_in.data_ptr()
    assert np.array_equal(host_bf16(r_in), outs[0][1]) and np.array_equal(host_bf16(y2), outs[0][0])


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
    wy, wro = _oracle_step(xs, ws, rows, res, gam, wl.eps)
    e1 = assert_bf16_close(host_bf16(ro), wro, "residual_out")
    e2 = assert_bf16_close(host_bf16(y), wy, "y")
    say(f"  max abs err residual_out {e1:.3g} y {e2:.3g}")
