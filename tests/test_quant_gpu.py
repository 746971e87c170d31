"""GPU parity of the per-token dynamic int8 quantiser and of the w8a8_dynamic
step it feeds (bf16 activation -> int8 codes + scale -> int8 partial -> chunk
reduce + RMSNorm), through the C ABI, against the CPU oracle.

Codes and scales are integers / fp32 values decided by correctly rounded fp32
divisions, so they must be bit-exact.  The int8 partial is then bit-exact too
(same codes, same fixed dequantisation order); the reduce + RMSNorm outputs
follow the bf16 rule |gpu - oracle| <= 2e-2 + 1e-2 |oracle|.
"""
import numpy as np
import pytest

import oracle
import row_matmul_reduce_amd as rpl
from row_matmul_reduce_amd import synth
from gpu_util import assert_bf16_close, dev, dev_bf16, host_bf16, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    rpl.lib()


def _compare(xq_gpu, sx_gpu, xq_want, sx_want, what):
    q = xq_gpu.cpu().numpy()
    s = sx_gpu.cpu().numpy()
    bad_s = np.flatnonzero(s.view(np.uint32) != sx_want.view(np.uint32))
    assert bad_s.size == 0, f"{what}: scale differs in rows {bad_s[:5].tolist()}: {s[bad_s[:5]]} vs {sx_want[bad_s[:5]]}"
    bad = np.argwhere(q != xq_want)
    assert bad.size == 0, (f"{what}: {len(bad)} codes differ, first {[tuple(b) for b in bad[:5]]}: "
                           f"{[int(q[tuple(b)]) for b in bad[:5]]} vs {[int(xq_want[tuple(b)]) for b in bad[:5]]}")


# (m, k): every kernel shape -- under 512 rows four waves per row with 1..8 chunks per
# lane; from 512 rows 1..4 chunks per lane with one wave per row, two and four waves per
# row, up to 8 chunks per lane; the two-pass kernel for rows longer than 16384 -- with
# ragged row counts and chunk tails.
QUANT_SHAPES = [(1, 8), (5, 24), (7, 1000), (64, 256), (33, 2048), (9, 2056), (17, 4096), (4, 4104),
                (12, 16384), (3, 16392), (2, 40000), (4099, 136), (18, 9472),
                (512, 8), (600, 1000), (520, 2056), (513, 4104), (530, 9472), (512, 16384)]


@pytest.mark.parametrize("m,k", QUANT_SHAPES)
def test_quant_shapes(m, k):
    say(f"[quant] m={m} k={k}")
    x = synth.quant_test_rows(m, k, seed=m * 131 + k)
    xq, sx = rpl.rpl_quant_per_token(dev_bf16(x))
    wq, ws = oracle.quant_per_token(x)
    _compare(xq, sx, wq, ws, f"m={m} k={k}")


def test_quant_strided_rows_and_padding_untouched():
    import torch
    m, k, ldx, ldq = 37, 520, 528, 544
    x = synth.quant_test_rows(m, ldx, seed=5)
    xd = dev_bf16(x)[:, :k]
    qbuf = torch.full((m, ldq), 99, dtype=torch.int8, device="cuda")
    sbuf = torch.full((m + 3,), 7.0, dtype=torch.float32, device="cuda")
    rpl.rpl_quant_per_token(xd, xq=qbuf[:, :k], x_scale=sbuf[:m])
    wq, ws = oracle.quant_per_token(np.ascontiguousarray(x[:, :k]))
    _compare(qbuf[:, :k], sbuf[:m], wq, ws, "strided")
    assert bool((qbuf[:, k:] == 99).all()), "columns past k were written"
    assert bool((sbuf[m:] == 7.0).all()), "scales past m were written"


def test_quant_empty_and_deterministic():
    import torch
    xq, sx = rpl.rpl_quant_per_token(torch.empty((0, 64), dtype=torch.bfloat16, device="cuda"))
    assert xq.shape == (0, 64) and sx.shape == (0,)
    x = dev_bf16(synth.quant_test_rows(256, 1792, seed=3))
    a, sa = rpl.rpl_quant_per_token(x)
    b, sb = rpl.rpl_quant_per_token(x)
    assert torch.equal(a, b) and torch.equal(sa, sb)


@pytest.mark.parametrize("wid", [2, 5])
def test_quant_workload_activation(wid):
    """The activations of the decode o_proj share and of the w8a8 prefill share, all rows."""
    wl = synth.WORKLOADS[wid]
    say(f"[quant full] {wl.name}")
    x = synth.x_shard(wl, 0)
    xq, sx = rpl.rpl_quant_per_token(dev_bf16(x))
    wq, ws = oracle.quant_per_token(x)
    _compare(xq, sx, wq, ws, wl.name)


def _dynamic_step(wl, rows_for_oracle, full_own=False):
    """bf16 X shards -> quantiser -> int8 partials -> reduce + RMSNorm on chunk 0."""
    mc = wl.m_chunk
    xs = [synth.x_shard(wl, 0)] + [synth.x_shard(wl, s, rows=mc) for s in range(1, wl.tp)]
    wts = [synth.w8a8_weight(wl, s) for s in range(wl.tp)]
    res, gam = synth.residual_chunk(wl), synth.gamma(wl)
    parts = []
    for s in range(wl.tp):
        q, sc = rpl.rpl_quant_per_token(dev_bf16(xs[s]))
        p = rpl.rpl_w8a8_partial(q, sc, dev(wts[s][0]), dev(wts[s][1]), wl.tp if s == 0 else 1)
        parts.append(p)
    own = parts[0]
    y, ro = rpl.rpl_reduce_chunk_rmsnorm([own[:mc]] + parts[1:], dev_bf16(res), dev_bf16(gam), wl.eps)
    rows = rows_for_oracle
    o_parts = []
    for s in range(wl.tp):
        if s == 0 and full_own:  # all the rank's rows, chunk 0 among them
            oq, osc = oracle.quant_per_token(xs[0])
            o_all, _ = oracle.w8a8_rows(oq, osc, wts[0][0], wts[0][1], wl.m, tp=wl.tp)
            assert np.array_equal(host_bf16(own), o_all), "own int8 partial differs"
            o_parts.append(np.ascontiguousarray(o_all[rows]))
            continue
        oq, osc = oracle.quant_per_token(xs[s], rows=int(rows.max()) + 1 if rows.size else 0)
        o_out, _ = oracle.w8a8_rows(oq, osc, wts[s][0], wts[s][1], wl.m if s == 0 else mc, rows=rows,
                                    tp=wl.tp if s == 0 else 1)
        o_parts.append(o_out)
    # the int8 partials see identical codes, so they match bit for bit
    assert np.array_equal(host_bf16(own)[rows], o_parts[0]), "own int8 partial differs"
    for s in range(1, wl.tp):
        assert np.array_equal(host_bf16(parts[s])[rows], o_parts[s]), f"peer {s} partial differs"
    wy, wro = oracle.reduce_chunk_rmsnorm(o_parts, res[rows], gam, wl.eps)
    e1 = assert_bf16_close(host_bf16(ro)[rows], wro, f"{wl.name} residual_out")
    e2 = assert_bf16_close(host_bf16(y)[rows], wy, f"{wl.name} y")
    say(f"  max abs err residual_out {e1:.3g} y {e2:.3g} over {rows.size} rows")


def test_w8a8_dynamic_small_end_to_end():
    wl = synth.custom(m=37, n=264, k_full=2 * 528, tp=2, kind="w8a8", x_dist="normal", seed=4)
    say(f"[w8a8 dynamic] {wl.name}")
    _dynamic_step(wl, np.arange(wl.m_chunk, dtype=np.int64))


def test_w8a8_dynamic_full_size():
    """The w8a8_dynamic step at full size: every code, every int8 partial output of the rank
    (all 4096 rows) and of the peer's chunk, and every element of the received chunk."""
    wl = synth.WORKLOADS[5]
    say(f"[w8a8 dynamic full] {wl.name}")
    _dynamic_step(wl, np.arange(wl.m_chunk, dtype=np.int64), full_own=True)
