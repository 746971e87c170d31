"""GPU parity of the other reduction forms, through the C ABI, against the CPU
oracle: the all-reduce sum of the shards' bf16 partials (rpl_sum_partials) and
the hidden-split epilogue of the 910C layout (rpl_reduce_slice_sumsq on each
rank's column slice, then rpl_rmsnorm_slice_apply after the cross-rank sum of
the per-row partial sums of squares).  bf16 outputs follow the rule
|gpu - oracle| <= 2e-2 + 1e-2 |oracle|; integer-valued partials are summed
exactly; fp32 sums of squares are within the fp32 accumulation bound.
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


def _partials(m, n, tp, seed, scale=1.0):
    rng = np.random.default_rng([seed, 11])
    return [synth.bf16_bits((rng.standard_normal((m, n), dtype=np.float32) * np.float32(scale)))
            for _ in range(tp)]


SUM_SHAPES = [(1, 8, 1), (5, 24, 2), (33, 520, 3), (300, 1032, 16), (4096, 3584, 2), (2048, 5120, 8)]


@pytest.mark.parametrize("m,n,tp", SUM_SHAPES)
def test_sum_partials(m, n, tp):
    say(f"[sum] m={m} n={n} tp={tp}")
    parts = _partials(m, n, tp, seed=m + n + tp)
    out = rpl.rpl_sum_partials([dev_bf16(p) for p in parts])
    rows = np.arange(m) if m <= 512 else np.unique(np.r_[0, 1, m // 2, m - 1, np.random.default_rng(2).integers(0, m, 12)])
    want = oracle.sum_partials([np.ascontiguousarray(p[rows]) for p in parts])
    e = assert_bf16_close(host_bf16(out)[rows], want, "all-reduce sum")
    say(f"  max abs err {e:.3g}")


def test_sum_partials_integers_exact_and_strided():
    import torch
    rng = np.random.default_rng(4)
    m, n, tp, ldp = 37, 264, 5, 280
    # |sum| <= 250: every partial sum is an integer that bf16 (8 significant bits) holds exactly
    parts = [synth.bf16_bits(rng.integers(-50, 51, (m, ldp)).astype(np.float32)) for _ in range(tp)]
    views = [dev_bf16(p)[:, :n] for p in parts]
    out = rpl.rpl_sum_partials(views)
    want = sum(synth.bf16_decode(p[:, :n]).astype(np.float64) for p in parts)
    assert np.array_equal(synth.bf16_decode(host_bf16(out)).astype(np.float64), want)
    empty = rpl.rpl_sum_partials([torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")] * 2)
    assert empty.shape == (0, 64)


# (m, n, tp, slice bounds): the decode o_proj share split over its 2 ranks, the 910C
# operator's case (40 rows, hidden 2048, TP=2), uneven slices, 8 slices of the long-prefill row,
# and slices wide enough for 2 to 6 chunks per lane
SPLIT_CASES = [(4, 3584, 2, [0, 1792, 3584]), (40, 2048, 2, [0, 1024, 2048]),
               (33, 520, 4, [0, 128, 264, 392, 520]), (2048, 5120, 8, list(range(0, 5121, 640))),
               (17, 16384, 2, [0, 4096, 16384]), (9, 6008, 3, [0, 2056, 4104, 6008])]


@pytest.mark.parametrize("m,n,tp,bounds", SPLIT_CASES, ids=lambda v: str(v) if not isinstance(v, list) else "slices")
def test_hidden_split_epilogue(m, n, tp, bounds):
    import torch
    say(f"[split] m={m} n={n} tp={tp} slices={len(bounds) - 1}")
    parts = _partials(m, n, tp, seed=m * 7 + n)
    rng = np.random.default_rng([m, n, 3])
    res = synth.bf16_bits(rng.standard_normal((m, n), dtype=np.float32))
    gam = synth.bf16_bits(rng.uniform(0.5, 1.5, n).astype(np.float32))
    eps = 1e-6
    dparts, dres, dgam = [dev_bf16(p) for p in parts], dev_bf16(res), dev_bf16(gam)
    ro = torch.empty_like(dres)
    y = torch.empty_like(dres)
    slices = list(zip(bounds[:-1], bounds[1:]))
    step1 = [rpl.rpl_reduce_slice_sumsq([p[:, a:b] for p in dparts], dres[:, a:b], ro[:, a:b]) for a, b in slices]
    ss_parts = [st[1] for st in step1]
    for (h, _), (a, b) in zip(step1, slices):
        rpl.rpl_rmsnorm_slice_apply(h, ss_parts, n, dgam[a:b], eps, y[:, a:b])
    rows = np.arange(m) if m <= 64 else np.unique(np.r_[0, 1, m - 1, np.random.default_rng(5).integers(0, m, 10)])
    sub = [np.ascontiguousarray(p[rows]) for p in parts]
    o1 = [oracle.reduce_slice_sumsq(sub, res[rows], a, b - a) for a, b in slices]
    for (h, ss), (oro, oh, oss), (a, b) in zip(step1, o1, slices):
        hg = h.cpu().numpy()[rows].astype(np.float64)
        # fp32 sum of tp partials and the residual: error <= (tp + 1) * 2^-24 * sum of |terms|
        mag = sum(np.abs(synth.bf16_decode(p[:, a:b]).astype(np.float64)) for p in sub) + \
            np.abs(synth.bf16_decode(res[rows][:, a:b]).astype(np.float64))
        assert np.all(np.abs(hg - oh) <= (tp + 1) * 2.0 ** -24 * mag), "fp32 h"
        # fp32 accumulation of n_slice squares: relative error below n_slice * 2^-23
        sg = ss.cpu().numpy()[rows].astype(np.float64)
        assert np.all(np.abs(sg - oss) <= (b - a) * 2.0 ** -23 * oss + 1e-30), "sum of squares"
        assert_bf16_close(host_bf16(ro)[rows][:, a:b], oro, f"residual_out slice {a}:{b}")
    oy = np.concatenate([oracle.rmsnorm_slice_apply(oh, [o[2] for o in o1], n, gam[a:b], eps)
                         for (oro, oh, oss), (a, b) in zip(o1, slices)], axis=1)
    e = assert_bf16_close(host_bf16(y)[rows], oy, "y")
    # the slices together are the token-chunk epilogue on whole rows
    y2, ro2 = rpl.rpl_reduce_chunk_rmsnorm(dparts, dres, dgam, eps)
    assert_bf16_close(host_bf16(y), host_bf16(y2), "split vs whole-row y")
    assert_bf16_close(host_bf16(ro), host_bf16(ro2), "split vs whole-row residual_out")
    say(f"  max abs err y {e:.3g}")
