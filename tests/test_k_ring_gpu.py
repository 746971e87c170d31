"""GPU: the tile engine's K-step rings across tile boundaries, against the oracle bit for bit.

The 256 x 224 engine keeps the activation's K steps in two LDS buffers and the weight's in three,
so the buffers a step uses follow its index modulo 2 and modulo 3, and the K loop is unrolled by
six.  Every shape here is 6144 x 2688 (288 tiles of 256 x 224 on 256 workgroups, so 32 of them run
a second tile whose rings start again at the first buffers), at every K-step count from 1 to 8, at
13, and with K tails (the engine's per-lane-cut form).  The operands are small integers, so every
partial sum is an integer below 2^24 and exact in fp32 in any order: the bf16 partial must equal the
oracle's exactly, and the w8a8 partial's int32 accumulators too.
"""
import numpy as np
import pytest

import oracle
import row_matmul_reduce_amd as rpl
from row_matmul_reduce_amd import synth
from gpu_util import assert_rel, dev, dev_bf16, host_bf16, say

pytestmark = pytest.mark.gpu

M, N = 6144, 2688  # 24 x 12 tiles of 256 x 224: two rounds over the 256 CUs (the 256-wide form would take two too)


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    rpl.lib()


def test_shape_runs_two_tiles_per_workgroup_on_the_224_wide_engine():
    tiles224 = -(-M // 256) * -(-N // 224)
    tiles256 = -(-M // 256) * -(-N // 256)
    assert 256 < tiles224 <= 512, "some workgroups run a second tile"
    assert -(-tiles224 // 256) * 224 < -(-tiles256 // 256) * 256, "the launcher picks the 256 x 224 tiles"


# K in bf16 elements: 64 per K step; the last two have a K tail (16 and 40 elements past whole steps)
@pytest.mark.parametrize("k", [64 * s for s in (1, 2, 3, 4, 5, 6, 7, 8, 13)] + [3 * 64 + 16, 7 * 64 + 40])
def test_bf16_rings_exact(k):
    say(f"[ring bf16] m={M} n={N} k={k} ({k / 64:.2f} K steps)")
    rng = np.random.default_rng(k)
    x = synth.bf16_bits(rng.integers(-2, 3, (M, k)).astype(np.float32))
    w = synth.bf16_bits(rng.integers(-2, 3, (N, k)).astype(np.float32))
    got = host_bf16(rpl.rpl_partial(dev_bf16(x), dev_bf16(w), 1))
    want = oracle.partial_rows(x, w, M)
    bad = np.argwhere(got != want)
    assert bad.size == 0, f"{len(bad)} outputs differ, first at {bad[:3].tolist()}"


# K in int8 elements: 128 per K step; the last one has a K tail
@pytest.mark.parametrize("k", [128 * s for s in (1, 2, 3, 5, 6, 7)] + [4 * 128 + 48])
def test_w8a8_rings_exact(k):
    say(f"[ring w8a8] m={M} n={N} k={k}")
    rng = np.random.default_rng(1000 + k)
    xq = rng.integers(-127, 128, (M, k), dtype=np.int8)
    wq = rng.integers(-127, 128, (N, k), dtype=np.int8)
    sx = rng.uniform(1e-3, 2e-2, M).astype(np.float32)
    sw = rng.uniform(1e-3, 1e-2, N).astype(np.float32)
    out, acc = rpl.rpl_w8a8_partial(dev(xq), dev(sx), dev(wq), dev(sw), 1, want_acc=True)
    wout, wacc = oracle.w8a8_rows(xq, sx, wq, sw, M)
    assert np.array_equal(acc.cpu().numpy(), wacc), "int32 accumulators must be bit-exact"
    assert_rel(host_bf16(out), wout, "dequantised output")
    # without the accumulators the last tile is stored through LDS: the same bits
    out2 = rpl.rpl_w8a8_partial(dev(xq), dev(sx), dev(wq), dev(sw), 1)
    assert np.array_equal(host_bf16(out2), host_bf16(out))
