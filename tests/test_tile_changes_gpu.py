"""GPU: multi-tile shares on the 256 x 256 engine, bit for bit against the oracle.

Every shape here takes the 256-wide tiles and runs two to four of them per workgroup, so most
workgroups change tiles: the finished tile is copied through the LDS operand buffers and stored
before the next tile's first DMAs into them.  One shape is ragged in M, so the tiles of its last
row band store only their valid rows.  The operands are small integers, so every partial sum is an
integer below 2^24 and exact in fp32 in any order: the partial must equal the oracle's exactly.
"""
import numpy as np
import pytest

import oracle
import row_matmul_reduce_amd as rpl
from row_matmul_reduce_amd import synth
from gpu_util import dev_bf16, host_bf16, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    rpl.lib()


def tiles_per_workgroup(m, n):
    """The launcher's choice for a K without tail: (tile width, tiles per workgroup)."""
    tm = -(-m // 256)
    nt224, nt256 = tm * -(-n // 224), tm * -(-n // 256)
    wide256 = -(-nt256 // 256) * 256 < -(-nt224 // 256) * 224
    return (256, -(-nt256 // 256)) if wide256 else (224, -(-nt224 // 256))


SHAPES = [(16384, 2048, 64), (16384, 4096, 192), (16384 - 77, 4096, 128), (16384, 4096, 7 * 64)]


def test_shapes_take_the_256_wide_tiles_several_per_workgroup():
    for m, n, k in SHAPES:
        bn, per = tiles_per_workgroup(m, n)
        assert bn == 256 and per >= 2, (m, n, bn, per)


@pytest.mark.parametrize("m, n, k", SHAPES)
def test_tile_changes_exact(m, n, k):
    say(f"[tile changes] m={m} n={n} k={k} tiles per workgroup {tiles_per_workgroup(m, n)[1]}")
    rng = np.random.default_rng(m + n + k)
    x = synth.bf16_bits(rng.integers(-2, 3, (m, k)).astype(np.float32))
    w = synth.bf16_bits(rng.integers(-2, 3, (n, k)).astype(np.float32))
    got = host_bf16(rpl.rpl_partial(dev_bf16(x), dev_bf16(w), 1))
    want = oracle.partial_rows(x, w, m)
    bad = np.argwhere(got != want)
    assert bad.size == 0, f"{len(bad)} outputs differ, first at {bad[:3].tolist()}"
