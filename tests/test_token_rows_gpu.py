"""GPU parity of the FlashComm1 token-row movement through the C ABI against the
CPU oracle: a rank's block of the zero-padded rows (rpl_shard_rows) and the
gather of all ranks' blocks cut back to the real rows (rpl_gather_rows).  Both
only move bf16 bit patterns, so every comparison is bit-exact.
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


def _rows(m, n, seed):
    rng = np.random.default_rng([seed, 17])
    return synth.bf16_bits(rng.standard_normal((m, n), dtype=np.float32))


# (m, n, tp): one rank; a pad row; tp not dividing m; ranks past the last real row;
# ragged n; the prefill residual (TP=2) and the long-prefill rows (TP=8)
SHAPES = [(1, 8, 1), (5, 64, 2), (7, 24, 4), (2, 8, 4), (1001, 520, 3), (4096, 3584, 2), (16384, 5120, 8)]


@pytest.mark.parametrize("m,n,tp", SHAPES)
def test_shard_then_gather(m, n, tp):
    say(f"[token rows] m={m} n={n} tp={tp}")
    x = _rows(m, n, m + n + tp)
    dx = dev_bf16(x)
    blocks = [rpl.rpl_shard_rows(dx, tp, r) for r in range(tp)]
    ranks = range(tp) if m * n <= 1 << 22 else [0, tp - 1]
    for r in ranks:
        assert np.array_equal(host_bf16(blocks[r]), oracle.shard_rows(x, tp, r)), f"rank {r} block"
    back = rpl.rpl_gather_rows(blocks, m)
    assert np.array_equal(host_bf16(back), x), "gathered blocks differ from the rows"


def test_gather_independent_blocks_and_strides():
    """Blocks that are not a shard of anything (nonzero in the dropped rows), given as strided
    column views of wider arrays; and a strided source for the shard."""
    import torch
    rng = np.random.default_rng(5)
    tp, mc, n, ld, m = 3, 11, 264, 280, 31
    wide = [synth.bf16_bits(rng.standard_normal((mc, ld), dtype=np.float32)) for _ in range(tp)]
    views = [dev_bf16(w)[:, :n] for w in wide]
    got = host_bf16(rpl.rpl_gather_rows(views, m))
    want = oracle.gather_rows([np.ascontiguousarray(w[:, :n]) for w in wide], m)
    assert np.array_equal(got, want)
    xs = synth.bf16_bits(rng.standard_normal((m, ld), dtype=np.float32))
    for r in range(tp):
        got = host_bf16(rpl.rpl_shard_rows(dev_bf16(xs)[:, :n], tp, r))
        assert np.array_equal(got, oracle.shard_rows(np.ascontiguousarray(xs[:, :n]), tp, r))
    # empty batch
    e = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    assert rpl.rpl_shard_rows(e, 2, 1).shape == (0, 64)
    assert rpl.rpl_gather_rows([e, e], 0).shape == (0, 64)


def test_shard_into_existing_buffer_leaves_nothing_stale():
    """A reused output buffer gets every element rewritten, pad rows included."""
    import torch
    m, n, tp = 9, 72, 4
    x = _rows(m, n, 3)
    out = torch.full((3, n), 7.0, dtype=torch.bfloat16, device="cuda")
    rpl.rpl_shard_rows(dev_bf16(x), tp, 3, out=out)
    assert np.array_equal(host_bf16(out), oracle.shard_rows(x, tp, 3))
