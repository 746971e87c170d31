"""Seeded random shapes through the C ABI against the CPU oracle: the bf16 partial (pad rows,
ragged tiles, K tails, 1-8 ranks), the w8a8 partial (accumulators bit-exact), the received-chunk
reduce + RMSNorm and the per-token quantiser.  The shapes are drawn once from a fixed seed, so a
failure names a reproducible case."""
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


def _shapes(seed, count, k_mult):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(count):
        m = int(rng.integers(1, 700))
        n = 8 * int(rng.integers(1, 140))
        k = k_mult * int(rng.integers(1, 1200 // k_mult))
        tp = int(rng.integers(1, 9))
        out.append((m, n, k, tp))
    return out


@pytest.mark.parametrize("m,n,k,tp", _shapes(2024, 10, 8))
def test_random_bf16_partial(m, n, k, tp):
    say(f"[random partial] m={m} n={n} k={k} tp={tp}")
    rng = np.random.default_rng([m, n, k, tp])
    x = synth.bf16_bits(rng.standard_normal((m, k), dtype=np.float32))
    w = synth.bf16_bits((rng.standard_normal((n, k), dtype=np.float32) * np.float32(0.05)))
    got = host_bf16(rpl.rpl_partial(dev_bf16(x), dev_bf16(w), tp))
    want = oracle.partial_rows(x, w, m, tp=tp)
    assert got.shape == want.shape
    assert_bf16_close(got, want, "partial")


@pytest.mark.parametrize("m,n,k,tp", _shapes(2025, 8, 16))
def test_random_w8a8_partial(m, n, k, tp):
    say(f"[random w8a8] m={m} n={n} k={k} tp={tp}")
    rng = np.random.default_rng([m, n, k, tp, 8])
    xq = rng.integers(-127, 128, (m, k), dtype=np.int8)
    wq = rng.integers(-127, 128, (n, k), dtype=np.int8)
    sx = rng.uniform(1e-3, 2e-2, m).astype(np.float32)
    sw = rng.uniform(1e-3, 1e-2, n).astype(np.float32)
    out, acc = rpl.rpl_w8a8_partial(dev(xq), dev(sx), dev(wq), dev(sw), tp, want_acc=True)
    wout, wacc = oracle.w8a8_rows(xq, sx, wq, sw, m, tp=tp)
    assert np.array_equal(acc.cpu().numpy(), wacc), "int32 accumulators must be bit-exact"
    assert np.array_equal(host_bf16(out), wout), "dequantised output (same fp32 operation order)"
    # without the accumulator store (the last tile then goes out through LDS) the bits are the same
    out2 = rpl.rpl_w8a8_partial(dev(xq), dev(sx), dev(wq), dev(sw), tp)
    assert np.array_equal(host_bf16(out2), wout), "dequantised output without the accumulator store"


@pytest.mark.parametrize("m,n,k,tp", _shapes(2026, 8, 8))
def test_random_reduce_and_quant(m, n, k, tp):
    say(f"[random reduce/quant] rows={m} n={n} k={k} tp={tp}")
    rng = np.random.default_rng([m, n, k, tp, 9])
    parts = [synth.bf16_bits(rng.standard_normal((m, n), dtype=np.float32)) for _ in range(tp)]
    res = synth.bf16_bits(rng.standard_normal((m, n), dtype=np.float32))
    gam = synth.bf16_bits(rng.uniform(0.5, 1.5, n).astype(np.float32))
    y, ro = rpl.rpl_reduce_chunk_rmsnorm([dev_bf16(p) for p in parts], dev_bf16(res), dev_bf16(gam), 1e-6)
    wy, wro = oracle.reduce_chunk_rmsnorm(parts, res, gam, 1e-6)
    assert_bf16_close(host_bf16(ro), wro, "residual_out")
    assert_bf16_close(host_bf16(y), wy, "y")
    x = synth.quant_test_rows(m, k, seed=m + k)
    xq, sx = rpl.rpl_quant_per_token(dev_bf16(x))
    oq, osx = oracle.quant_per_token(x)
    assert np.array_equal(xq.cpu().numpy(), oq) and np.array_equal(sx.cpu().numpy(), osx), "quantiser"
