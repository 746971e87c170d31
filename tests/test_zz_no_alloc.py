"""GPU check of rpl_matmul_reduce_rmsnorm_noalloc, the single-launch decode path for callers
that cannot allocate (its hand-offs use a device array inside the library instead of a
workspace).  Called through the C ABI with outputs the test allocated beforehand, its results
must equal, bit for bit, those of rpl_matmul_reduce_rmsnorm with a workspace on the same inputs
(the same kernel and summation order), and both must satisfy the bf16 rule against the oracle's
unfused composition.  Two calls in a row, the second with a smaller input, then a shape whose
hand-off memory exceeds the array is refused with its outputs untouched."""
import ctypes

import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import oracle  # noqa: E402
import row_matmul_reduce_amd as rpl  # noqa: E402
from row_matmul_reduce_amd import synth  # noqa: E402
from gpu_util import assert_bf16_close, dev_bf16, host_bf16, say  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    rpl.lib()


def _noalloc(xs, ws, res, gam, eps, y, ro):
    """The raw C-ABI call (no binding logic, nothing allocated)."""
    tp = len(ws)
    xa = (ctypes.c_void_p * tp)(*[t.data_ptr() for t in xs])
    wa = (ctypes.c_void_p * tp)(*[t.data_ptr() for t in ws])
    m, n = res.shape
    return rpl.lib().rpl_matmul_reduce_rmsnorm_noalloc(
        ctypes.cast(xa, ctypes.c_void_p), xs[0].stride(0) if xs[0].shape[0] > 1 else xs[0].shape[1],
        ctypes.cast(wa, ctypes.c_void_p), ws[0].stride(0), tp, m, xs[0].shape[0], n, ws[0].shape[1],
        res.data_ptr(), gam.data_ptr(), float(eps), y.data_ptr(), ro.data_ptr(),
        torch.cuda.current_stream().cuda_stream)


def _inputs(m, n, k, tp, seed):
    wl = synth.custom(m=m, n=n, k_full=k * tp, tp=tp, seed=seed)
    xs = [synth.x_shard(wl, s) for s in range(tp)]
    ws = [synth.w_shard(wl, s) for s in range(tp)]
    rng = np.random.default_rng([seed, 9])
    res = synth.bf16_bits(rng.standard_normal((m, n), dtype=np.float32))
    gam = synth.bf16_bits(rng.uniform(0.5, 1.5, n).astype(np.float32))
    return xs, ws, res, gam


def test_noalloc_equals_the_workspace_entry_point():
    eps = 1e-6
    # the decode o_proj share's all-rows step, then a smaller one (fewer rows, narrower, shorter K)
    for i, (m, n, k, tp) in enumerate([(8, 3584, 1792, 2), (3, 1040, 520, 2)]):
        say(f"[noalloc] call {i}: m={m} n={n} k={k} tp={tp}")
        xs, ws, res, gam = _inputs(m, n, k, tp, seed=70 + i)
        dx, dw, dr, dg = [dev_bf16(x) for x in xs], [dev_bf16(w) for w in ws], dev_bf16(res), dev_bf16(gam)
        y_ref, ro_ref = rpl.rpl_matmul_reduce_rmsnorm(dx, dw, dr, dg, eps)
        y = torch.full_like(dr, float("nan"))
        ro = torch.full_like(dr, float("nan"))
        torch.cuda.synchronize()
        before = torch.cuda.memory_allocated()
        st = _noalloc(dx, dw, dr, dg, eps, y, ro)
        assert st == rpl.RPL_OK, rpl.rpl_status_string(st)
        torch.cuda.synchronize()
        assert torch.cuda.memory_allocated() == before
        assert np.array_equal(host_bf16(y), host_bf16(y_ref)), "y differs from the workspace entry point"
        assert np.array_equal(host_bf16(ro), host_bf16(ro_ref)), "residual_out differs from the workspace entry point"
        wy, wro = oracle.reduce_chunk_rmsnorm([oracle.partial_rows(x, w, m) for x, w in zip(xs, ws)], res, gam, eps)
        assert_bf16_close(host_bf16(ro), wro, f"call {i} residual_out")
        assert_bf16_close(host_bf16(y), wy, f"call {i} y")


def test_noalloc_refuses_a_shape_beyond_its_array():
    m, n, k, tp = 64, 8192, 64, 2  # needs 4 MiB + header of hand-off memory
    assert rpl.lib().rpl_matmul_reduce_rmsnorm_workspace_size(m, n, tp) > 4 << 20
    xs, ws, res, gam = _inputs(m, n, k, tp, seed=5)
    dx, dw, dr, dg = [dev_bf16(x) for x in xs], [dev_bf16(w) for w in ws], dev_bf16(res), dev_bf16(gam)
    y = torch.full_like(dr, 3.0)
    ro = torch.full_like(dr, 5.0)
    assert _noalloc(dx, dw, dr, dg, 1e-6, y, ro) == rpl.RPL_ERR_UNSUPPORTED
    torch.cuda.synchronize()
    assert bool((y == 3.0).all()) and bool((ro == 5.0).all()), "outputs of a refused call must be untouched"
