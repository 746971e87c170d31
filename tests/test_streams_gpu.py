"""The library's calls on caller streams other than the default one.

Every call enqueues its kernels on the stream the caller passes (the binding passes torch's
current stream) and keeps no state, so calls on different streams may run at the same time.
Checked here: (1) calls on two side streams running at once give the results of the same calls
made one after another on the default stream, bit for bit; (2) a call is ordered after the work
already queued on its stream: its input is written by copies queued just before it on the same
side stream, with nothing synchronised in between, so a kernel launched on any other stream would
read the stale input.  The expected values are the library's own default-stream results (the
kernels are deterministic); parity with the oracle is checked elsewhere."""
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import row_matmul_reduce_amd as rpl  # noqa: E402
from gpu_util import say  # noqa: E402


def _bf16(shape, gen, scale=1.0):
    return (torch.randn(shape, generator=gen, device="cuda") * scale).to(torch.bfloat16)


def _i8(shape, gen):
    return torch.randint(-127, 128, shape, generator=gen, device="cuda", dtype=torch.int8)


def _scales(n, gen, lo, hi):
    return torch.rand(n, generator=gen, device="cuda") * (hi - lo) + lo


def _same(a, b, what):
    assert a.shape == b.shape, what
    if a.dtype == torch.bfloat16:
        a, b = a.view(torch.int16), b.view(torch.int16)
    diff = int((a != b).sum())
    assert diff == 0, f"{what}: {diff} of {a.numel()} elements differ"


def test_two_side_streams_at_once_match_default_stream():
    say("[streams] bf16 partial + reduce on one side stream, w8a8 partial on another")
    gen = torch.Generator(device="cuda").manual_seed(11)
    m, k, n, tp = 1024, 2048, 1536, 2
    mc = m // tp
    x, w = _bf16((m, k), gen), _bf16((n, k), gen, 0.02)
    peer = _bf16((mc, n), gen)
    res, gam = _bf16((mc, n), gen), _bf16((n,), gen, 0.5) + 1.0
    xq, wq = _i8((512, 4096), gen), _i8((1024, 4096), gen)
    sx, sw = _scales(512, gen, 1e-3, 2e-2), _scales(1024, gen, 1e-3, 1e-2)
    torch.cuda.synchronize()

    p_ref = rpl.rpl_partial(x, w, tp)
    y_ref, ro_ref = rpl.rpl_reduce_chunk_rmsnorm([p_ref[:mc], peer], res, gam, 1e-6)
    q_ref = rpl.rpl_w8a8_partial(xq, sx, wq, sw, 1)
    torch.cuda.synchronize()

    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()  # default priority
    p = torch.empty_like(p_ref)
    y, ro = torch.empty_like(y_ref), torch.empty_like(ro_ref)
    q = torch.empty_like(q_ref)
    torch.cuda.synchronize()
    for rep in range(3):
        for t in (p, y, ro, q):
            t.zero_()
        torch.cuda.synchronize()
        with torch.cuda.stream(s1):
            rpl.rpl_partial(x, w, tp, out=p)
            rpl.rpl_reduce_chunk_rmsnorm([p[:mc], peer], res, gam, 1e-6, y=y, residual_out=ro)
        with torch.cuda.stream(s2):
            rpl.rpl_w8a8_partial(xq, sx, wq, sw, 1, out=q)
        s1.synchronize()
        s2.synchronize()
        _same(p, p_ref, f"bf16 partial, round {rep}")
        _same(y, y_ref, f"y, round {rep}")
        _same(ro, ro_ref, f"residual_out, round {rep}")
        _same(q, q_ref, f"w8a8 partial, round {rep}")


def test_call_is_ordered_after_work_queued_on_its_stream():
    say("[streams] inputs written by copies queued just before the calls on the same side stream")
    gen = torch.Generator(device="cuda").manual_seed(12)
    m, k, n = 256, 4096, 2048
    x_src, w = _bf16((m, k), gen), _bf16((n, k), gen, 0.02)
    res_src, gam = _bf16((m, n), gen), _bf16((n,), gen, 0.5) + 1.0
    big_src = torch.empty(64 << 20, dtype=torch.int32, device="cuda").fill_(7)  # 256 MiB
    big_dst = torch.empty_like(big_src)
    torch.cuda.synchronize()
    p_ref = rpl.rpl_partial(x_src, w, 1)
    y_ref, ro_ref = rpl.rpl_reduce_chunk_rmsnorm([p_ref], res_src, gam, 1e-6)
    torch.cuda.synchronize()

    s = torch.cuda.Stream()  # default priority
    x, res = torch.zeros_like(x_src), torch.zeros_like(res_src)
    p, y, ro = torch.empty_like(p_ref), torch.empty_like(y_ref), torch.empty_like(ro_ref)
    torch.cuda.synchronize()
    for rep in range(3):
        x.zero_()
        res.zero_()
        torch.cuda.synchronize()
        with torch.cuda.stream(s):
            big_dst.copy_(big_src)  # keeps the stream busy before the inputs are written
            x.copy_(x_src)
            res.copy_(res_src)
            rpl.rpl_partial(x, w, 1, out=p)
            rpl.rpl_reduce_chunk_rmsnorm([p], res, gam, 1e-6, y=y, residual_out=ro)
        s.synchronize()
        _same(p, p_ref, f"partial after the queued copy, round {rep}")
        _same(y, y_ref, f"y after the queued copy, round {rep}")
        _same(ro, ro_ref, f"residual_out after the queued copy, round {rep}")
