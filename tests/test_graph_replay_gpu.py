"""HIP graph capture and replay of the library's calls.

The decode-sized paths are timed by replaying HIP graphs, and a caller may capture any call.
Each case captures a sequence of calls once, then several times changes the inputs in place,
runs the same calls eagerly, and replays the graph with eager work and synchronisation in
between: every replay must reproduce the eager outputs bit for bit (the same kernels on the
same bytes).  The single-launch decode path hands values between its workgroups through tagged
slots in its workspace, the tag coming from a ticket every launch advances; repeated replays
rely on that, and the workspace's status word must stay zero.  The expected values here are the
library's own eager results: this checks capture and replay, parity with the oracle is checked
elsewhere."""
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import row_matmul_reduce_amd as rpl  # noqa: E402
from gpu_util import say  # noqa: E402

REPLAYS = 4


def _fill_bf16(t, gen, scale=1.0):
    t.copy_((torch.randn(t.shape, generator=gen, device="cuda") * scale).to(torch.bfloat16))


def _check_replays(name, run, outputs, refill):
    say(f"[graph] {name}")
    run()  # library loaded, kernels resident
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    torch.cuda.synchronize()
    for rep in range(REPLAYS):
        refill(rep)
        run()
        torch.cuda.synchronize()
        want = [o.clone() for o in outputs]
        for o in outputs:
            o.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (o, w) in enumerate(zip(outputs, want)):
            same = torch.equal(o.contiguous().view(torch.uint8), w.contiguous().view(torch.uint8))
            assert same, f"{name}: replay {rep}, output {i}"
    say(f"  {REPLAYS} replays identical to the eager calls")


def test_graph_decode_step():
    """Decode o_proj share: the rank partial (8 tokens, two shards) + the chunk reduce/RMSNorm."""
    gen = torch.Generator(device="cuda").manual_seed(11)
    m, k, n, tp, mc = 8, 1792, 3584, 2, 4
    x = torch.empty((m, k), dtype=torch.bfloat16, device="cuda")
    w = torch.empty((n, k), dtype=torch.bfloat16, device="cuda")
    peer = torch.empty((mc, n), dtype=torch.bfloat16, device="cuda")
    res = torch.empty((mc, n), dtype=torch.bfloat16, device="cuda")
    gam = torch.empty((n,), dtype=torch.bfloat16, device="cuda")
    p = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
    y = torch.empty((mc, n), dtype=torch.bfloat16, device="cuda")
    ro = torch.empty((mc, n), dtype=torch.bfloat16, device="cuda")

    def refill(rep):
        _fill_bf16(x, gen)
        _fill_bf16(w, gen, 0.02)
        _fill_bf16(peer, gen)
        _fill_bf16(res, gen)
        gam.copy_((torch.rand(n, generator=gen, device="cuda") + 0.5).to(torch.bfloat16))

    def run():
        rpl.rpl_partial(x, w, tp, out=p)
        rpl.rpl_reduce_chunk_rmsnorm([p[:mc], peer], res, gam, 1e-6, y=y, residual_out=ro)

    refill(-1)
    _check_replays("decode partial + chunk reduce", run, [p, y, ro], refill)


@pytest.mark.parametrize("rows", [4, 8])
def test_graph_single_launch_decode(rows):
    """The single-launch decode path for a token chunk (4 rows) and for all rows (8)."""
    gen = torch.Generator(device="cuda").manual_seed(12 + rows)
    k, n, tp = 1792, 3584, 2
    xs = [torch.empty((rows, k), dtype=torch.bfloat16, device="cuda") for _ in range(tp)]
    ws = [torch.empty((n, k), dtype=torch.bfloat16, device="cuda") for _ in range(tp)]
    res = torch.empty((rows, n), dtype=torch.bfloat16, device="cuda")
    gam = torch.empty((n,), dtype=torch.bfloat16, device="cuda")
    y = torch.empty((rows, n), dtype=torch.bfloat16, device="cuda")
    ro = torch.empty((rows, n), dtype=torch.bfloat16, device="cuda")
    work = rpl.rpl_matmul_reduce_rmsnorm_workspace(rows, n, tp)

    def refill(rep):
        for t in xs:
            _fill_bf16(t, gen)
        for t in ws:
            _fill_bf16(t, gen, 0.02)
        _fill_bf16(res, gen)
        gam.copy_((torch.rand(n, generator=gen, device="cuda") + 0.5).to(torch.bfloat16))

    def run():
        rpl.rpl_matmul_reduce_rmsnorm(xs, ws, res, gam, 1e-6, workspace=work, y=y, residual_out=ro)

    refill(-1)
    _check_replays(f"single-launch decode, {rows} rows", run, [y, ro], refill)
    assert rpl.rpl_matmul_reduce_rmsnorm_status(work) == 0, "no wait may have given up"


def test_graph_w8a8_dynamic_and_prefill_tiles():
    """Quantiser + int8 partial, and a bf16 partial over several tiles with a ragged tail."""
    gen = torch.Generator(device="cuda").manual_seed(13)
    m, k, n, tp = 300, 512, 640, 2
    x = torch.empty((m, k), dtype=torch.bfloat16, device="cuda")
    w = torch.empty((n, k), dtype=torch.bfloat16, device="cuda")
    wq = torch.empty((n, k), dtype=torch.int8, device="cuda")
    sw = torch.empty((n,), dtype=torch.float32, device="cuda")
    xq = torch.empty((m, k), dtype=torch.int8, device="cuda")
    sx = torch.empty((m,), dtype=torch.float32, device="cuda")
    p = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
    p8 = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
    acc = torch.empty((m, n), dtype=torch.int32, device="cuda")

    def refill(rep):
        _fill_bf16(x, gen)
        _fill_bf16(w, gen, 0.02)
        wq.copy_(torch.randint(-127, 128, (n, k), generator=gen, device="cuda", dtype=torch.int32).to(torch.int8))
        sw.copy_(torch.rand(n, generator=gen, device="cuda") * 9e-3 + 1e-3)

    def run():
        rpl.rpl_partial(x, w, tp, out=p)
        rpl.rpl_quant_per_token(x, xq=xq, x_scale=sx)
        rpl.rpl_w8a8_partial(xq, sx, wq, sw, tp, out=p8, acc=acc)

    refill(-1)
    _check_replays("bf16 partial, quantiser, w8a8 partial", run, [p, xq, sx, p8, acc], refill)


def test_graph_reduce_variants_and_token_rows():
    """All-reduce sum, hidden-split steps and the token-row shard / gather."""
    gen = torch.Generator(device="cuda").manual_seed(14)
    tp, m, n, ns = 3, 70, 384, 128
    parts = [torch.empty((m, n), dtype=torch.bfloat16, device="cuda") for _ in range(tp)]
    res = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
    gam = torch.empty((ns,), dtype=torch.bfloat16, device="cuda")
    total = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
    ro = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
    h = torch.empty((m, ns), dtype=torch.float32, device="cuda")
    ss = torch.empty((m,), dtype=torch.float32, device="cuda")
    y = torch.empty((m, ns), dtype=torch.bfloat16, device="cuda")
    mc = -(-m // tp)
    blocks = [torch.empty((mc, n), dtype=torch.bfloat16, device="cuda") for _ in range(tp)]
    back = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")

    def refill(rep):
        for t in parts:
            _fill_bf16(t, gen)
        _fill_bf16(res, gen)
        gam.copy_((torch.rand(ns, generator=gen, device="cuda") + 0.5).to(torch.bfloat16))

    def run():
        rpl.rpl_sum_partials(parts, out=total)
        rpl.rpl_reduce_slice_sumsq([t[:, :ns] for t in parts], res[:, :ns], ro[:, :ns], h=h, sumsq=ss)
        rpl.rpl_rmsnorm_slice_apply(h, [ss], ns, gam, 1e-6, y)
        for r in range(tp):
            rpl.rpl_shard_rows(total, tp, r, out=blocks[r])
        rpl.rpl_gather_rows(blocks, m, out=back)

    refill(-1)
    _check_replays("sum, hidden split, shard and gather", run, [total, ro[:, :ns], h, ss, y, back] + blocks,
                   refill)
