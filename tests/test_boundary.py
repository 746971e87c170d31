"""CPU-only tests of the C ABI boundary (librpl.so), no GPU needed.

The library must load without a GPU and export every function that
include/rpl.h declares.  Every argument check runs on the host before any HIP
call, so calls that fail validation are safe to make here; they must return
the documented status and leave the output buffers untouched.  Buffers here
are host memory standing in for device memory: a rejected call must not
touch them.  No call in this file reaches a kernel launch.
"""
import ctypes
import glob
import os
import re

import numpy as np
import pytest

import row_matmul_reduce_amd as rpl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "rpl.h")
HEADERS = sorted(glob.glob(os.path.join(ROOT, "include", "*.h")))

OK, NULL, INVALID, UNSUP = rpl.RPL_OK, rpl.RPL_ERR_NULL, rpl.RPL_ERR_INVALID, rpl.RPL_ERR_UNSUPPORTED


def declared_functions(headers=None):
    names = set()
    for h in headers or HEADERS:
        src = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"\b(rpl_[a-z0-9_]+)\s*\(", src))
    return sorted(names)


def test_header_declares_the_path_calls():
    names = declared_functions([HEADER])
    for f in ("rpl_partial", "rpl_reduce_chunk_rmsnorm", "rpl_w8a8_partial", "rpl_quant_per_token",
              "rpl_matmul_reduce_rmsnorm", "rpl_matmul_reduce_rmsnorm_workspace_size",
              "rpl_sum_partials", "rpl_reduce_slice_sumsq", "rpl_rmsnorm_slice_apply",
              "rpl_shard_rows", "rpl_gather_rows", "rpl_status_string", "rpl_version"):
        assert f in names


def test_library_exports_every_declared_symbol():
    L = rpl.lib()
    for name in declared_functions():
        assert hasattr(L, name), f"{name} declared in include/ but not exported"
    # and exports no other rpl_ function (nm on the built object)
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", rpl.LIB_PATH], capture_output=True, text=True).stdout
    exported = sorted({ln.split()[-1] for ln in out.splitlines() if re.search(r" T rpl_", ln)})
    assert exported == declared_functions()


def test_status_strings_and_version():
    assert [rpl.rpl_status_string(s) for s in range(5)] == [
        "RPL_OK", "RPL_ERR_NULL", "RPL_ERR_INVALID", "RPL_ERR_UNSUPPORTED", "RPL_ERR_LAUNCH"]
    assert rpl.rpl_status_string(99) == "unknown"
    assert rpl.rpl_version() == (2 << 16) | 2


class Buf:
    """16-byte aligned host buffer filled with a sentinel; reports whether it changed."""

    def __init__(self, nbytes, offset=0):
        # generous slack so that spans of strided test shapes stay inside the buffer
        self.raw = np.full(2 * nbytes + 4096, 0xA5, dtype=np.uint8)
        base = self.raw.ctypes.data
        self.start = (-base) % 16 + offset
        self.ptr = base + self.start

    def untouched(self):
        return bool(np.all(self.raw == 0xA5))


def partial(x, ldx, w, ldw, out, m, n, k, tp):
    return rpl.lib().rpl_partial(x, ldx, w, ldw, out, m, n, k, tp, None)


def test_partial_validation():
    m, n, k, tp = 6, 16, 32, 2
    X, W, O = Buf(m * k * 2), Buf(n * k * 2), Buf(m * n * 2)
    x, w, o = X.ptr, W.ptr, O.ptr
    cases = [
        ((x, k, None, k, o, m, n, k, tp), NULL),
        ((None, k, w, k, o, m, n, k, tp), NULL),
        ((x, k, w, k, None, m, n, k, tp), NULL),
        ((x, k, w, k, o, -1, n, k, tp), INVALID),
        ((x, k, w, k, o, m, 0, k, tp), INVALID),
        ((x, k, w, k, o, m, n, 0, tp), INVALID),
        ((x, k, w, k, o, m, n, k, 0), INVALID),
        ((x, k - 8, w, k, o, m, n, k, tp), INVALID),
        ((x, k, w, k - 8, o, m, n, k, tp), INVALID),
        ((x, k, w, k, x + 16, m, n, k, tp), INVALID),            # out overlaps x
        ((x, k, w, k, w, m, n, k, tp), INVALID),                 # out overlaps w
        ((x, k, w, k, o, m, n, k, 17), UNSUP),
        ((x, 40, w, 40, o, m, n, 36, tp), UNSUP),                 # k % 8
        ((x, k, w, k, o, m, 20, k, tp), UNSUP),                   # n % 8
        ((x, 36, w, k, o, m, n, k, tp), UNSUP),                   # ldx % 8
        ((x + 2, k, w, k, o, m, n, k, tp), UNSUP),                # misaligned x
        ((x, k, w + 8, k, o, m, n, k, tp), UNSUP),                # misaligned w
        ((x, k, w, k, o + 4, m, n, k, tp), UNSUP),                # misaligned out
        # row stride of 8 MiB or more (far-apart fake addresses: never dereferenced)
        ((1 << 44, 1 << 22, 1 << 45, k, 1 << 46, m, n, k, tp), UNSUP),
        # too many rows (far-apart fake addresses: never dereferenced, no overlap)
        ((1 << 44, k, 1 << 45, k, 1 << 46, 1 << 31, n, k, tp), UNSUP),
    ]
    for args, want in cases:
        assert partial(*args) == want, args
    assert X.untouched() and W.untouched() and O.untouched()
    # empty batch: OK without touching anything (x and out may be NULL)
    assert partial(None, k, w, k, None, 0, n, k, tp) == OK
    assert partial(x, k, w, k, o, 0, n, k, tp) == OK
    assert X.untouched() and W.untouched() and O.untouched()


def reduce_call(parts, tp, mc, n, res, gam, eps, y, ro):
    arr = None if parts is None else (ctypes.c_void_p * len(parts))(*parts)
    return rpl.lib().rpl_reduce_chunk_rmsnorm(None if arr is None else ctypes.cast(arr, ctypes.c_void_p), tp, mc,
                                              n, res, gam, eps, y, ro, None)


def test_reduce_validation():
    tp, mc, n = 2, 4, 64
    mat = mc * n * 2
    P0, P1, R, G, Y, RO = Buf(mat), Buf(mat), Buf(mat), Buf(n * 2), Buf(mat), Buf(mat)
    p = [P0.ptr, P1.ptr]
    r, g, y, ro = R.ptr, G.ptr, Y.ptr, RO.ptr
    cases = [
        ((None, tp, mc, n, r, g, 1e-6, y, ro), NULL),
        (([p[0], None], tp, mc, n, r, g, 1e-6, y, ro), NULL),
        ((p, tp, mc, n, None, g, 1e-6, y, ro), NULL),
        ((p, tp, mc, n, r, None, 1e-6, y, ro), NULL),
        ((p, tp, mc, n, r, g, 1e-6, None, ro), NULL),
        ((p, tp, mc, n, r, g, 1e-6, y, None), NULL),
        ((p, 0, mc, n, r, g, 1e-6, y, ro), INVALID),
        ((p, tp, -1, n, r, g, 1e-6, y, ro), INVALID),
        ((p, tp, mc, 0, r, g, 1e-6, y, ro), INVALID),
        ((p, tp, mc, n, r, g, -1e-6, y, ro), INVALID),
        ((p, tp, mc, n, r, g, float("nan"), y, ro), INVALID),
        ((p, tp, mc, n, r, g, float("inf"), y, ro), INVALID),
        ((p, tp, mc, n, r, g, 1e-6, r, ro), INVALID),             # y aliases residual
        ((p, tp, mc, n, r, g, 1e-6, p[1], ro), INVALID),          # y aliases a partial
        ((p, tp, mc, n, r, g, 1e-6, y, y), INVALID),              # y aliases residual_out
        ((p, tp, mc, n, r, g, 1e-6, g, ro), INVALID),             # y overlaps gamma
        ((p, tp, mc, n, r, g, 1e-6, y, r + 16), INVALID),         # residual_out partially overlaps residual
        ((p, tp, mc, n, r, g, 1e-6, y, p[0]), INVALID),           # residual_out aliases a partial
        ((p * 9, 18, mc, n, r, g, 1e-6, y, ro), UNSUP),           # tp > 16
        ((p, tp, mc, 60, r, g, 1e-6, y, ro), UNSUP),              # n % 8
        # n > 16384 (far-apart fake addresses: never dereferenced, no overlap)
        (([1 << 40, 1 << 41], tp, mc, 16392, 1 << 42, 1 << 43, 1e-6, 1 << 44, 1 << 45), UNSUP),
        (([p[0] + 8, p[1]], tp, mc, n, r, g, 1e-6, y, ro), UNSUP),
        ((p, tp, mc, n, r, g + 2, 1e-6, y, ro), UNSUP),
        ((p, tp, mc, n, r, g, 1e-6, y + 8, ro), UNSUP),
    ]
    for args, want in cases:
        assert reduce_call(*args) == want, args
    for b in (P0, P1, R, G, Y, RO):
        assert b.untouched()
    assert reduce_call([None, None], tp, 0, n, None, g, 1e-6, None, None) == OK
    for b in (P0, P1, R, G, Y, RO):
        assert b.untouched()


def w8a8_call(xq, ldx, sx, wq, ldw, sw, out, acc, m, n, k, tp):
    return rpl.lib().rpl_w8a8_partial(xq, ldx, sx, wq, ldw, sw, out, acc, m, n, k, tp, None)


def test_w8a8_validation():
    m, n, k, tp = 6, 16, 64, 2
    XQ, SX, WQ, SW, O, A = Buf(m * k), Buf(m * 4), Buf(n * k), Buf(n * 4), Buf(m * n * 2), Buf(m * n * 4)
    xq, sx, wq, sw, o, a = XQ.ptr, SX.ptr, WQ.ptr, SW.ptr, O.ptr, A.ptr
    cases = [
        ((None, k, sx, wq, k, sw, o, a, m, n, k, tp), NULL),
        ((xq, k, None, wq, k, sw, o, a, m, n, k, tp), NULL),
        ((xq, k, sx, None, k, sw, o, a, m, n, k, tp), NULL),
        ((xq, k, sx, wq, k, None, o, a, m, n, k, tp), NULL),       # weight_scale is required
        ((xq, k, sx, wq, k, sw, None, a, m, n, k, tp), NULL),
        ((xq, k, sx, wq, k, sw, o, a, -2, n, k, tp), INVALID),
        ((xq, k, sx, wq, k, sw, o, a, m, n, k, 0), INVALID),
        ((xq, 48, sx, wq, k, sw, o, a, m, n, k, tp), INVALID),
        ((xq, k, sx, wq, k, sw, o, o, m, n, k, tp), INVALID),      # acc aliases out
        ((xq, k, sx, wq, k, sw, xq, a, m, n, k, tp), INVALID),     # out aliases xq
        ((xq, k, sx, wq, k, sw, o, sw, m, n, k, tp), INVALID),     # acc overlaps w_scale
        ((xq, 80, sx, wq, 80, sw, o, a, m, n, 72, tp), UNSUP),     # k % 16
        ((xq, 72, sx, wq, k, sw, o, a, m, n, k, tp), UNSUP),       # ldx % 16
        ((xq, k, sx, wq, k, sw, o, a, m, 12, k, tp), UNSUP),       # n % 8
        ((xq + 8, k, sx, wq, k, sw, o, a, m, n, k, tp), UNSUP),
        ((xq, k, sx + 2, wq, k, sw, o, a, m, n, k, tp), UNSUP),
        ((xq, k, sx, wq, k, sw, o, a + 4, m, n, k, tp), UNSUP),
        ((xq, k, sx, wq, k, sw, o, a, m, n, k, 32), UNSUP),
    ]
    for args, want in cases:
        assert w8a8_call(*args) == want, args
    for b in (XQ, SX, WQ, SW, O, A):
        assert b.untouched()
    assert w8a8_call(None, k, None, wq, k, sw, None, None, 0, n, k, tp) == OK
    for b in (XQ, SX, WQ, SW, O, A):
        assert b.untouched()


def quant_call(x, ldx, xq, ldq, sx, m, k):
    return rpl.lib().rpl_quant_per_token(x, ldx, xq, ldq, sx, m, k, None)


def test_quant_validation():
    m, k = 5, 64
    X, Q, S = Buf(m * k * 2), Buf(m * k), Buf(m * 4)
    x, q, sx = X.ptr, Q.ptr, S.ptr
    cases = [
        ((None, k, q, k, sx, m, k), NULL),
        ((x, k, None, k, sx, m, k), NULL),
        ((x, k, q, k, None, m, k), NULL),
        ((x, k, q, k, sx, -1, k), INVALID),
        ((x, k, q, k, sx, m, 0), INVALID),
        ((x, 56, q, k, sx, m, k), INVALID),            # ldx < k
        ((x, k, q, 56, sx, m, k), INVALID),            # ldq < k
        ((x, k, x + 16, k, sx, m, k), INVALID),        # xq overlaps x
        ((x, k, q, k, x + 64, m, k), INVALID),         # x_scale overlaps x
        ((x, k, q, k, q + 32, m, k), INVALID),         # x_scale overlaps xq
        ((x, 76, q, 76, sx, m, 68), UNSUP),            # k % 8
        ((x, 68, q, k, sx, m, k), UNSUP),              # ldx % 8
        ((x, k, q, 68, sx, m, k), UNSUP),              # ldq % 8
        ((x + 8, k, q, k, sx, m, k), UNSUP),
        ((x, k, q + 8, k, sx, m, k), UNSUP),
        ((x, k, q, k, sx + 2, m, k), UNSUP),
        ((1 << 44, k, 1 << 45, k, 1 << 46, 1 << 31, k), UNSUP),   # m >= 2^31 (far-apart fake addresses)
    ]
    for args, want in cases:
        assert quant_call(*args) == want, args
    for b in (X, Q, S):
        assert b.untouched()
    assert quant_call(None, k, None, k, None, 0, k) == OK


def fused_call(xs, ldx, ws, ldw, tp, m, mv, n, k, res, gam, eps, y, ro, work, wbytes):
    import ctypes
    xa = (ctypes.c_void_p * max(tp, 1))(*(xs + [None] * max(0, tp - len(xs)))[:max(tp, 1)])
    wa = (ctypes.c_void_p * max(tp, 1))(*(ws + [None] * max(0, tp - len(ws)))[:max(tp, 1)])
    return rpl.lib().rpl_matmul_reduce_rmsnorm(ctypes.cast(xa, ctypes.c_void_p), ldx, ctypes.cast(wa, ctypes.c_void_p),
                                               ldw, tp, m, mv, n, k, res, gam, eps, y, ro, work, wbytes, None)


def test_fused_decode_workspace_size():
    L = rpl.lib()
    # header (256 B + a 4-byte call count for each of up to 1024 workgroups), then the 8-byte
    # slots of two bf16 products each: [m][tp][n/2]
    hdr = 256 + 4 * 1024
    assert L.rpl_matmul_reduce_rmsnorm_workspace_size(4, 3584, 2) == hdr + 4 * 4 * 2 * 3584
    assert L.rpl_matmul_reduce_rmsnorm_workspace_size(1, 8, 1) == hdr + 4 * 8
    assert L.rpl_matmul_reduce_rmsnorm_workspace_size(64, 8192, 16) == hdr + 4 * 64 * 16 * 8192
    assert L.rpl_matmul_reduce_rmsnorm_workspace_size(65, 64, 2) == -1
    assert L.rpl_matmul_reduce_rmsnorm_workspace_size(-1, 64, 2) == -1
    assert L.rpl_matmul_reduce_rmsnorm_workspace_size(4, 8200, 2) == -1
    assert L.rpl_matmul_reduce_rmsnorm_workspace_size(4, 64, 0) == -1
    assert L.rpl_matmul_reduce_rmsnorm_workspace_size(4, 64, 17) == -1


def test_fused_decode_validation():
    tp, m, n, k = 2, 4, 64, 32
    wsz = rpl.lib().rpl_matmul_reduce_rmsnorm_workspace_size(m, n, tp)
    X0, X1, W0, W1 = Buf(m * k * 2), Buf(m * k * 2), Buf(n * k * 2), Buf(n * k * 2)
    R, G, Y, RO = Buf(m * n * 2), Buf(n * 2), Buf(m * n * 2), Buf(m * n * 2)
    WS = Buf(wsz + 512)
    ws_ptr = WS.ptr + ((-WS.ptr) % 256)
    xs, wl = [X0.ptr, X1.ptr], [W0.ptr, W1.ptr]
    r, g, y, ro = R.ptr, G.ptr, Y.ptr, RO.ptr
    base = (xs, k, wl, k, tp, m, m, n, k, r, g, 1e-6, y, ro, ws_ptr, wsz)

    def case(**kw):
        names = ["xs", "ldx", "ws", "ldw", "tp", "m", "mv", "n", "k", "res", "gam", "eps", "y", "ro", "work", "wbytes"]
        a = dict(zip(names, base))
        a.update(kw)
        return fused_call(*[a[nm] for nm in names])

    cases = [
        (dict(xs=[X0.ptr, None]), NULL), (dict(ws=[None, W1.ptr]), NULL), (dict(res=None), NULL),
        (dict(gam=None), NULL), (dict(y=None), NULL), (dict(work=None), NULL),
        (dict(m=-1), INVALID), (dict(mv=5), INVALID), (dict(mv=-1), INVALID), (dict(n=0), INVALID),
        (dict(k=0), INVALID), (dict(tp=0), INVALID), (dict(ldx=24), INVALID), (dict(ldw=24), INVALID),
        (dict(eps=-1.0), INVALID), (dict(eps=float("nan")), INVALID), (dict(wbytes=wsz - 1), INVALID),
        (dict(y=r), INVALID),                       # y aliases the residual
        (dict(ro=y), INVALID),                      # residual_out aliases y
        (dict(work=ws_ptr, y=ws_ptr + 256), INVALID),  # y inside the workspace
        (dict(ro=r + 16), INVALID),                 # residual_out partially overlaps the residual
        (dict(tp=17, xs=xs * 9, ws=wl * 9), UNSUP), (dict(m=65, mv=4, res=1 << 40, y=1 << 41, ro=1 << 42, work=1 << 43, wbytes=1 << 20), UNSUP),
        (dict(n=60, res=1 << 40, y=1 << 41, ro=1 << 42, work=1 << 43, wbytes=1 << 20), UNSUP), (dict(k=36, ldx=40, ldw=40), UNSUP), (dict(ldx=36), UNSUP),
        (dict(n=8200, res=1 << 40, y=1 << 41, ro=1 << 42, work=1 << 43, wbytes=1 << 30), UNSUP),  # n > 8192
        (dict(xs=[X0.ptr + 8, X1.ptr]), UNSUP), (dict(work=ws_ptr + 16, wbytes=wsz), UNSUP),
        (dict(y=y + 8), UNSUP),
    ]
    for kw, want in cases:
        assert case(**kw) == want, kw
    for b in (X0, X1, W0, W1, R, G, Y, RO, WS):
        assert b.untouched()
    assert case(m=0, mv=0, res=None, y=None, ro=None, work=None, wbytes=0) == OK


def _parr(ptrs):
    import ctypes
    return ctypes.cast((ctypes.c_void_p * len(ptrs))(*ptrs), ctypes.c_void_p)


def test_sum_partials_validation():
    L = rpl.lib()
    m, n, tp = 3, 64, 2
    P0, P1, O = Buf(m * n * 2), Buf(m * n * 2), Buf(m * n * 2)
    p, o = [P0.ptr, P1.ptr], O.ptr
    call = lambda ps, tp_, m_, n_, ld, out: L.rpl_sum_partials(_parr(ps) if ps is not None else None, tp_, m_, n_,
                                                              ld, out, None)
    cases = [((None, tp, m, n, n, o), NULL), (([P0.ptr, None], tp, m, n, n, o), NULL), ((p, tp, m, n, n, None), NULL),
             ((p, 0, m, n, n, o), INVALID), ((p, tp, -1, n, n, o), INVALID), ((p, tp, m, 0, n, o), INVALID),
             ((p, tp, m, n, 56, o), INVALID), ((p, tp, m, n, n, P1.ptr + 32), INVALID),
             ((p * 9, 17, m, n, n, o), UNSUP), ((p, tp, m, 60, 64, o), UNSUP), ((p, tp, m, n, 68, o), UNSUP),
             ((p, tp, m, n, n, o + 8), UNSUP), (([P0.ptr + 8, P1.ptr], tp, m, n, n, o), UNSUP)]
    for args, want in cases:
        assert call(*args) == want, args
    for b in (P0, P1, O):
        assert b.untouched()
    assert call([None, None], tp, 0, n, n, None) == OK


def test_token_rows_validation():
    L = rpl.lib()
    m, n, tp = 5, 64, 2
    mc = 3
    X, O = Buf(m * n * 2), Buf(mc * n * 2)
    x, o = X.ptr, O.ptr
    shard = lambda x_, ld, m_, n_, tp_, r, out: L.rpl_shard_rows(x_, ld, m_, n_, tp_, r, out, None)
    cases = [((None, n, m, n, tp, 0, o), NULL), ((x, n, m, n, tp, 0, None), NULL),
             ((x, n, -1, n, tp, 0, o), INVALID), ((x, n, m, 0, tp, 0, o), INVALID), ((x, n, m, n, 0, 0, o), INVALID),
             ((x, n, m, n, tp, 2, o), INVALID), ((x, n, m, n, tp, -1, o), INVALID), ((x, 56, m, n, tp, 0, o), INVALID),
             ((x, n, m, n, tp, 0, x + 64), INVALID),
             ((x, 60, m, 60, tp, 0, o), UNSUP), ((x, 68, m, n, tp, 0, o), UNSUP), ((x + 8, n, m, n, tp, 0, o), UNSUP),
             ((x, n, m, n, tp, 0, o + 8), UNSUP)]
    for args, want in cases:
        assert shard(*args) == want, args
    assert shard(None, n, 0, n, tp, 1, None) == OK
    C0, C1, G = Buf(mc * n * 2), Buf(mc * n * 2), Buf(m * n * 2)
    c, g = [C0.ptr, C1.ptr], G.ptr
    gather = lambda cs, tp_, mc_, ld, m_, n_, out: L.rpl_gather_rows(_parr(cs) if cs is not None else None, tp_, mc_,
                                                                    ld, m_, n_, out, None)
    cases = [((None, tp, mc, n, m, n, g), NULL), (([C0.ptr, None], tp, mc, n, m, n, g), NULL),
             ((c, tp, mc, n, m, n, None), NULL),
             ((c, 0, mc, n, m, n, g), INVALID), ((c, tp, -1, n, m, n, g), INVALID), ((c, tp, mc, n, -1, n, g), INVALID),
             ((c, tp, mc, n, 7, n, g), INVALID), ((c, tp, mc, n, m, 0, g), INVALID), ((c, tp, mc, 56, m, n, g), INVALID),
             ((c, tp, mc, n, m, n, C1.ptr + 32), INVALID),
             ((c * 9, 17, mc, n, m, n, g), UNSUP), ((c, tp, mc, 68, m, n, g), UNSUP), ((c, tp, mc, 60, m, 60, g), UNSUP),
             ((c, tp, mc, n, m, n, g + 8), UNSUP), (([C0.ptr + 8, C1.ptr], tp, mc, n, m, n, g), UNSUP)]
    for args, want in cases:
        assert gather(*args) == want, args
    for b in (X, O, C0, C1, G):
        assert b.untouched()
    assert gather([None, None], tp, mc, n, 0, n, None) == OK


def test_hidden_split_validation():
    L = rpl.lib()
    m, ns, ld, tp = 3, 32, 64, 2
    P0, P1, R, RO = Buf(m * ld * 2), Buf(m * ld * 2), Buf(m * ld * 2), Buf(m * ld * 2)
    H, S0, S1, G, Y = Buf(m * ns * 4), Buf(m * 4), Buf(m * 4), Buf(ns * 2), Buf(m * ld * 2)
    p = [P0.ptr, P1.ptr]
    s1 = lambda ps, tp_, m_, ns_, ld_, r, ro, h, ss: L.rpl_reduce_slice_sumsq(
        _parr(ps) if ps is not None else None, tp_, m_, ns_, ld_, r, ro, h, ss, None)
    base1 = (p, tp, m, ns, ld, R.ptr, RO.ptr, H.ptr, S0.ptr)
    c1 = [((None,) + base1[1:], NULL), (base1[:5] + (None,) + base1[6:], NULL), (base1[:8] + (None,), NULL),
          ((p, 0) + base1[2:], INVALID), ((p, tp, m, 0) + base1[4:], INVALID), ((p, tp, m, ns, 24) + base1[5:], INVALID),
          (base1[:6] + (P0.ptr + 16,) + base1[7:], INVALID), (base1[:7] + (RO.ptr,) + base1[8:], INVALID),
          (base1[:8] + (H.ptr + 8,), INVALID), ((p * 9, 17) + base1[2:], UNSUP), ((p, tp, m, 36, ld) + base1[5:], UNSUP),
          ((p, tp, m, ns, 68) + base1[5:], UNSUP), (base1[:7] + (H.ptr + 8, S0.ptr), UNSUP),
          ((p, tp, m, 16392, 16392, 1 << 40, 1 << 41, 1 << 42, 1 << 43), UNSUP)]
    for args, want in c1:
        assert s1(*args) == want, args
    s2 = lambda h, sp, tp_, m_, ns_, nt, g, eps, y, ld_: L.rpl_rmsnorm_slice_apply(
        h, _parr(sp) if sp is not None else None, tp_, m_, ns_, nt, g, eps, y, ld_, None)
    sp = [S0.ptr, S1.ptr]
    base2 = (H.ptr, sp, tp, m, ns, 64, G.ptr, 1e-6, Y.ptr, ld)
    c2 = [((H.ptr, None) + base2[2:], NULL), (base2[:6] + (None,) + base2[7:], NULL), ((None,) + base2[1:], NULL),
          (base2[:8] + (None, ld), NULL), ((H.ptr, [S0.ptr, None]) + base2[2:], NULL),
          (base2[:5] + (16,) + base2[6:], INVALID), (base2[:7] + (-1.0,) + base2[8:], INVALID),
          (base2[:9] + (16,), INVALID), (base2[:8] + (H.ptr, ld), INVALID),
          (base2[:4] + (36,) + base2[5:], UNSUP), (base2[:8] + (Y.ptr + 8, ld), UNSUP),
          ((H.ptr + 4,) + base2[1:], UNSUP), ((H.ptr, [S0.ptr + 2, S1.ptr]) + base2[2:], UNSUP)]
    for args, want in c2:
        assert s2(*args) == want, args
    for b in (P0, P1, R, RO, H, S0, S1, G, Y):
        assert b.untouched()
    assert s1([None, None], tp, 0, ns, ld, None, None, None, None) == OK
    assert s2(None, sp, tp, 0, ns, 64, G.ptr, 1e-6, None, ld) == OK


def test_binding_rejects_host_tensors():
    """The Python binding refuses CPU tensors before anything reaches the library."""
    import torch
    x = torch.zeros(4, 16, dtype=torch.bfloat16)
    w = torch.zeros(8, 16, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU"):
        rpl.rpl_partial(x, w, 2)


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(rpl, "_lib", None)
    monkeypatch.setattr(rpl, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="not built"):
        rpl.lib()


def test_product_path_does_not_import_the_oracle():
    pkg = os.path.join(ROOT, "row_matmul_reduce_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".cpp", ".h")):
                text = open(os.path.join(dirpath, f), encoding="utf-8").read()
                assert not re.search(r"^\s*(import|from)\s+oracle\b|rpl_oracle|\borc_", text, flags=re.M), f


def test_read_ceiling_validation():
    """The measurement helper checks its arguments on the host like the path's calls."""
    L = rpl.lib()
    B, S = Buf(4096), Buf(64)
    call = lambda p, nbytes, grid, sink: L.rpl_read_ceiling(p, nbytes, grid, sink, None)
    assert call(None, 4096, 256, S.ptr) == NULL
    assert call(B.ptr, 4096, 256, None) == NULL
    assert call(B.ptr, 8, 256, S.ptr) == INVALID
    assert call(B.ptr, 4100, 256, S.ptr) == INVALID
    assert call(B.ptr, 4096, 0, S.ptr) == INVALID
    assert call(B.ptr, 4096, 65537, S.ptr) == INVALID
    assert call(B.ptr + 8, 4080, 256, S.ptr) == UNSUP
    assert call(B.ptr, 4096, 256, S.ptr + 2) == UNSUP
    assert B.untouched() and S.untouched()


def test_mfma_ceiling_validation():
    """The MFMA measurement helper checks its arguments on the host before any HIP call."""
    L = rpl.lib()
    B, C, S = Buf(4096), Buf(4096), Buf(64)
    need = rpl.MFMA_CEILING_OPS_BYTES
    call = lambda p, nbytes, kind, iters, c, s: L.rpl_mfma_ceiling(p, nbytes, kind, iters, c, s, None)
    assert call(None, need, 0, 10, C.ptr, S.ptr) == NULL
    assert call(B.ptr, need, 0, 10, None, S.ptr) == NULL
    assert call(B.ptr, need, 0, 10, C.ptr, None) == NULL
    assert call(B.ptr, need - 16, 0, 10, C.ptr, S.ptr) == INVALID
    assert call(B.ptr, need, 2, 10, C.ptr, S.ptr) == INVALID
    assert call(B.ptr, need, -1, 10, C.ptr, S.ptr) == INVALID
    assert call(B.ptr, need, 0, 0, C.ptr, S.ptr) == INVALID
    assert call(B.ptr, need, 1, (1 << 20) + 1, C.ptr, S.ptr) == INVALID
    assert call(B.ptr + 8, need, 0, 10, C.ptr, S.ptr) == UNSUP
    assert call(B.ptr, need, 0, 10, C.ptr + 4, S.ptr) == UNSUP
    assert call(B.ptr, need, 1, 10, C.ptr, S.ptr + 2) == UNSUP
    assert B.untouched() and C.untouched() and S.untouched()


def test_fused_noalloc_validation():
    """The no-allocation form checks like the workspace form (no workspace arguments) and refuses
    shapes whose hand-off memory exceeds its 4 MiB array, all on the host before any HIP call."""
    import ctypes
    L = rpl.lib()
    tp, m, n, k = 2, 4, 64, 32
    X0, X1, W0, W1 = Buf(m * k * 2), Buf(m * k * 2), Buf(n * k * 2), Buf(n * k * 2)
    R, G, Y, RO = Buf(m * n * 2), Buf(n * 2), Buf(m * n * 2), Buf(m * n * 2)

    def call(xs=None, ws=None, **kw):
        a = dict(ldx=k, ldw=k, tp=tp, m=m, mv=m, n=n, k=k, res=R.ptr, gam=G.ptr, eps=1e-6, y=Y.ptr, ro=RO.ptr)
        a.update(kw)
        xs = xs if xs is not None else [X0.ptr, X1.ptr]
        ws = ws if ws is not None else [W0.ptr, W1.ptr]
        xa = (ctypes.c_void_p * len(xs))(*xs)
        wa = (ctypes.c_void_p * len(ws))(*ws)
        return L.rpl_matmul_reduce_rmsnorm_noalloc(ctypes.cast(xa, ctypes.c_void_p), a["ldx"],
                                                   ctypes.cast(wa, ctypes.c_void_p), a["ldw"], a["tp"], a["m"],
                                                   a["mv"], a["n"], a["k"], a["res"], a["gam"], a["eps"], a["y"],
                                                   a["ro"], None)

    cases = [
        (dict(xs=[X0.ptr, None]), NULL), (dict(res=None), NULL), (dict(gam=None), NULL), (dict(ro=None), NULL),
        (dict(m=-1), INVALID), (dict(mv=5), INVALID), (dict(n=0), INVALID), (dict(ldw=24), INVALID),
        (dict(eps=-1.0), INVALID), (dict(y=R.ptr), INVALID), (dict(ro=Y.ptr), INVALID),
        (dict(n=60), UNSUP), (dict(y=Y.ptr + 8), UNSUP),
        # m > 64 (fake device pointers far apart, so no overlap check fires first)
        (dict(m=65, mv=4, res=1 << 40, y=1 << 41, ro=1 << 42), UNSUP),
        # hand-off memory of 4,352 + 4 * 64 * 2 * 8192 bytes > 4 MiB (fake device pointers: refused first)
        (dict(m=64, mv=0, n=8192, res=1 << 40, y=1 << 41, ro=1 << 42, gam=1 << 43), UNSUP),
    ]
    for kw, want in cases:
        assert call(**kw) == want, kw
    for b in (X0, X1, W0, W1, R, G, Y, RO):
        assert b.untouched()
    assert call(m=0, mv=0, res=None, y=None, ro=None) == OK
