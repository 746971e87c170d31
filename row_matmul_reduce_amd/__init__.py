"""row_matmul_reduce_amd -- row-parallel matmul + reduce on AMD MI355X (gfx950).

Thin Python binding over the C ABI of ``librpl.so`` (declared in
``include/rpl.h``).  It only marshals arguments: it checks dtypes, devices
and layouts of torch tensors, allocates outputs when none are given, and
passes raw device pointers plus torch's current HIP stream.  Every step of
the computation runs in the library's HIP kernels; there is no fallback: if
the library is missing, every call raises.

    rpl_partial(x, w, tp)                      -> [M_pad, n] bf16 partial
    rpl_reduce_chunk_rmsnorm(partials, residual, gamma, eps)
                                               -> (y, residual_out)
    rpl_w8a8_partial(xq, x_scale, wq, w_scale, tp, want_acc=False)
                                               -> out (, acc)
    rpl_quant_per_token(x)                     -> (xq int8, x_scale fp32)
    rpl_matmul_reduce_rmsnorm(x_shards, w_shards, residual, gamma, eps)
                                               -> (y, residual_out), one launch
    rpl_sum_partials(partials)                 -> bf16 sum (all-reduce form)
    rpl_reduce_slice_sumsq / rpl_rmsnorm_slice_apply
                                               hidden-split epilogue, two steps
    rpl_shard_rows(x, tp, rank)                -> the rank's block of the padded rows
    rpl_gather_rows(chunks, m)                 -> blocks in rank order, pad rows dropped
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "librpl.so")

RPL_OK, RPL_ERR_NULL, RPL_ERR_INVALID, RPL_ERR_UNSUPPORTED, RPL_ERR_LAUNCH = range(5)
RPL_MAX_TP = 16

_p, _i64, _i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
_lib = None


class RplError(RuntimeError):
    """A non-OK status from librpl."""

    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn}: {rpl_status_string(status)}")


def lib() -> ctypes.CDLL:
    """Load librpl.so (built in-tree by ``python -m row_matmul_reduce_amd.build``)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"librpl.so is not built ({LIB_PATH}); run python -m row_matmul_reduce_amd.build")
        L = ctypes.CDLL(LIB_PATH)
        L.rpl_partial.restype = ctypes.c_int
        L.rpl_partial.argtypes = [_p, _i64, _p, _i64, _p, _i64, _i64, _i64, _i32, _p]
        L.rpl_reduce_chunk_rmsnorm.restype = ctypes.c_int
        L.rpl_reduce_chunk_rmsnorm.argtypes = [_p, _i32, _i64, _i64, _p, _p, ctypes.c_float, _p, _p, _p]
        L.rpl_w8a8_partial.restype = ctypes.c_int
        L.rpl_w8a8_partial.argtypes = [_p, _i64, _p, _p, _i64, _p, _p, _p, _i64, _i64, _i64, _i32, _p]
        L.rpl_matmul_reduce_rmsnorm_workspace_size.restype = _i64
        L.rpl_matmul_reduce_rmsnorm_workspace_size.argtypes = [_i64, _i64, _i32]
        L.rpl_matmul_reduce_rmsnorm.restype = ctypes.c_int
        L.rpl_matmul_reduce_rmsnorm.argtypes = [_p, _i64, _p, _i64, _i32, _i64, _i64, _i64, _i64, _p, _p,
                                                ctypes.c_float, _p, _p, _p, _i64, _p]
        L.rpl_matmul_reduce_rmsnorm_noalloc.restype = ctypes.c_int
        L.rpl_matmul_reduce_rmsnorm_noalloc.argtypes = [_p, _i64, _p, _i64, _i32, _i64, _i64, _i64, _i64, _p, _p,
                                                         ctypes.c_float, _p, _p, _p]
        L.rpl_sum_partials.restype = ctypes.c_int
        L.rpl_sum_partials.argtypes = [_p, _i32, _i64, _i64, _i64, _p, _p]
        L.rpl_reduce_slice_sumsq.restype = ctypes.c_int
        L.rpl_reduce_slice_sumsq.argtypes = [_p, _i32, _i64, _i64, _i64, _p, _p, _p, _p, _p]
        L.rpl_rmsnorm_slice_apply.restype = ctypes.c_int
        L.rpl_rmsnorm_slice_apply.argtypes = [_p, _p, _i32, _i64, _i64, _i64, _p, ctypes.c_float, _p, _i64, _p]
        L.rpl_quant_per_token.restype = ctypes.c_int
        L.rpl_quant_per_token.argtypes = [_p, _i64, _p, _i64, _p, _i64, _i64, _p]
        L.rpl_shard_rows.restype = ctypes.c_int
        L.rpl_shard_rows.argtypes = [_p, _i64, _i64, _i64, _i32, _i32, _p, _p]
        L.rpl_gather_rows.restype = ctypes.c_int
        L.rpl_gather_rows.argtypes = [_p, _i32, _i64, _i64, _i64, _i64, _p, _p]
        L.rpl_read_ceiling.restype = ctypes.c_int
        L.rpl_read_ceiling.argtypes = [_p, _i64, _i32, _p, _p]
        L.rpl_mfma_ceiling.restype = ctypes.c_int
        L.rpl_mfma_ceiling.argtypes = [_p, _i64, _i32, _i32, _p, _p, _p]
        L.rpl_status_string.restype = ctypes.c_char_p
        L.rpl_status_string.argtypes = [ctypes.c_int]
        L.rpl_version.restype = ctypes.c_int32
        L.rpl_version.argtypes = []
        _lib = L
    return _lib


def rpl_status_string(status: int) -> str:
    return lib().rpl_status_string(int(status)).decode()


def rpl_version() -> int:
    return int(lib().rpl_version())


def _check(fn: str, status: int) -> None:
    if status != RPL_OK:
        raise RplError(fn, status)


def _torch():
    import torch
    return torch


def _dev(t, name: str, dtype, ndim: int):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name}: must be a GPU (HIP) tensor, got {t.device}")
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if t.dim() != ndim:
        raise ValueError(f"{name}: expected {ndim}-D, got shape {tuple(t.shape)}")
    if ndim == 2 and t.shape[1] > 1 and t.stride(1) != 1:
        raise ValueError(f"{name}: rows must be contiguous (stride(1) == 1)")
    if ndim == 1 and t.shape[0] > 1 and t.stride(0) != 1:
        raise ValueError(f"{name}: must be contiguous")
    return t


def _stream(t, stream):
    torch = _torch()
    if stream is None:
        return torch.cuda.current_stream(t.device).cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _ld(t) -> int:
    return t.stride(0) if t.shape[0] > 1 else t.shape[1]


def m_pad_of(m: int, tp: int) -> int:
    return -(-m // tp) * tp


def rpl_partial(x, w, tp: int, out=None, stream=None):
    """One rank's bf16 partial, [M_pad, n] in reduce-scatter chunk layout."""
    torch = _torch()
    _dev(x, "x", torch.bfloat16, 2)
    _dev(w, "w", torch.bfloat16, 2)
    m, k = x.shape
    n = w.shape[0]
    if w.shape[1] != k:
        raise ValueError(f"x {tuple(x.shape)} and w {tuple(w.shape)} disagree on k")
    mp = m_pad_of(m, tp) if tp >= 1 else m
    if out is None:
        out = torch.empty((mp, n), dtype=torch.bfloat16, device=x.device)
    _dev(out, "out", torch.bfloat16, 2)
    if tuple(out.shape) != (mp, n) or not out.is_contiguous():
        raise ValueError(f"out must be a contiguous [{mp}, {n}] tensor")
    st = lib().rpl_partial(x.data_ptr(), _ld(x), w.data_ptr(), _ld(w), out.data_ptr(), m, n, k, tp,
                           _stream(x, stream))
    _check("rpl_partial", st)
    return out


def rpl_reduce_chunk_rmsnorm(partials, residual, gamma, eps: float, y=None, residual_out=None, stream=None):
    """Sum of the tp chunk partials + residual, then RMSNorm -> (y, residual_out)."""
    torch = _torch()
    partials = list(partials)
    if not partials:
        raise ValueError("need at least one partial")
    for i, p in enumerate(partials):
        _dev(p, f"partials[{i}]", torch.bfloat16, 2)
        if tuple(p.shape) != tuple(partials[0].shape) or not p.is_contiguous():
            raise ValueError("partials must be contiguous and share one shape")
    m_chunk, n = partials[0].shape
    _dev(residual, "residual", torch.bfloat16, 2)
    _dev(gamma, "gamma", torch.bfloat16, 1)
    if tuple(residual.shape) != (m_chunk, n) or not residual.is_contiguous():
        raise ValueError("residual must be a contiguous [m_chunk, n] tensor")
    if gamma.shape[0] != n:
        raise ValueError("gamma must have n entries")
    if y is None:
        y = torch.empty((m_chunk, n), dtype=torch.bfloat16, device=residual.device)
    if residual_out is None:
        residual_out = torch.empty((m_chunk, n), dtype=torch.bfloat16, device=residual.device)
    for name, t in (("y", y), ("residual_out", residual_out)):
        _dev(t, name, torch.bfloat16, 2)
        if tuple(t.shape) != (m_chunk, n) or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous [m_chunk, n] tensor")
    arr = (ctypes.c_void_p * len(partials))(*[p.data_ptr() for p in partials])
    st = lib().rpl_reduce_chunk_rmsnorm(ctypes.cast(arr, ctypes.c_void_p), len(partials), m_chunk, n,
                                        residual.data_ptr(), gamma.data_ptr(), float(eps), y.data_ptr(),
                                        residual_out.data_ptr(), _stream(residual, stream))
    _check("rpl_reduce_chunk_rmsnorm", st)
    return y, residual_out


def rpl_w8a8_partial(xq, x_scale, wq, w_scale, tp: int, out=None, acc=None, want_acc: bool = False,
                     stream=None):
    """int8 x int8 rank partial, dequantised to bf16 [M_pad, n]; optionally the int32 accumulators."""
    torch = _torch()
    _dev(xq, "xq", torch.int8, 2)
    _dev(wq, "wq", torch.int8, 2)
    _dev(x_scale, "x_scale", torch.float32, 1)
    _dev(w_scale, "w_scale", torch.float32, 1)
    m, k = xq.shape
    n = wq.shape[0]
    if wq.shape[1] != k:
        raise ValueError("xq and wq disagree on k")
    if x_scale.shape[0] != m or w_scale.shape[0] != n:
        raise ValueError("x_scale must have m entries and w_scale n entries")
    mp = m_pad_of(m, tp) if tp >= 1 else m
    if out is None:
        out = torch.empty((mp, n), dtype=torch.bfloat16, device=xq.device)
    _dev(out, "out", torch.bfloat16, 2)
    if tuple(out.shape) != (mp, n) or not out.is_contiguous():
        raise ValueError(f"out must be a contiguous [{mp}, {n}] tensor")
    if acc is None and want_acc:
        acc = torch.empty((mp, n), dtype=torch.int32, device=xq.device)
    if acc is not None:
        _dev(acc, "acc", torch.int32, 2)
        if tuple(acc.shape) != (mp, n) or not acc.is_contiguous():
            raise ValueError(f"acc must be a contiguous [{mp}, {n}] tensor")
    st = lib().rpl_w8a8_partial(xq.data_ptr(), _ld(xq), x_scale.data_ptr(), wq.data_ptr(), _ld(wq),
                                w_scale.data_ptr(), out.data_ptr(), None if acc is None else acc.data_ptr(),
                                m, n, k, tp, _stream(xq, stream))
    _check("rpl_w8a8_partial", st)
    return (out, acc) if acc is not None else out


def rpl_quant_per_token(x, xq=None, x_scale=None, stream=None):
    """Per-token dynamic int8 quantisation of a bf16 [m, k] activation.

    Returns (xq int8 [m, k], x_scale fp32 [m]), the operands of rpl_w8a8_partial.
    """
    torch = _torch()
    _dev(x, "x", torch.bfloat16, 2)
    m, k = x.shape
    if xq is None:
        xq = torch.empty((m, k), dtype=torch.int8, device=x.device)
    if x_scale is None:
        x_scale = torch.empty((m,), dtype=torch.float32, device=x.device)
    _dev(xq, "xq", torch.int8, 2)
    _dev(x_scale, "x_scale", torch.float32, 1)
    if tuple(xq.shape) != (m, k) or x_scale.shape[0] != m:
        raise ValueError(f"xq must be [{m}, {k}] and x_scale [{m}]")
    st = lib().rpl_quant_per_token(x.data_ptr(), _ld(x), xq.data_ptr(), _ld(xq), x_scale.data_ptr(), m, k,
                                   _stream(x, stream))
    _check("rpl_quant_per_token", st)
    return xq, x_scale


def _ptrs(tensors):
    arr = (ctypes.c_void_p * len(tensors))(*[t.data_ptr() for t in tensors])
    return arr, ctypes.cast(arr, _p)


def rpl_sum_partials(partials, out=None, stream=None):
    """All-reduce form: bf16 sum of the tp [m, n] bf16 partials (same row stride)."""
    torch = _torch()
    for i, t in enumerate(partials):
        _dev(t, f"partials[{i}]", torch.bfloat16, 2)
    m, n = partials[0].shape
    ldp = _ld(partials[0])
    if any(t.shape != (m, n) or _ld(t) != ldp for t in partials):
        raise ValueError("partials must share shape and row stride")
    if out is None:
        out = torch.empty((m, n), dtype=torch.bfloat16, device=partials[0].device)
    _dev(out, "out", torch.bfloat16, 2)
    if tuple(out.shape) != (m, n) or not out.is_contiguous():
        raise ValueError(f"out must be a contiguous [{m}, {n}] tensor")
    keep, arr = _ptrs(partials)
    st = lib().rpl_sum_partials(arr, len(partials), m, n, ldp, out.data_ptr(), _stream(out, stream))
    _check("rpl_sum_partials", st)
    return out


def rpl_shard_rows(x, tp: int, rank: int, out=None, stream=None):
    """Rank `rank`'s block of the zero-padded token rows of x [m, n]: [ceil(m/tp), n]."""
    torch = _torch()
    _dev(x, "x", torch.bfloat16, 2)
    m, n = x.shape
    mc = -(-m // tp) if tp >= 1 else 0
    if out is None:
        out = torch.empty((mc, n), dtype=torch.bfloat16, device=x.device)
    _dev(out, "out", torch.bfloat16, 2)
    if tuple(out.shape) != (mc, n) or not out.is_contiguous():
        raise ValueError(f"out must be a contiguous [{mc}, {n}] tensor")
    st = lib().rpl_shard_rows(x.data_ptr(), _ld(x), m, n, tp, rank, out.data_ptr(), _stream(out, stream))
    _check("rpl_shard_rows", st)
    return out


def rpl_gather_rows(chunks, m: int, out=None, stream=None):
    """The tp [m_chunk, n] blocks in rank order, cut back to the first m rows: [m, n]."""
    torch = _torch()
    for i, t in enumerate(chunks):
        _dev(t, f"chunks[{i}]", torch.bfloat16, 2)
    mc, n = chunks[0].shape
    ld = _ld(chunks[0])
    if any(t.shape != (mc, n) or _ld(t) != ld for t in chunks):
        raise ValueError("chunks must share shape and row stride")
    if out is None:
        out = torch.empty((m, n), dtype=torch.bfloat16, device=chunks[0].device)
    _dev(out, "out", torch.bfloat16, 2)
    if tuple(out.shape) != (m, n) or not out.is_contiguous():
        raise ValueError(f"out must be a contiguous [{m}, {n}] tensor")
    keep, arr = _ptrs(chunks)
    st = lib().rpl_gather_rows(arr, len(chunks), mc, ld, m, n, out.data_ptr(), _stream(out, stream))
    _check("rpl_gather_rows", st)
    return out


def rpl_reduce_slice_sumsq(partials, residual, residual_out, h=None, sumsq=None, stream=None):
    """Hidden-split step 1 on one column slice.  partials, residual and residual_out are
    [m, n_slice] views sharing one row stride (e.g. full[:, c0:c0 + n_slice]).
    Returns (h fp32 [m, n_slice], sumsq fp32 [m])."""
    torch = _torch()
    for i, t in enumerate(partials):
        _dev(t, f"partials[{i}]", torch.bfloat16, 2)
    _dev(residual, "residual", torch.bfloat16, 2)
    _dev(residual_out, "residual_out", torch.bfloat16, 2)
    m, ns = residual.shape
    ld = _ld(residual)
    views = list(partials) + [residual_out]
    if any(t.shape != (m, ns) or _ld(t) != ld for t in views):
        raise ValueError("slices must share shape and row stride")
    if h is None:
        h = torch.empty((m, ns), dtype=torch.float32, device=residual.device)
    if sumsq is None:
        sumsq = torch.empty((m,), dtype=torch.float32, device=residual.device)
    _dev(h, "h", torch.float32, 2)
    _dev(sumsq, "sumsq", torch.float32, 1)
    if tuple(h.shape) != (m, ns) or not h.is_contiguous() or sumsq.shape[0] != m:
        raise ValueError("h must be a contiguous [m, n_slice] fp32 tensor and sumsq [m]")
    keep, arr = _ptrs(partials)
    st = lib().rpl_reduce_slice_sumsq(arr, len(partials), m, ns, ld, residual.data_ptr(), residual_out.data_ptr(),
                                      h.data_ptr(), sumsq.data_ptr(), _stream(residual, stream))
    _check("rpl_reduce_slice_sumsq", st)
    return h, sumsq


def rpl_rmsnorm_slice_apply(h, sumsq_parts, n_total: int, gamma, eps: float, y, stream=None):
    """Hidden-split step 2: y (an [m, n_slice] bf16 view) = gamma * h / sqrt(sum_r sumsq_r / n_total + eps)."""
    torch = _torch()
    _dev(h, "h", torch.float32, 2)
    _dev(gamma, "gamma", torch.bfloat16, 1)
    _dev(y, "y", torch.bfloat16, 2)
    m, ns = h.shape
    for i, t in enumerate(sumsq_parts):
        _dev(t, f"sumsq_parts[{i}]", torch.float32, 1)
        if t.shape[0] != m:
            raise ValueError("each sumsq part has m entries")
    if tuple(y.shape) != (m, ns) or gamma.shape[0] != ns or not h.is_contiguous():
        raise ValueError("shape mismatch")
    keep, arr = _ptrs(sumsq_parts)
    st = lib().rpl_rmsnorm_slice_apply(h.data_ptr(), arr, len(sumsq_parts), m, ns, n_total, gamma.data_ptr(),
                                       float(eps), y.data_ptr(), _ld(y), _stream(h, stream))
    _check("rpl_rmsnorm_slice_apply", st)
    return y


def rpl_matmul_reduce_rmsnorm_workspace(m: int, n: int, tp: int, device=None):
    """A zero-filled workspace for rpl_matmul_reduce_rmsnorm on [m, n] with tp shards (reusable
    across calls, which leave it ready for the next one)."""
    torch = _torch()
    size = lib().rpl_matmul_reduce_rmsnorm_workspace_size(m, n, tp)
    if size < 0:
        raise ValueError(f"unsupported shape m={m} n={n} tp={tp} for rpl_matmul_reduce_rmsnorm")
    return torch.zeros(max(size, 16), dtype=torch.uint8, device=device or "cuda")


def rpl_matmul_reduce_rmsnorm_status(workspace) -> int:
    """The workspace's status word (synchronises): 0, or nonzero once a call's workgroup waited past
    its bound for another (that call's y is NaN)."""
    return int(workspace[8:12].view(_torch().int32).item())


def rpl_matmul_reduce_rmsnorm_set_poll_bound(workspace, polls: int):
    """Bound, in polls, on every wait of the calls that use this workspace (0 = the default)."""
    workspace[12:16].view(_torch().int32).fill_(int(polls))


def rpl_matmul_reduce_rmsnorm(x_shards, w_shards, residual, gamma, eps: float, workspace=None, y=None,
                              residual_out=None, stream=None):
    """Single launch: every shard's product for the rows, their sum, residual add, RMSNorm.

    x_shards: tp tensors [m_valid, k] (the block's activation rows per shard, same row stride);
    w_shards: tp tensors [n, k]; residual [m, n]; gamma [n].  Rows m_valid..m-1 are padding.
    Returns (y, residual_out).
    """
    torch = _torch()
    tp = len(w_shards)
    if tp < 1 or len(x_shards) != tp:
        raise ValueError("need as many activation shards as weight shards (at least one)")
    _dev(residual, "residual", torch.bfloat16, 2)
    _dev(gamma, "gamma", torch.bfloat16, 1)
    m, n = residual.shape
    for i, t in enumerate(w_shards):
        _dev(t, f"w_shards[{i}]", torch.bfloat16, 2)
    for i, t in enumerate(x_shards):
        _dev(t, f"x_shards[{i}]", torch.bfloat16, 2)
    k = w_shards[0].shape[1]
    m_valid = x_shards[0].shape[0]
    if any(t.shape != (n, k) for t in w_shards) or any(t.shape != (m_valid, k) for t in x_shards):
        raise ValueError("shard shapes disagree")
    ldx, ldw = _ld(x_shards[0]), _ld(w_shards[0])
    if any(_ld(t) != ldx for t in x_shards) or any(_ld(t) != ldw for t in w_shards):
        raise ValueError("all shards must share one row stride")
    if not residual.is_contiguous():
        raise ValueError("residual must be contiguous")
    if y is None:
        y = torch.empty_like(residual)
    if residual_out is None:
        residual_out = torch.empty_like(residual)
    if workspace is None:
        workspace = rpl_matmul_reduce_rmsnorm_workspace(m, n, tp, residual.device)
    xs = (ctypes.c_void_p * tp)(*[t.data_ptr() for t in x_shards])
    ws = (ctypes.c_void_p * tp)(*[t.data_ptr() for t in w_shards])
    st = lib().rpl_matmul_reduce_rmsnorm(ctypes.cast(xs, _p), ldx, ctypes.cast(ws, _p), ldw, tp, m, m_valid, n, k,
                                         residual.data_ptr(), gamma.data_ptr(), float(eps), y.data_ptr(),
                                         residual_out.data_ptr(), workspace.data_ptr(),
                                         workspace.numel() * workspace.element_size(), _stream(residual, stream))
    _check("rpl_matmul_reduce_rmsnorm", st)
    return y, residual_out


def rpl_read_ceiling(t, grid: int, sink, stream=None):
    """Measurement only: read every byte of device tensor t once with `grid` workgroups (a plain
    streaming read that writes nothing; sink is a device int32 tensor of at least one element)."""
    if not t.is_cuda or not sink.is_cuda or not t.is_contiguous():
        raise ValueError("device tensors, t contiguous")
    st = lib().rpl_read_ceiling(t.data_ptr(), t.numel() * t.element_size(), int(grid), sink.data_ptr(),
                                _stream(t, stream))
    _check("rpl_read_ceiling", st)


MFMA_CEILING_OPS_BYTES = 256 * 256 * 512


def rpl_mfma_ceiling(ops, kind: int, iters: int, clocks, sink, stream=None):
    """Measurement only: 256 workgroups of four waves issue iters x 128 MFMAs per wave on operands
    taken from device tensor ops (at least MFMA_CEILING_OPS_BYTES bytes): kind 0 the bf16
    v_mfma_f32_16x16x32_bf16, kind 1 the int8 v_mfma_i32_16x16x64_i8.  clocks (device int64, 512
    entries) receives per workgroup the shader-clock and 100 MHz ticks of its MFMA loop; sink is a
    device int32 tensor of at least one element."""
    if not ops.is_cuda or not clocks.is_cuda or not sink.is_cuda or not ops.is_contiguous():
        raise ValueError("device tensors, ops contiguous")
    if clocks.numel() * clocks.element_size() < 512 * 8 or not clocks.is_contiguous():
        raise ValueError("clocks must hold 512 contiguous 8-byte entries")
    st = lib().rpl_mfma_ceiling(ops.data_ptr(), ops.numel() * ops.element_size(), int(kind), int(iters),
                                clocks.data_ptr(), sink.data_ptr(), _stream(ops, stream))
    _check("rpl_mfma_ceiling", st)


def rpl_matmul_reduce_rmsnorm_noalloc(x_shards, w_shards, residual, gamma, eps: float, y, residual_out,
                                      stream=None):
    """rpl_matmul_reduce_rmsnorm without a workspace, for callers that cannot allocate: the
    library's own device array carries the hand-offs (calls on one GPU must not overlap in
    time).  y and residual_out must be given; nothing is allocated.  Returns (y, residual_out)."""
    torch = _torch()
    tp = len(w_shards)
    if tp < 1 or len(x_shards) != tp:
        raise ValueError("need as many activation shards as weight shards (at least one)")
    _dev(residual, "residual", torch.bfloat16, 2)
    _dev(gamma, "gamma", torch.bfloat16, 1)
    _dev(y, "y", torch.bfloat16, 2)
    _dev(residual_out, "residual_out", torch.bfloat16, 2)
    m, n = residual.shape
    k = w_shards[0].shape[1]
    m_valid = x_shards[0].shape[0]
    if any(t.shape != (n, k) for t in w_shards) or any(t.shape != (m_valid, k) for t in x_shards):
        raise ValueError("shard shapes disagree")
    ldx, ldw = _ld(x_shards[0]), _ld(w_shards[0])
    if any(_ld(t) != ldx for t in x_shards) or any(_ld(t) != ldw for t in w_shards):
        raise ValueError("all shards must share one row stride")
    xs = (ctypes.c_void_p * tp)(*[t.data_ptr() for t in x_shards])
    ws = (ctypes.c_void_p * tp)(*[t.data_ptr() for t in w_shards])
    st = lib().rpl_matmul_reduce_rmsnorm_noalloc(ctypes.cast(xs, _p), ldx, ctypes.cast(ws, _p), ldw, tp, m, m_valid,
                                                 n, k, residual.data_ptr(), gamma.data_ptr(), float(eps),
                                                 y.data_ptr(), residual_out.data_ptr(), _stream(residual, stream))
    _check("rpl_matmul_reduce_rmsnorm_noalloc", st)
    return y, residual_out


__all__ = ["rpl_partial", "rpl_reduce_chunk_rmsnorm", "rpl_w8a8_partial", "rpl_quant_per_token",
           "rpl_matmul_reduce_rmsnorm", "rpl_matmul_reduce_rmsnorm_workspace", "rpl_matmul_reduce_rmsnorm_status",
           "rpl_matmul_reduce_rmsnorm_set_poll_bound", "rpl_matmul_reduce_rmsnorm_noalloc", "rpl_sum_partials",
           "rpl_reduce_slice_sumsq", "rpl_rmsnorm_slice_apply",
           "rpl_status_string", "rpl_version", "rpl_read_ceiling", "rpl_mfma_ceiling", "MFMA_CEILING_OPS_BYTES",
           "RplError", "lib", "m_pad_of", "LIB_PATH"]
