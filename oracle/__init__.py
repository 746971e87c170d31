"""CPU oracle for the row-parallel matmul + reduce hot path.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The product path
(``row_matmul_reduce_amd``) never imports, loads or calls it, and the two share
no code: the oracle is plain C (``rpl_oracle.c``), built with gcc, wrapped here
with ctypes and numpy.

Every function computes the unfused definition in fp64 (see the header of
``rpl_oracle.c`` for the passages followed and the readings taken).  Inputs are
numpy arrays: bfloat16 tensors are carried as ``uint16`` bit patterns.

Parity status of each function (what pins it lives in tests/test_oracle_pins.py):
  partial_rows           pinned: exact rational brute force, numpy fp64 GEMM,
                         one-hot / small-integer closed forms, hand-worked golden
  reduce_chunk_rmsnorm   pinned: 60-digit decimal brute force, RMS invariant,
                         scale invariance, zero row, hand-worked golden
  w8a8_rows              pinned: numpy int64 GEMM, sign symmetry, numpy float32
                         dequant in the same operation order
  sum_partials           pinned: exact rational brute force, permutation invariance
                         (fp64 sums of bf16 values are exact), integer partials, TP=1
  reduce_slice_sumsq,    pinned: slices over the whole row reproduce the pinned
  rmsnorm_slice_apply    reduce_chunk_rmsnorm; exact rational sums of squares;
                         slice-boundary invariance
  quant_per_token        pinned: exact rational nearest-integer bound, absmax code
                         +-127, power-of-two scale invariance, negation symmetry,
                         zero row, hand-worked ties-to-even golden
  f64_to_bf16            pinned: exact rational nearest-even search
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "rpl_oracle.c")
_LIB = os.path.join(_HERE, "librpl_oracle.so")

_i64 = ctypes.c_int64
_p = ctypes.c_void_p


GCC_FLAGS = ["-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
             "-fPIC", "-shared", "-Wall", "-Wextra"]


def compile_source(src: str, out: str) -> str:
    """gcc a C oracle source into a shared object (no fast-math, no FMA contraction)."""
    tmp = out + ".tmp"
    subprocess.run(["gcc", *GCC_FLAGS, "-o", tmp, src, "-lm"], check=True)
    os.replace(tmp, out)
    return out


def build(force: bool = True) -> str:
    """Compile the C oracle next to its source."""
    if force or not os.path.exists(_LIB):
        compile_source(_SRC, _LIB)
    return _LIB


_lib = None


def load(path: str):
    """Load an oracle shared object and declare its C signatures."""
    L = ctypes.CDLL(path)
    L.orc_bf16_to_f64.restype = ctypes.c_double
    L.orc_bf16_to_f64.argtypes = [ctypes.c_uint16]
    L.orc_f64_to_bf16.restype = ctypes.c_uint16
    L.orc_f64_to_bf16.argtypes = [ctypes.c_double]
    L.orc_f32_to_bf16.restype = ctypes.c_uint16
    L.orc_f32_to_bf16.argtypes = [ctypes.c_float]
    L.orc_partial_rows.restype = ctypes.c_int
    L.orc_partial_rows.argtypes = [_p, _i64, _p, _i64, _i64, _i64, _i64, _p, _i64, _p, _p]
    L.orc_reduce_chunk_rmsnorm.restype = ctypes.c_int
    L.orc_reduce_chunk_rmsnorm.argtypes = [_p, ctypes.c_int, _i64, _i64, _i64, _p, _p,
                                           ctypes.c_float, _p, _p, _p, _p]
    L.orc_w8a8_rows.restype = ctypes.c_int
    L.orc_w8a8_rows.argtypes = [_p, _i64, _p, _p, _i64, _p, _i64, _i64, _i64, _p, _i64, _p, _p]
    L.orc_sum_partials.restype = ctypes.c_int
    L.orc_sum_partials.argtypes = [_p, ctypes.c_int, _i64, _i64, _i64, _p, _p]
    L.orc_reduce_slice_sumsq.restype = ctypes.c_int
    L.orc_reduce_slice_sumsq.argtypes = [_p, ctypes.c_int, _i64, _i64, _i64, _p, _p, _p, _p]
    L.orc_rmsnorm_slice_apply.restype = ctypes.c_int
    L.orc_rmsnorm_slice_apply.argtypes = [_p, _p, ctypes.c_int, _i64, _i64, _i64, _p, ctypes.c_float, _p,
                                          _i64, _p]
    L.orc_quant_per_token.restype = ctypes.c_int
    L.orc_quant_per_token.argtypes = [_p, _i64, _i64, _i64, _p, _i64, _p]
    L.orc_num_threads.restype = ctypes.c_int
    L.orc_set_num_threads.argtypes = [ctypes.c_int]
    L.orc_shard_rows.argtypes = [_p, _i64, _i64, _i64, ctypes.c_int, ctypes.c_int, _p]
    L.orc_shard_rows.restype = ctypes.c_int
    L.orc_gather_rows.argtypes = [_p, ctypes.c_int, _i64, _i64, _i64, _i64, _p]
    L.orc_gather_rows.restype = ctypes.c_int
    return L


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=True)
        _lib = load(_LIB)
    return _lib


def _ptr(a: np.ndarray | None):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _check2d(a: np.ndarray, dtype, name: str):
    if a.dtype != dtype or a.ndim != 2:
        raise TypeError(f"{name}: expected 2-D {np.dtype(dtype)}, got {a.dtype} {a.shape}")
    if a.strides[1] != a.itemsize:
        raise ValueError(f"{name}: rows must be contiguous")
    return a.strides[0] // a.itemsize


def num_threads() -> int:
    return int(lib().orc_num_threads())


def set_num_threads(t: int) -> None:
    lib().orc_set_num_threads(int(t))


def f64_to_bf16(v: float) -> int:
    return int(lib().orc_f64_to_bf16(float(v)))


def bf16_to_f64(b: int) -> float:
    return float(lib().orc_bf16_to_f64(int(b)))


def f64_to_bf16_array(a: np.ndarray) -> np.ndarray:
    f = lib().orc_f64_to_bf16
    flat = np.asarray(a, dtype=np.float64).ravel()
    return np.array([f(float(v)) for v in flat], dtype=np.uint16).reshape(np.shape(a))


def bf16_to_f64_array(b: np.ndarray) -> np.ndarray:
    """Exact decode of bf16 bit patterns (a float32 with zero low half)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def partial_rows(x: np.ndarray, w: np.ndarray, m: int, rows=None, tp: int = 1,
                 want_f64: bool = False):
    """Rank partial rows: bf16(x[r] . w[j]) for r < m, zero for pad rows.

    x: [>=m, k] uint16 (bf16 bits) -- only rows < m are read;  w: [n, k] uint16.
    rows: output row indices into the padded [M_pad, n] output (default: all
    M_pad = ceil(m/tp)*tp rows).  Returns uint16 [len(rows), n] (and the fp64
    values when want_f64).
    """
    ldx = _check2d(x, np.uint16, "x")
    ldw = _check2d(w, np.uint16, "w")
    k = x.shape[1]
    if w.shape[1] != k:
        raise ValueError("x and w disagree on k")
    n = w.shape[0]
    m_pad = -(-m // tp) * tp
    if rows is None:
        rows = np.arange(m_pad, dtype=np.int64)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    if rows.size and (rows.min() < 0 or rows.max() >= m_pad):
        raise ValueError("row index outside the padded output")
    live = rows[rows < m]
    if live.size and int(live.max()) >= x.shape[0]:
        raise ValueError("x has fewer rows than the requested output rows need")
    out = np.empty((rows.size, n), dtype=np.uint16)
    f64 = np.empty((rows.size, n), dtype=np.float64) if want_f64 else None
    rc = lib().orc_partial_rows(_ptr(x), ldx, _ptr(w), ldw, m, n, k, _ptr(rows), rows.size,
                                _ptr(out), _ptr(f64))
    if rc != 0:
        raise RuntimeError(f"orc_partial_rows failed: {rc}")
    return (out, f64) if want_f64 else out


def reduce_chunk_rmsnorm(partials, residual: np.ndarray, gamma: np.ndarray, eps: float,
                         want_f64: bool = False):
    """Sum of TP bf16 partial chunks + residual, then RMSNorm.

    partials: list of [m_chunk, n] uint16 arrays (same row stride);
    residual: [m_chunk, n] uint16; gamma: [n] uint16.
    Returns (y, residual_out) as uint16, plus (h_f64, y_f64) when want_f64.
    """
    tp = len(partials)
    if tp < 1:
        raise ValueError("need at least one partial")
    ldp = _check2d(partials[0], np.uint16, "partials[0]")
    m_chunk, n = partials[0].shape
    for i, p in enumerate(partials):
        if _check2d(p, np.uint16, f"partials[{i}]") != ldp or p.shape != (m_chunk, n):
            raise ValueError("partials must share shape and row stride")
    residual = np.ascontiguousarray(residual, dtype=np.uint16)
    gamma = np.ascontiguousarray(gamma, dtype=np.uint16)
    if residual.shape != (m_chunk, n) or gamma.shape != (n,):
        raise ValueError("residual/gamma shape mismatch")
    ptrs = (ctypes.c_void_p * tp)(*[p.ctypes.data for p in partials])
    y = np.empty((m_chunk, n), dtype=np.uint16)
    ro = np.empty((m_chunk, n), dtype=np.uint16)
    hf = np.empty((m_chunk, n), dtype=np.float64) if want_f64 else None
    yf = np.empty((m_chunk, n), dtype=np.float64) if want_f64 else None
    rc = lib().orc_reduce_chunk_rmsnorm(ctypes.cast(ptrs, ctypes.c_void_p), tp, ldp, m_chunk, n,
                                        _ptr(residual), _ptr(gamma), float(eps),
                                        _ptr(y), _ptr(ro), _ptr(hf), _ptr(yf))
    if rc != 0:
        raise RuntimeError(f"orc_reduce_chunk_rmsnorm failed: {rc}")
    return (y, ro, hf, yf) if want_f64 else (y, ro)


def w8a8_rows(xq: np.ndarray, sx: np.ndarray, wq: np.ndarray, sw: np.ndarray, m: int,
              rows=None, tp: int = 1):
    """int8 x int8 -> exact int32 accumulators and the bf16 dequantised output.

    Returns (out uint16 [len(rows), n], acc int32 [len(rows), n]).
    """
    ldx = _check2d(xq, np.int8, "xq")
    ldw = _check2d(wq, np.int8, "wq")
    k = xq.shape[1]
    if wq.shape[1] != k:
        raise ValueError("xq and wq disagree on k")
    n = wq.shape[0]
    sx = np.ascontiguousarray(sx, dtype=np.float32)
    sw = np.ascontiguousarray(sw, dtype=np.float32)
    if sw.shape != (n,) or sx.shape[0] < min(m, xq.shape[0]):
        raise ValueError("scale shape mismatch")
    m_pad = -(-m // tp) * tp
    if rows is None:
        rows = np.arange(m_pad, dtype=np.int64)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    if rows.size and (rows.min() < 0 or rows.max() >= m_pad):
        raise ValueError("row index outside the padded output")
    out = np.empty((rows.size, n), dtype=np.uint16)
    acc = np.empty((rows.size, n), dtype=np.int32)
    rc = lib().orc_w8a8_rows(_ptr(xq), ldx, _ptr(sx), _ptr(wq), ldw, _ptr(sw), m, n, k,
                             _ptr(rows), rows.size, _ptr(out), _ptr(acc))
    if rc == 2:
        raise OverflowError("int32 accumulator overflow")
    if rc != 0:
        raise RuntimeError(f"orc_w8a8_rows failed: {rc}")
    return out, acc


def quant_per_token(x: np.ndarray, rows: int | None = None):
    """Per-token dynamic int8 quantisation of bf16 rows (reading R6).

    x: uint16 bf16 bits [m, k].  Returns (xq int8 [r, k], sx float32 [r]) for the
    first ``rows`` rows (default all).
    """
    ldx = _check2d(x, np.uint16, "x")
    m = x.shape[0] if rows is None else min(int(rows), x.shape[0])
    k = x.shape[1]
    xq = np.empty((m, k), dtype=np.int8)
    sx = np.empty((m,), dtype=np.float32)
    rc = lib().orc_quant_per_token(_ptr(x), ldx, m, k, _ptr(xq), k, _ptr(sx))
    if rc != 0:
        raise RuntimeError(f"orc_quant_per_token failed: {rc}")
    return xq, sx


def _ptr_array(arrays):
    arr = (ctypes.c_void_p * len(arrays))(*[a.ctypes.data for a in arrays])
    return arr


def sum_partials(partials, want_f64: bool = False):
    """bf16(sum of the tp bf16 partials), all rows ([MMAR] all-reduce form)."""
    parts = [np.ascontiguousarray(p, dtype=np.uint16) for p in partials]
    m, n = parts[0].shape
    if any(p.shape != (m, n) for p in parts):
        raise ValueError("partials disagree in shape")
    out = np.empty((m, n), dtype=np.uint16)
    of = np.empty((m, n), dtype=np.float64) if want_f64 else None
    arr = _ptr_array(parts)
    rc = lib().orc_sum_partials(ctypes.cast(arr, _p), len(parts), n, m, n, _ptr(out), _ptr(of))
    if rc != 0:
        raise RuntimeError(f"orc_sum_partials failed: {rc}")
    return (out, of) if want_f64 else out


def reduce_slice_sumsq(partials, residual, c0: int, n_slice: int):
    """Step 1 of the hidden-split epilogue for columns [c0, c0 + n_slice) of full [m, n] arrays.

    Returns (residual_out slice uint16 [m, n_slice], h float64 [m, n_slice], sumsq float64 [m]).
    """
    parts = [np.ascontiguousarray(p, dtype=np.uint16) for p in partials]
    residual = np.ascontiguousarray(residual, dtype=np.uint16)
    m, n = residual.shape
    if any(p.shape != (m, n) for p in parts) or c0 < 0 or c0 + n_slice > n:
        raise ValueError("bad slice or shapes")
    ro = np.zeros((m, n), dtype=np.uint16)
    h = np.empty((m, n_slice), dtype=np.float64)
    ss = np.empty((m,), dtype=np.float64)
    ptrs = (ctypes.c_void_p * len(parts))(*[p.ctypes.data + 2 * c0 for p in parts])
    rc = lib().orc_reduce_slice_sumsq(ctypes.cast(ptrs, _p), len(parts), n, m, n_slice,
                                      ctypes.c_void_p(residual.ctypes.data + 2 * c0),
                                      ctypes.c_void_p(ro.ctypes.data + 2 * c0), _ptr(h), _ptr(ss))
    if rc != 0:
        raise RuntimeError(f"orc_reduce_slice_sumsq failed: {rc}")
    return np.ascontiguousarray(ro[:, c0:c0 + n_slice]), h, ss


def rmsnorm_slice_apply(h, sumsq_parts, n_total: int, gamma_slice, eps: float, want_f64: bool = False):
    """Step 2: y = bf16(gamma * h / sqrt(sum_r sumsq_r / n_total + eps)) for one slice."""
    h = np.ascontiguousarray(h, dtype=np.float64)
    m, ns = h.shape
    parts = [np.ascontiguousarray(s, dtype=np.float64) for s in sumsq_parts]
    gamma_slice = np.ascontiguousarray(gamma_slice, dtype=np.uint16)
    if any(p.shape != (m,) for p in parts) or gamma_slice.shape != (ns,):
        raise ValueError("shape mismatch")
    y = np.empty((m, ns), dtype=np.uint16)
    yf = np.empty((m, ns), dtype=np.float64) if want_f64 else None
    arr = _ptr_array(parts)
    rc = lib().orc_rmsnorm_slice_apply(_ptr(h), ctypes.cast(arr, _p), len(parts), m, ns, n_total,
                                       _ptr(gamma_slice), ctypes.c_float(eps), _ptr(y), ns, _ptr(yf))
    if rc != 0:
        raise RuntimeError(f"orc_rmsnorm_slice_apply failed: {rc}")
    return (y, yf) if want_f64 else y


def shard_rows(x: np.ndarray, tp: int, rank: int) -> np.ndarray:
    """Rank `rank`'s token chunk of the zero-padded rows of x ([FC1] pad/shard helpers)."""
    x = np.ascontiguousarray(x, dtype=np.uint16)
    m, n = x.shape
    mc = -(-m // tp)
    out = np.empty((mc, n), dtype=np.uint16)
    rc = lib().orc_shard_rows(_ptr(x), n, m, n, tp, rank, _ptr(out))
    if rc != 0:
        raise RuntimeError(f"orc_shard_rows failed: {rc}")
    return out


def gather_rows(chunks, m: int) -> np.ndarray:
    """The tp chunks in rank order, cut back to the first m rows ([FC1] gather + unpad)."""
    parts = [np.ascontiguousarray(c, dtype=np.uint16) for c in chunks]
    mc, n = parts[0].shape
    if any(p.shape != (mc, n) for p in parts):
        raise ValueError("chunks disagree in shape")
    out = np.empty((m, n), dtype=np.uint16)
    arr = _ptr_array(parts)
    rc = lib().orc_gather_rows(ctypes.cast(arr, _p), len(parts), mc, n, m, n, _ptr(out))
    if rc != 0:
        raise RuntimeError(f"orc_gather_rows failed: {rc}")
    return out
