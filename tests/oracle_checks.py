"""Pins of the CPU oracle against facts fixed outside the oracle itself.

Each ``check_*`` function raises AssertionError on a mismatch.  They pin the
oracle to: exact rational arithmetic (``fractions.Fraction``), 60-digit
``decimal`` square roots, numpy's fp64 / int64 matrix products, numpy float32
arithmetic, torch's fp32 -> bf16 conversion, closed forms (one-hot rows, small
integers, power-of-two scaling) and the hand-worked golden file.  The same
checks are run against deliberately broken copies of the oracle (see
test_oracle_pins.py) to show each plausible mistake is caught.
"""
from __future__ import annotations

import decimal
import json
import os
from fractions import Fraction

import numpy as np

from row_matmul_reduce_amd import synth

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "hand_worked.json")


# ------------------------------------------------------------ exact bf16 helpers
def bf16_value(b: int) -> Fraction:
    """Exact value of a finite bf16 bit pattern."""
    b = int(b) & 0xFFFF
    sign = -1 if b & 0x8000 else 1
    e = (b >> 7) & 0xFF
    f = b & 0x7F
    if e == 0xFF:
        raise ValueError("not finite")
    if e == 0:
        return sign * Fraction(f, 1 << 7) * Fraction(1, 1 << 126)
    return sign * (1 + Fraction(f, 1 << 7)) * (Fraction(2) ** (e - 127))


def exact_bf16(v: Fraction) -> int:
    """Nearest bf16 (ties to even) of an exact rational, by search over neighbours."""
    if v == 0:
        return 0
    neg = v < 0
    a = -v if neg else v
    # bracket: walk the positive bf16 patterns (monotone in value) by bisection
    lo, hi = 0, 0x7F7F                      # 0 .. largest finite
    if a >= bf16_value(0x7F7F):
        top = bf16_value(0x7F7F)
        half_ulp = (Fraction(2) ** 128 - top) / 2
        res = 0x7F80 if a >= top + half_ulp else 0x7F7F
        return res | (0x8000 if neg else 0)
    while hi - lo > 1:
        mid = (lo + hi) // 2
        if bf16_value(mid) <= a:
            lo = mid
        else:
            hi = mid
    dl, dh = a - bf16_value(lo), bf16_value(hi) - a
    if dl < dh:
        r = lo
    elif dh < dl:
        r = hi
    else:
        r = lo if lo % 2 == 0 else hi
    return r | (0x8000 if neg else 0)


def frac_of_bits(b) -> np.ndarray:
    return np.vectorize(bf16_value, otypes=[object])(b)


def _bits(vals) -> np.ndarray:
    return synth.bf16_bits(np.asarray(vals, dtype=np.float32))


# ------------------------------------------------------------------------ codec
def check_codec(orc):
    rng = np.random.default_rng(1234)
    cases = [1.0, -1.0, 1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8), 3.0e38, 3.4e38, -3.4e38,
             2.0 ** -126, 2.0 ** -133, 1.5 * 2.0 ** -133, 2.5 * 2.0 ** -133, 2.0 ** -134,
             0.1, 1e-3, 123456.789, 65535.0, 2.0 ** 127 * (2 - 2 ** -8)]
    mags = rng.uniform(-140, 130, 400)
    cases += list(np.sign(rng.standard_normal(400)) * 2.0 ** mags)
    # exact ties between adjacent bf16 values
    for b in rng.integers(1, 0x7F7F, 100):
        mid = (bf16_value(b) + bf16_value(b + 1)) / 2
        cases.append(float(mid))  # a tie is exactly representable in fp64
    for v in cases:
        want = exact_bf16(Fraction(v))
        got = orc.f64_to_bf16(v)
        assert got == want, f"f64_to_bf16({v!r}) = {got:#06x}, exact nearest-even {want:#06x}"
    # decode is exact
    for b in rng.integers(0, 0x7F7F, 200):
        assert Fraction(orc.bf16_to_f64(int(b))) == bf16_value(int(b))


# --------------------------------------------------------------------- partials
def check_partial_bruteforce(orc):
    """Tiny shapes: exact rational dot products, rounded by exact nearest-even."""
    rng = np.random.default_rng(7)
    for (m, k_full, n, tp) in [(4, 16, 8, 1), (3, 16, 5, 2), (5, 8, 3, 4), (1, 12, 2, 2), (4, 4, 7, 4)]:
        x = _bits(rng.standard_normal((m, k_full)) * 0.7)
        w = _bits(rng.standard_normal((n, k_full)) * 1.3)
        ks = k_full // tp
        xf, wf = frac_of_bits(x), frac_of_bits(w)
        m_pad = -(-m // tp) * tp
        for s in range(tp):
            xs = np.ascontiguousarray(x[:, s * ks:(s + 1) * ks])
            ws = np.ascontiguousarray(w[:, s * ks:(s + 1) * ks])
            out, f64 = orc.partial_rows(xs, ws, m, tp=tp, want_f64=True)
            assert out.shape == (m_pad, n)
            for r in range(m_pad):
                for j in range(n):
                    if r < m:
                        exact = sum(xf[r, s * ks + t] * wf[j, s * ks + t] for t in range(ks))
                    else:
                        exact = Fraction(0)
                    assert abs(Fraction(f64[r, j]) - exact) <= abs(exact) * Fraction(1, 10 ** 15), \
                        (m, k_full, n, tp, s, r, j)
                    assert int(out[r, j]) == exact_bf16(exact), (m, k_full, n, tp, s, r, j)


def check_partial_sum_is_unsharded_gemm(orc):
    """Sum over ranks of the unrounded partials = numpy's fp64 X.W^T over K_full."""
    rng = np.random.default_rng(11)
    for (m, k_full, n, tp) in [(37, 96, 29, 4), (20, 64, 40, 2), (9, 48, 17, 1), (16, 256, 24, 8)]:
        x = _bits(rng.standard_normal((m, k_full)))
        w = _bits(rng.standard_normal((n, k_full)) * 0.05)
        ref = synth.bf16_decode(x).astype(np.float64) @ synth.bf16_decode(w).astype(np.float64).T
        ks = k_full // tp
        tot = np.zeros((m, n))
        for s in range(tp):
            xs = np.ascontiguousarray(x[:, s * ks:(s + 1) * ks])
            ws = np.ascontiguousarray(w[:, s * ks:(s + 1) * ks])
            _, f64 = orc.partial_rows(xs, ws, m, tp=1, want_f64=True)
            tot += f64
        scale = np.abs(synth.bf16_decode(x)).astype(np.float64) @ np.abs(synth.bf16_decode(w)).astype(np.float64).T
        assert np.all(np.abs(tot - ref) <= 1e-12 * scale + 1e-300), (m, k_full, n, tp)


def check_partial_one_hot(orc):
    """x rows one-hot at column c_r: partial row r equals column c_r of w, bit for bit."""
    rng = np.random.default_rng(3)
    m, k, n = 6, 40, 13
    cols = rng.integers(0, k, m)
    xf = np.zeros((m, k), np.float32)
    xf[np.arange(m), cols] = 1.0
    x = _bits(xf)
    w = _bits(rng.standard_normal((n, k)))
    out = orc.partial_rows(x, w, m)
    for r in range(m):
        assert np.array_equal(out[r], w[:, cols[r]]), r


def check_partial_small_integers(orc):
    """Integer inputs: the exact integer product, which bf16 holds when below 2^8."""
    rng = np.random.default_rng(5)
    m, k, n = 7, 24, 9
    xi = rng.integers(-2, 3, (m, k))
    wi = rng.integers(-2, 3, (n, k))
    out = orc.partial_rows(_bits(xi), _bits(wi), m)
    want = xi @ wi.T
    assert np.max(np.abs(want)) < 256
    assert np.array_equal(synth.bf16_decode(out).astype(np.int64), want)


def check_partial_padding_and_chunks(orc):
    """m not divisible by tp: rows m..m_pad-1 are zero; chunk c = rows [c*mc,(c+1)*mc)."""
    rng = np.random.default_rng(9)
    m, k, n, tp = 5, 16, 6, 2
    x = _bits(rng.standard_normal((m, k)))
    w = _bits(rng.standard_normal((n, k)))
    full = orc.partial_rows(x, w, m, tp=tp)
    assert full.shape == (6, n)
    assert np.all(full[5] == 0)
    mc = 3
    for c in range(tp):
        rows = np.arange(c * mc, (c + 1) * mc)
        assert np.array_equal(orc.partial_rows(x, w, m, rows=rows, tp=tp), full[c * mc:(c + 1) * mc])
    # rows drawn out of order come back in the requested order
    perm = np.array([4, 0, 5, 2])
    assert np.array_equal(orc.partial_rows(x, w, m, rows=perm, tp=tp), full[perm])


# ----------------------------------------------------------------------- reduce
def _dec(fr: Fraction) -> decimal.Decimal:
    return decimal.Decimal(fr.numerator) / decimal.Decimal(fr.denominator)


def check_reduce_bruteforce(orc):
    """60-digit decimal evaluation of sum, residual add and RMSNorm."""
    rng = np.random.default_rng(21)
    with decimal.localcontext() as ctx:
        ctx.prec = 60
        for (tp, mc, n, eps) in [(1, 2, 5, 1e-6), (2, 3, 8, 1e-6), (4, 2, 7, 0.0), (8, 1, 16, 1e-2)]:
            parts = [_bits(rng.standard_normal((mc, n)) * 1.1) for _ in range(tp)]
            res = _bits(rng.standard_normal((mc, n)))
            gam = _bits(rng.uniform(0.5, 1.5, n))
            y, ro, hf, yf = orc.reduce_chunk_rmsnorm(parts, res, gam, eps, want_f64=True)
            pf = [frac_of_bits(p) for p in parts]
            rf, gf = frac_of_bits(res), frac_of_bits(gam)
            epsf = Fraction(float(np.float32(eps)))
            for i in range(mc):
                h = [sum(p[i, j] for p in pf) + rf[i, j] for j in range(n)]
                ms = sum(v * v for v in h) / n
                denom = _dec(ms + epsf).sqrt()
                for j in range(n):
                    assert hf[i, j] == float(h[j])          # h is exact in fp64 at these sizes
                    assert int(ro[i, j]) == exact_bf16(h[j])
                    yd = _dec(gf[j] * h[j]) / denom
                    assert abs(decimal.Decimal(yf[i, j]) - yd) <= abs(yd) * decimal.Decimal("1e-14")
                    yfr = Fraction(yd)
                    want = exact_bf16(yfr)
                    if int(y[i, j]) != want:
                        # only acceptable where the exact value sits on a rounding boundary
                        mid = (bf16_value(int(y[i, j])) + bf16_value(want)) / 2
                        assert abs(yfr - mid) <= abs(yfr) * Fraction(1, 10 ** 13), (tp, i, j)


def check_rms_invariant(orc):
    """Per row: RMS(y/gamma) = sqrt(ms/(ms+eps)) in fp64; rounded output within 2^-8."""
    rng = np.random.default_rng(31)
    tp, mc, n, eps = 4, 6, 96, 1e-3
    parts = [_bits(rng.standard_normal((mc, n)) * 0.3) for _ in range(tp)]
    res = _bits(rng.standard_normal((mc, n)) * 0.2)
    gam = _bits(rng.uniform(0.5, 1.5, n))
    y, ro, hf, yf = orc.reduce_chunk_rmsnorm(parts, res, gam, eps, want_f64=True)
    g = synth.bf16_decode(gam).astype(np.float64)
    ms = np.mean(hf * hf, axis=1)
    want = np.sqrt(ms / (ms + float(np.float32(eps))))
    got = np.sqrt(np.mean((yf / g) ** 2, axis=1))
    assert np.allclose(got, want, rtol=1e-12, atol=0)
    got_r = np.sqrt(np.mean((synth.bf16_decode(y).astype(np.float64) / g) ** 2, axis=1))
    assert np.all(np.abs(got_r - want) <= 2.0 ** -8 * want)


def check_unit_rms_and_scale_invariance(orc):
    rng = np.random.default_rng(41)
    tp, mc, n = 2, 4, 64
    parts = [_bits(rng.standard_normal((mc, n))) for _ in range(tp)]
    res = _bits(rng.standard_normal((mc, n)))
    ones = _bits(np.ones(n))
    y, ro, hf, yf = orc.reduce_chunk_rmsnorm(parts, res, ones, 0.0, want_f64=True)
    assert np.allclose(np.sqrt(np.mean(yf ** 2, axis=1)), 1.0, rtol=1e-13, atol=0)
    # scaling every input by 4 (exact in bf16) leaves y unchanged when eps = 0
    x4 = lambda b: _bits(synth.bf16_decode(b) * np.float32(4.0))
    y4, ro4 = orc.reduce_chunk_rmsnorm([x4(p) for p in parts], x4(res), ones, 0.0)
    assert np.array_equal(y4, y)
    assert np.array_equal(synth.bf16_decode(ro4), synth.bf16_decode(ro) * np.float32(4.0))


def check_zero_row_and_tp1(orc):
    rng = np.random.default_rng(51)
    mc, n = 3, 32
    p = _bits(rng.standard_normal((mc, n)))
    p[1] = 0
    res = _bits(rng.standard_normal((mc, n)))
    res[1] = 0
    gam = _bits(rng.uniform(0.5, 1.5, n))
    y, ro, hf, yf = orc.reduce_chunk_rmsnorm([p], res, gam, 1e-6, want_f64=True)
    assert np.all(synth.bf16_decode(y[1]) == 0) and np.all(synth.bf16_decode(ro[1]) == 0)
    # TP = 1: h is the partial plus the residual
    want_h = synth.bf16_decode(p).astype(np.float64) + synth.bf16_decode(res).astype(np.float64)
    assert np.array_equal(hf, want_h)


def check_integer_partials_exact(orc):
    rng = np.random.default_rng(61)
    tp, mc, n = 8, 3, 40
    ints = [rng.integers(-50, 51, (mc, n)) for _ in range(tp)]
    ri = rng.integers(-50, 51, (mc, n))
    y, ro = orc.reduce_chunk_rmsnorm([_bits(a) for a in ints], _bits(ri), _bits(np.ones(n)), 1e-6)
    want = sum(ints) + ri
    assert np.max(np.abs(want)) < 256
    assert np.array_equal(synth.bf16_decode(ro).astype(np.int64), want)


# ------------------------------------------------------------------------- w8a8
def check_w8a8(orc):
    import torch
    rng = np.random.default_rng(71)
    for (m, k, n, tp) in [(9, 64, 11, 2), (16, 272, 24, 4), (5, 32, 3, 2)]:
        xq = rng.integers(-127, 128, (m, k), dtype=np.int8)
        wq = rng.integers(-127, 128, (n, k), dtype=np.int8)
        sx = rng.uniform(1e-3, 2e-2, m).astype(np.float32)
        sw = rng.uniform(1e-3, 1e-2, n).astype(np.float32)
        out, acc = orc.w8a8_rows(xq, sx, wq, sw, m, tp=tp)
        m_pad = -(-m // tp) * tp
        want = xq.astype(np.int64) @ wq.astype(np.int64).T
        assert np.array_equal(acc[:m].astype(np.int64), want)
        assert np.all(acc[m:m_pad] == 0) and np.all(out[m:m_pad] == 0)
        # sign symmetry
        _, acc_neg = orc.w8a8_rows((-xq.astype(np.int16)).astype(np.int8), sx, wq, sw, m, tp=tp)
        assert np.array_equal(acc_neg[:m].astype(np.int64), -want)
        # dequant: two fp32 multiplies in numpy, bf16 by torch's nearest-even conversion
        deq = (want.astype(np.float32) * sx[:, None]) * sw[None, :]
        assert deq.dtype == np.float32
        ref = torch.from_numpy(deq).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        assert np.array_equal(out[:m], ref)


def check_w8a8_overflow(orc):
    k = 133152                           # 127*127*k > 2^31 - 1
    xq = np.full((1, k), 127, np.int8)
    wq = np.full((1, k), 127, np.int8)
    try:
        orc.w8a8_rows(xq, np.ones(1, np.float32), wq, np.ones(1, np.float32), 1)
    except OverflowError:
        return
    raise AssertionError("int32 overflow not reported")


# ------------------------------------------------- all-reduce form, hidden split
def check_sum_partials(orc):
    """Exact rational sums; permutation invariance (a sum of at most 16 bf16 values is exact in
    fp64, so the bf16 result is unique); integer partials exact; TP=1 is the identity."""
    rng = np.random.default_rng(55)
    for tp in (1, 2, 3, 5):
        parts = [_bits(rng.standard_normal((3, 5)).astype(np.float32) * np.float32(10.0 ** rng.integers(-3, 4)))
                 for _ in range(tp)]
        out, of = orc.sum_partials(parts, want_f64=True)
        for i in range(3):
            for j in range(5):
                exact = sum(bf16_value(p[i, j]) for p in parts)
                assert Fraction(of[i, j]) == exact
                assert int(out[i, j]) == exact_bf16(exact), (tp, i, j)
        perm = orc.sum_partials(parts[::-1])
        assert np.array_equal(perm, out)
        if tp == 1:
            assert np.array_equal(out, parts[0])
    ints = [_bits(rng.integers(-50, 51, (4, 8)).astype(np.float32)) for _ in range(4)]
    want = sum(synth.bf16_decode(p).astype(np.float64) for p in ints)
    assert np.array_equal(synth.bf16_decode(orc.sum_partials(ints)).astype(np.float64), want)


def check_hidden_split_epilogue(orc):
    """Hidden-split epilogue: the column slices of all ranks reproduce the pinned token-chunk
    epilogue (residual_out bit-exact, y to fp64 rounding), the slice sums of squares are exact
    rational sums, and the partition does not matter."""
    rng = np.random.default_rng(56)
    m, n, tp = 5, 48, 3
    parts = [_bits(rng.standard_normal((m, n)).astype(np.float32)) for _ in range(tp)]
    res = _bits(rng.standard_normal((m, n)).astype(np.float32))
    gam = _bits(rng.uniform(0.5, 1.5, n).astype(np.float32))
    eps = 1e-6
    y_ref, ro_ref, h_ref, y_ref64 = orc.reduce_chunk_rmsnorm(parts, res, gam, eps, want_f64=True)
    for bounds in ([0, 16, 40, 48], [0, 8, 16, 24, 32, 40, 48], [0, 48]):
        slices = list(zip(bounds[:-1], bounds[1:]))
        step1 = [orc.reduce_slice_sumsq(parts, res, a, b - a) for a, b in slices]
        ss_parts = [st[2] for st in step1]
        ro = np.concatenate([st[0] for st in step1], axis=1)
        assert np.array_equal(ro, ro_ref), bounds
        assert np.allclose(np.sum(ss_parts, axis=0), np.sum(h_ref ** 2, axis=1), rtol=1e-13, atol=0)
        ys = [orc.rmsnorm_slice_apply(st[1], ss_parts, n, gam[a:b], eps, want_f64=True) for st, (a, b) in
              zip(step1, slices)]
        y64 = np.concatenate([yy[1] for yy in ys], axis=1)
        assert np.allclose(y64, y_ref64, rtol=1e-12, atol=0), bounds
        y = np.concatenate([yy[0] for yy in ys], axis=1)
        flips = np.flatnonzero(y != y_ref)
        assert flips.size <= 1, f"{flips.size} bf16 results differ beyond fp64 summation order"
    # exact rational sum of squares of one slice
    ro, h, ss = orc.reduce_slice_sumsq(parts, res, 8, 12)
    for i in range(m):
        exact = Fraction(0)
        for j in range(8, 20):
            hv = sum(bf16_value(p[i, j]) for p in parts) + bf16_value(res[i, j])
            assert Fraction(h[i, j - 8]) == hv
            exact += hv * hv
        assert abs(Fraction(ss[i]) - exact) <= exact * Fraction(1, 2 ** 48)


# ------------------------------------------------------- per-token quantiser
def _f32_nearest(v: Fraction) -> np.float32:
    """The float32 nearest to an exact rational (ties to even), by neighbour search."""
    f = np.float32(float(v))
    best = None
    for c in (np.nextafter(f, np.float32(-np.inf)), f, np.nextafter(f, np.float32(np.inf))):
        d = abs(Fraction(float(c)) - v)
        if best is None or d < best[0] or (d == best[0] and (int(c.view(np.uint32)) & 1) == 0):
            best = (d, c)
    return np.float32(best[1])


def _quant_rows_exact(x_bits: np.ndarray):
    """Exact-rational evaluation of the quantiser's reading, element by element."""
    codes = np.zeros(x_bits.shape, dtype=np.int64)
    scales = np.zeros(x_bits.shape[0], dtype=np.float32)
    for r in range(x_bits.shape[0]):
        vals = [bf16_value(b) for b in x_bits[r]]
        amax = max(abs(v) for v in vals)
        s = _f32_nearest(amax / 127)
        scales[r] = s
        if amax == 0:
            continue
        for j, v in enumerate(vals):
            q = _f32_nearest(v / Fraction(float(s)))
            codes[r, j] = max(-127, min(127, round(Fraction(float(q)))))   # half to even
    return codes, scales


def _quant_test_rows(rng) -> np.ndarray:
    rows = []
    for scale in [1.0, 1e-3, 3.0e4, 2.0 ** -120, 2.0 ** -130, 1.0e36]:
        z = rng.standard_normal((3, 40)).astype(np.float32) * np.float32(scale)
        rows.append(z)
    z = rng.standard_normal((2, 40)).astype(np.float32)
    z[0, 0] = 9.0                 # absmax first
    z[1, -1] = -9.0               # absmax last, negative
    rows.append(z)
    return _bits(np.concatenate(rows))


def check_quant_exact(orc):
    """Brute force: every scale is the fp32 nearest to absmax/127 and every code is
    the half-to-even integer of the fp32 nearest to x/scale (exact rationals)."""
    x = _quant_test_rows(np.random.default_rng(91))
    xq, sx = orc.quant_per_token(x)
    want_q, want_s = _quant_rows_exact(x)
    assert np.array_equal(sx.view(np.uint32), want_s.view(np.uint32))
    assert np.array_equal(xq.astype(np.int64), want_q)


def check_quant_properties(orc):
    """Closed-form facts of a symmetric per-row quantiser: the absmax element maps to
    +-127, every code is within half a step, negation and power-of-two scaling."""
    rng = np.random.default_rng(92)
    x = _bits(rng.standard_normal((64, 300)).astype(np.float32))
    xq, sx = orc.quant_per_token(x)
    xv = synth.bf16_decode(x).astype(np.float64)
    i = np.argmax(np.abs(xv), axis=1)
    assert np.array_equal(xq[np.arange(64), i].astype(np.int64), np.sign(xv[np.arange(64), i]) * 127)
    err = np.abs(xv - xq.astype(np.float64) * sx[:, None].astype(np.float64))
    assert np.all(err <= sx[:, None] * (0.5 + 1e-5))
    assert xq.min() >= -127
    xn, sn = orc.quant_per_token(x ^ np.uint16(0x8000))
    assert np.array_equal(sn, sx) and np.array_equal(xn.astype(np.int64), -xq.astype(np.int64))
    for j in (-20, 9):
        xs = _bits(xv.astype(np.float32) * np.float32(2.0 ** j))
        q2, s2 = orc.quant_per_token(xs)
        assert np.array_equal(q2, xq) and np.array_equal(s2, sx * np.float32(2.0 ** j))
    xz = x.copy()
    xz[5] = 0
    q0, s0 = orc.quant_per_token(xz)
    assert s0[5] == 0 and not q0[5].any()
    assert np.array_equal(q0[:5], xq[:5]) and np.array_equal(q0[6:], xq[6:])


# ----------------------------------------------------------------------- golden
def check_token_rows(orc):
    """[FC1] pad/shard and gather/unpad: the hand-worked blocks, then properties that hold for any
    shape -- the gathered blocks give back x exactly, the blocks past the last real row are zero,
    and with one rank the block is x itself."""
    with open(GOLDEN) as f:
        g = json.load(f)["token_rows"]
    for c in g["cases"]:
        x = _bits(c["x"])
        blocks = [orc.shard_rows(x, c["tp"], r) for r in range(c["tp"])]
        for r, b in enumerate(blocks):
            assert np.array_equal(b, _bits(c["chunks"][r])), (c["m"], c["tp"], r)
        assert np.array_equal(orc.gather_rows(blocks, c["m"]), x)
    rng = np.random.default_rng(91)
    for m, n, tp in [(1, 8, 1), (9, 16, 1), (9, 16, 2), (13, 8, 4), (29, 24, 8), (64, 8, 8), (3, 8, 8)]:
        x = rng.integers(1, 0x7F80, (m, n), dtype=np.uint16)  # nonzero finite bf16 patterns
        blocks = [orc.shard_rows(x, tp, r) for r in range(tp)]
        mc = -(-m // tp)
        assert all(b.shape == (mc, n) for b in blocks)
        assert np.array_equal(orc.gather_rows(blocks, m), x), (m, n, tp)
        stacked = np.concatenate(blocks, axis=0)
        assert np.all(stacked[m:] == 0) and np.all(stacked[:m] != 0), (m, n, tp)
        if tp == 1:
            assert np.array_equal(blocks[0], x)


def check_golden(orc):
    with open(GOLDEN) as f:
        g = json.load(f)
    b = g["bf16_partial_and_rmsnorm"]
    x, w = _bits(b["x"]), _bits(b["w"])
    m, tp, ks = b["m"], b["tp"], b["k_full"] // b["tp"]
    parts = []
    for s in range(tp):
        xs = np.ascontiguousarray(x[:, s * ks:(s + 1) * ks])
        ws = np.ascontiguousarray(w[:, s * ks:(s + 1) * ks])
        p = orc.partial_rows(xs, ws, m, tp=tp)
        assert np.array_equal(synth.bf16_decode(p), np.asarray(b[f"partial_shard{s}"], np.float32))
        parts.append(p)
    mc = -(-m // tp)
    gam = _bits(b["gamma"])
    for c in range(tp):
        chunk = [np.ascontiguousarray(p[c * mc:(c + 1) * mc]) for p in parts]
        y, ro = orc.reduce_chunk_rmsnorm(chunk, _bits(b["residual_chunks"][c]), gam, b["eps"])
        assert np.array_equal(synth.bf16_decode(y), np.asarray(b["y_chunks"][c], np.float32)), c
        assert np.array_equal(synth.bf16_decode(ro), np.asarray(b["residual_out_chunks"][c], np.float32)), c
    q = g["w8a8"]
    out, acc = orc.w8a8_rows(np.asarray(q["xq"], np.int8), np.asarray(q["sx"], np.float32),
                             np.asarray(q["wq"], np.int8), np.asarray(q["sw"], np.float32), 1)
    assert np.array_equal(acc, np.asarray(q["acc"], np.int32))
    assert np.array_equal(synth.bf16_decode(out), np.asarray(q["out"], np.float32))
    q = g["quant_per_token"]
    xq, sx = orc.quant_per_token(_bits(q["x"]))
    assert np.array_equal(xq, np.asarray(q["codes"], np.int8))
    assert np.array_equal(sx, np.asarray(q["scale"], np.float32))


ALL_CHECKS = [
    check_codec, check_partial_bruteforce, check_partial_sum_is_unsharded_gemm,
    check_partial_one_hot, check_partial_small_integers, check_partial_padding_and_chunks,
    check_reduce_bruteforce, check_rms_invariant, check_unit_rms_and_scale_invariance,
    check_zero_row_and_tp1, check_integer_partials_exact, check_w8a8, check_w8a8_overflow,
    check_sum_partials, check_hidden_split_epilogue, check_quant_exact, check_quant_properties,
    check_golden, check_token_rows,
]
