"""CPU-only: pin the oracle to facts outside itself, and show the pins bite.

The second half plants plausible mistakes in copies of the oracle's C source
(a dropped term, a wrong sign, a transposed operand, a wrong mean, eps outside
the root, ties rounded away from zero, a missing subnormal clamp, a dropped
residual, a reordered dequantisation, a quantiser that rounds ties away from
zero, truncates, divides by 128, drops the absolute value or the last column,
or gives a zero row scale 1; an all-reduce sum that drops a shard; a
hidden-split epilogue that sums h instead of h^2, averages over the slice or
drops a rank; token blocks at the wrong stride, pad rows that repeat the last
row, blocks gathered in reverse rank order), compiles each copy with gcc and checks that at
least one pin fails for every one of them.
"""
import os
import shutil

import numpy as np
import pytest

import oracle
import oracle_checks as oc

pytestmark = []


@pytest.mark.parametrize("check", oc.ALL_CHECKS, ids=lambda f: f.__name__)
def test_pin(orc, check):
    check(orc)


def check_w8a8_dequant_many(orc):
    """Many outputs so that an fp32 operation-order slip shows in the bf16 result."""
    import torch
    rng = np.random.default_rng(81)
    m, k, n = 512, 32, 1024
    xq = rng.integers(-127, 128, (m, k), dtype=np.int8)
    wq = rng.integers(-127, 128, (n, k), dtype=np.int8)
    sx = rng.uniform(1e-3, 2e-2, m).astype(np.float32)
    sw = rng.uniform(1e-3, 1e-2, n).astype(np.float32)
    out, acc = orc.w8a8_rows(xq, sx, wq, sw, m)
    deq = (acc.astype(np.float32) * sx[:, None]) * sw[None, :]
    ref = torch.from_numpy(deq).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(out, ref)


def test_w8a8_dequant_many(orc):
    check_w8a8_dequant_many(orc)


MUTANTS = [
    ("dropped_last_k_term",
     "for (int64_t kk = 0; kk < k; ++kk)\n                    s += orc_bf16",
     "for (int64_t kk = 0; kk < k - 1; ++kk)\n                    s += orc_bf16"),
    ("partial_sum_sign",
     "acc += orc_bf16_to_f64(partials[s][i * ldp + j]);",
     "acc += (s == 1 ? -1.0 : 1.0) * orc_bf16_to_f64(partials[s][i * ldp + j]);"),
    ("transposed_weight",
     "s += orc_bf16_to_f64(xr[kk]) * orc_bf16_to_f64(wr[kk]);",
     "s += orc_bf16_to_f64(xr[kk]) * orc_bf16_to_f64(w[(kk * n + j) % (n * k)]);"),
    ("mean_over_n_minus_1", "double ms = sumsq / (double)n;", "double ms = sumsq / (double)(n > 1 ? n - 1 : 1);"),
    ("eps_outside_sqrt", "double denom = sqrt(ms + deps);", "double denom = sqrt(ms) + deps;"),
    ("ties_away_from_zero", "double r = nearbyint(q);", "double r = floor(q + 0.5);"),
    ("no_subnormal_clamp", "if (binade < -126) binade = -126;", ""),
    ("residual_dropped_from_new_residual",
     "if (residual_out) residual_out[i * n + j] = orc_f64_to_bf16(h);",
     "if (residual_out) residual_out[i * n + j] = orc_f64_to_bf16(acc);"),
    ("dequant_scales_multiplied_first",
     "volatile float v = u * sw[j];",
     "volatile float v = t * (((r < m) ? sx[r] : 0.0f) * sw[j]);"),
    ("sum_partials_drops_shard_0",
     "for (int s = 0; s < tp; ++s)\n                acc += orc_bf16_to_f64(partials[s][i * ldp + j]);\n            if (out) out[i * n + j]",
     "for (int s = 1; s < tp; ++s)\n                acc += orc_bf16_to_f64(partials[s][i * ldp + j]);\n            if (out) out[i * n + j]"),
    ("slice_sum_of_h_not_squares", "            ss += h * h;\n        }\n        sumsq[i] = ss;",
     "            ss += h;\n        }\n        sumsq[i] = ss;"),
    ("slice_mean_over_slice_width", "const double denom = sqrt(ss / (double)n_total + deps);",
     "const double denom = sqrt(ss / (double)n_slice + deps);"),
    ("slice_drops_last_rank", "for (int r = 0; r < tp; ++r) ss += sumsq_parts[r][i];",
     "for (int r = 0; r + 1 < tp; ++r) ss += sumsq_parts[r][i];"),
    ("quant_ties_away_from_zero", "float v = nearbyintf(t);", "float v = roundf(t);"),
    ("quant_scale_over_128", "volatile float s = amax / 127.0f;", "volatile float s = amax / 128.0f;"),
    ("quant_absmax_without_abs", "float a = fabsf((float)orc_bf16_to_f64(xr[kk]));",
     "float a = (float)orc_bf16_to_f64(xr[kk]);"),
    ("quant_absmax_skips_last_column", "for (int64_t kk = 0; kk < k; ++kk) {\n            float a",
     "for (int64_t kk = 0; kk + 1 < k; ++kk) {\n            float a"),
    ("quant_zero_row_scale_one", "volatile float s = amax / 127.0f;",
     "volatile float s = amax > 0.0f ? amax / 127.0f : 1.0f;"),
    ("quant_truncates", "float v = nearbyintf(t);", "float v = truncf(t);"),
    ("shard_block_stride_m_over_tp",
     "const int64_t src = (int64_t)rank * mc + i;",
     "const int64_t src = (int64_t)rank * (m / tp) + i;"),
    ("shard_pad_rows_repeat_last_row",
     "out[i * n + j] = src < m ? x[src * ldx + j] : (uint16_t)0;",
     "out[i * n + j] = x[(src < m ? src : m - 1) * ldx + j];"),
    ("gather_blocks_in_reverse_rank_order",
     "const int64_t c = i / m_chunk, r = i % m_chunk;",
     "const int64_t c = tp - 1 - i / m_chunk, r = i % m_chunk;"),
    ("w8a8_sign_of_weight",
     "s += (int64_t)xr[kk] * (int64_t)wr[kk];",
     "s += (int64_t)xr[kk] * (int64_t)(kk == 0 ? -wr[kk] : wr[kk]);"),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_is_caught(tmp_path, monkeypatch, name, old, new):
    src = open(oracle._SRC).read()
    assert src.count(old) >= 1, f"mutation anchor for {name} not found"
    mutated = src.replace(old, new)
    path = tmp_path / f"mut_{name}.c"
    path.write_text(mutated)
    so = oracle.compile_source(str(path), str(tmp_path / f"mut_{name}.so"))
    monkeypatch.setattr(oracle, "_lib", oracle.load(so))
    failed = []
    for check in oc.ALL_CHECKS + [check_w8a8_dequant_many]:
        try:
            check(oracle)
        except (AssertionError, OverflowError, RuntimeError, ValueError):
            failed.append(check.__name__)
    assert failed, f"no pin caught the planted mistake {name}"
