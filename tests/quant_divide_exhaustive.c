/*
 * quant_divide_exhaustive.c -- exhaustive host check of the per-token
 * quantiser's division (test infrastructure; built and run by
 * tests/test_quant_divide_exhaustive.py).
 *
 * The quantiser (w8a8_dynamic step of xLLM pull request #1890, "feat: add
 * FlashComm1 and MMRS fusion support for Qwen3.5 NPU", review thread) defines
 * each code as rint(RN(x / s)) clamped to [-127, 127], with s = RN(amax / 127)
 * in fp32 and rint half-to-even.  For rows with amax >= 2^-60 the kernel does
 * not divide per element: it takes y = RN(1 / s) once per row and forms
 *     q0 = RN(x * y),  r = fma(-q0, s, x),  t = fma(r, y, q0)
 * (Markstein's correction step, P. Markstein, IBM J. Res. Dev. 34(1), 1990),
 * and rounds t.  This program replays exactly that fp32 arithmetic on the CPU
 * for every positive finite bf16 amax and every bf16 x with |x| <= amax (both
 * signs), and compares the code with the one from the correctly rounded
 * quotient.  Rows with amax < 2^-60 divide element by element in the kernel;
 * for them (and for all rows) it checks that the clamp never binds, i.e.
 * |rint(RN(x / s))| <= 127.
 *
 * Build: gcc -O2 -ffp-contract=off -fopenmp (no contraction: x * y must be a
 * separate rounding, as in the kernel; fmaf is the single-rounding FMA).
 *
 * Usage: quant_divide_exhaustive [mode]
 *   mode 0: the kernel's corrected quotient (expected: 0 code mismatches)
 *   mode 1: a planted mistake, the uncorrected q0 (expected: mismatches), so
 *           that the harness is shown to detect a wrong division.
 * Prints one line: key=value pairs.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static float bf16_value(uint32_t bits) {
    const uint32_t u = bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

static int clamp_code(float t) {
    const float q = fminf(fmaxf(rintf(t), -127.f), 127.f);
    return (int)q;
}

int main(int argc, char **argv) {
    const int mode = argc > 1 ? atoi(argv[1]) : 0;
    long long pairs_fast = 0, pairs_slow = 0, code_mismatch = 0, quot_mismatch = 0, quot_mismatch_big = 0;
    long long clamp_binds = 0;
    const uint32_t inf_bits = 0x7F80u;
#pragma omp parallel for schedule(dynamic, 64) reduction(+ : pairs_fast, pairs_slow, code_mismatch, quot_mismatch, \
                                                             quot_mismatch_big, clamp_binds)
    for (uint32_t ab = 1; ab < inf_bits; ++ab) {
        const float amax = bf16_value(ab);
        const float s = amax / 127.f;
        const int fast = amax >= 0x1p-60f;
        const float y = 1.f / s;
        for (uint32_t xb = 0; xb <= ab; ++xb) {
            for (int sign = 0; sign < 2; ++sign) {
                if (sign && xb == 0) continue;
                const float x = sign ? -bf16_value(xb) : bf16_value(xb);
                const float exact = x / s; /* correctly rounded quotient */
                if (fabsf(rintf(exact)) > 127.f) ++clamp_binds;
                if (!fast) {
                    ++pairs_slow;
                    continue;
                }
                ++pairs_fast;
                const float q0 = x * y;
                float t;
                if (mode == 1) {
                    t = q0;
                } else {
                    const float r = fmaf(-q0, s, x);
                    t = fmaf(r, y, q0);
                }
                if (clamp_code(t) != clamp_code(exact)) ++code_mismatch;
                if (t != exact) {
                    ++quot_mismatch;
                    if (fabsf(exact) >= 0.25f) ++quot_mismatch_big;
                }
            }
        }
    }
    printf("mode=%d pairs_fast=%lld pairs_slow=%lld code_mismatch=%lld quot_mismatch=%lld "
           "quot_mismatch_ge_quarter=%lld clamp_binds=%lld\n",
           mode, pairs_fast, pairs_slow, code_mismatch, quot_mismatch, quot_mismatch_big, clamp_binds);
    return 0;
}
