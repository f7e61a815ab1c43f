"""CPU check of the division-free quotient the INT4, FP8-row and NVFP4-row paths use.

The encoders need q = RN(d / s) bit for bit (the INT4 code is rne(q), the FP8-row code is the
E4M3 rounding of q). They compute y = RN(1 / s) once per group or row, then per element
q0 = RN(d * y), r = fma(-s, q0, d), q = fma(r, y, q0) (Markstein's correction step; P. Markstein,
IBM J. Res. Dev. 34(1), 1990). q0 can be two ulps off, which the theorem alone does not cover,
so the identity is checked here with the host's IEEE single-precision operations, on the inputs
where an ulp matters, for a sample of scale significands over each encoder's fast range: INT4
(scales 2^-100 .. 2^100) with d at and next to s times every half-integer quotient in
[0.5, 15.5] (its code boundaries, 32 float offsets around each) plus random d; FP8-row (scales
2^-90 .. 2^100) with d at and next to s times every E4M3 midpoint down to 2^-10 (8 offsets
each); NVFP4-row's block decode scale fl(e4m3 / g) for every E4M3 code and multipliers g from
2^-100 to 2^99. The device probe
(tests/probes/cvt_probe.hip) runs the same kind of sweep on the GPU's own instructions over every
significand; this test pins the arithmetic identity the encoders rely on.
"""

import os
import subprocess

import pytest

C_SRC = r"""
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>
static float bf(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t fb(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }
static float quot3(float d, float s, float y) {
    const float q0 = d * y;
    const float r = fmaf(-s, q0, d);
    return fmaf(r, y, q0);
}
/* E4M3 code (0 .. 126) -> value: subnormals m 2^-9, normals (1 + m/8) 2^(e-7) */
static float e4m3(int c) {
    const int e = c >> 3, m = c & 7;
    return e == 0 ? ldexpf((float)m, -9) : ldexpf(1.0f + (float)m / 8.0f, e - 7);
}
/* argv: stride over scale significands, mode (0: INT4 boundaries at the INT4 exponents, 1: E4M3
   midpoints at the FP8-row exponents, 2: E4M3 midpoints at scales 2^-100 and 2^-99, below the
   FP8-row fast range, 3: every E4M3 code over NVFP4-row multipliers g from 2^-100 to 2^99) */
int main(int argc, char** argv) {
    const uint32_t stride = (uint32_t)atoi(argv[1]);
    const int mode = atoi(argv[2]);
    if (mode == 3) {
        const int gexps[] = {-100, -99, -40, 0, 63, 99};
        long long n = 0, bad = 0;
        for (int ei = 0; ei < 6; ++ei)
            for (uint32_t sig = 0; sig < (1u << 23); sig += (sig < 64u || sig > (1u << 23) - 64u) ? 1u : stride) {
                const float g = ldexpf(bf(0x3F800000u | sig), gexps[ei]);
                const float y = 1.0f / g;
                for (int c = 0; c < 127; ++c) {
                    const float a = e4m3(c);
                    ++n;
                    if (fb(quot3(a, g, y)) != fb(a / g)) {
                        if (bad < 5) printf("mismatch g=%a a=%a\n", g, a);
                        ++bad;
                    }
                }
            }
        printf("%lld %lld\n", n, bad);
        return 0;
    }
    const int exps_int4[] = {-100, -99, -60, -1, 0, 1, 37, 99};
    const int exps_fp8[] = {-90, -89, -50, -1, 0, 1, 60, 99};
    const int exps_low[] = {-100, -99};
    const int* exps = mode == 0 ? exps_int4 : mode == 1 ? exps_fp8 : exps_low;
    const int n_exps = mode == 2 ? 2 : 8;
    /* quotient boundaries: INT4 the 16 half-integers 0.5 .. 15.5 with 32 float offsets each;
       FP8 the E4M3 midpoints (1 + (2i+1)/16) 2^e for e in [-9, 8], and 2^-10 (between 0 and the
       smallest subnormal), with 8 offsets each */
    const int n_j = mode == 0 ? 16 * 32 : (144 + 1) * 8;
    long long n = 0, bad = 0;
    uint32_t rng = 12345u;
    for (int ei = 0; ei < n_exps; ++ei) {
        for (uint32_t sig = 0; sig < (1u << 23); sig += (sig < 64u || sig > (1u << 23) - 64u) ? 1u : stride) {
            const float s = ldexpf(bf(0x3F800000u | sig), exps[ei]);
            const float y = 1.0f / s;
            for (int j = 0; j < n_j; ++j) {
                double h;
                int k;
                if (mode == 0) {
                    h = 0.5 + (double)(j & 15);
                    k = (j >> 4) - 16;
                } else {
                    const int u = j >> 3;
                    h = u < 144 ? ldexp(1.0 + (2.0 * (u & 7) + 1.0) / 16.0, (u >> 3) - 9) : ldexp(1.0, -10);
                    k = (j & 7) - 4;
                }
                int eh;
                frexp(h, &eh);
                eh -= 1; /* h in [2^eh, 2^(eh+1)) */
                const double m = h + (double)k * ldexp(1.0, eh - 24);
                const float d0 = (float)(m * (double)s);
                const uint32_t db = fb(d0);
                rng = rng * 1664525u + 1013904223u;
                const float dr = (float)(rng >> 8) * (1.0f / 16777216.0f) * 15.0f * s;
                const float ds[4] = {d0, bf(db - 1u), bf(db + 1u), dr};
                for (int t = 0; t < (mode == 0 ? 4 : 3); ++t) {
                    const float d = ds[t];
                    if (!(d >= 0.0f) || isinf(d)) continue;
                    ++n;
                    if (fb(quot3(d, s, y)) != fb(d / s)) {
                        if (bad < 5) printf("mismatch s=%a d=%a\n", s, d);
                        ++bad;
                    }
                }
            }
        }
    }
    printf("%lld %lld\n", n, bad);
    return 0;
}
"""


@pytest.fixture(scope="module")
def sweep_binary(tmp_path_factory):
    d = str(tmp_path_factory.mktemp("kvq_quot"))
    src, exe = os.path.join(d, "quot.c"), os.path.join(d, "quot")
    with open(src, "w") as f:
        f.write(C_SRC)
    # no contraction: every product and FMA is exactly the one written
    r = subprocess.run(["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-o", exe, src, "-lm"],
                       capture_output=True, text=True)
    if r.returncode != 0:
        pytest.skip(f"gcc unavailable: {r.stderr[-300:]}")
    return exe


def run_sweep(exe, stride, mode):
    r = subprocess.run([exe, str(stride), str(mode)], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr
    *detail, last = r.stdout.strip().splitlines()
    n, bad = (int(x) for x in last.split())
    return n, bad, "\n".join(detail)


def test_int4_quotient_equals_ieee_division(sweep_binary):
    """INT4 fast groups: scale in [2^-100, 2^100], quotients at the code boundaries."""
    n, bad, detail = run_sweep(sweep_binary, 2048, 0)
    assert n > 10_000_000
    assert bad == 0, detail


def test_fp8_row_quotient_equals_ieee_division(sweep_binary):
    """FP8-row fast rows: scale in [2^-90, 2^100], quotients at the E4M3 midpoints down to 2^-10."""
    n, bad, detail = run_sweep(sweep_binary, 2048, 1)
    assert n > 10_000_000
    assert bad == 0, detail


def test_nvfp4_row_block_scale_equals_ieee_division(sweep_binary):
    """NVFP4-row decode scale fl(e4m3 / g): every E4M3 code over multipliers g in [2^-100, 2^100]
    (the encoder's and decoders' quotient with y = RN(1/g))."""
    n, bad, detail = run_sweep(sweep_binary, 512, 3)
    assert n > 10_000_000
    assert bad == 0, detail


def test_fp8_row_range_bound_is_needed(sweep_binary):
    """Below 2^-90 the remainder of the smallest E4M3 quotients falls under 2^-126 and loses bits:
    at scales near 2^-100 the corrected quotient misses RN(x/s) there, which is why FP8-row rows
    with a smaller scale take the division."""
    n, bad, _ = run_sweep(sweep_binary, 2048, 2)
    assert n > 0 and bad > 0


def test_plain_product_is_not_enough(sweep_binary, tmp_path):
    """The correction is needed: RN(d * RN(1/s)) alone misses RN(d/s) on these inputs, so the
    sweeps above are not vacuous."""
    src = C_SRC.replace("return fmaf(r, y, q0);", "(void)r; return q0;")
    d = str(tmp_path)
    with open(os.path.join(d, "p.c"), "w") as f:
        f.write(src)
    exe = os.path.join(d, "p")
    subprocess.run(["gcc", "-O2", "-ffp-contract=off", "-o", exe, os.path.join(d, "p.c"), "-lm"], check=True)
    for mode in (0, 1):
        n, bad, _ = run_sweep(exe, 65536, mode)
        assert n > 0 and bad > 0
