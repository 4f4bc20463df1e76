"""Host-side check of the division the UE4M3/UE5M3 kernels use for x / d.

The kernels form q = x r, n = fma(q, d, -x), y = fma(-n, r, q) with
r = RN(1/d) (Markstein's FMA-corrected reciprocal product, written with the
negated remainder so that -0 / d stays -0) on blocks whose
decode scale d lies in [2^-96, 2^100] with |x| <= 4096 d, and a plain division
elsewhere.  This test runs the same binary32 sequence on the CPU (fmaf is the
correctly rounded fused multiply-add) and checks it against IEEE division:
  - y is bitwise RN(x / d) for every |x| >= 2^-100 tested: all 2^23 significands
    of d against a spread of x significands, and random (x, d) over the whole
    fast-path range;
  - for |x| < 2^-100, |y| < 0.25 and y has the sign of x, so the E2M1 code is
    the same sign-only zero as for the exact quotient;
  - x = +0 and -0 give +0 and -0 for every d, and d = 0 with r = 0 gives a zero
    of x's sign for every finite x (the zero-scale blocks).
"""
import os
import subprocess

import pytest

SRC = r"""
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

static float f_of(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t u_of(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

/* noinline + volatile: the sequence must run as instructions, not be
   constant-folded by the compiler (which mishandles the sign of zero here). */
__attribute__((noinline)) static float fast_div(float x_in, float d_in, float r_in) {
    volatile float vx = x_in, vd = d_in, vr = r_in;
    float x = vx, d = vd, r = vr;
    volatile float q = x * r;
    volatile float nrem = fmaf(q, d, f_of(u_of(x) ^ 0x80000000u));  /* q d - x */
    return fmaf(f_of(u_of(nrem) ^ 0x80000000u), r, q);  /* negated remainder keeps the sign of zero */
}

static uint64_t state = 0x9E3779B97F4A7C15ull;
static uint64_t next(void) {            /* splitmix64 */
    uint64_t z = (state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

int main(void) {
    long bad = 0, checked = 0;
    /* 1: every significand of d in [1, 2) against 64 x significands in [1, 4) */
    for (uint32_t md = 0; md < (1u << 23); ++md) {
        float d = f_of(0x3F800000u | md);
        float r = 1.0f / d;
        for (int k = 0; k < 64; ++k) {
            uint32_t mx = (k < 32) ? ((uint32_t)k << 18) : (uint32_t)(next() & 0x7FFFFF);
            float x = f_of(((127u + (k & 1)) << 23) | mx);
            float y = fast_div(x, d, r), e = x / d;
            ++checked;
            if (u_of(y) != u_of(e)) { if (bad < 5) printf("exh x=%a d=%a y=%a e=%a\n", x, d, y, e); ++bad; }
        }
    }
    /* 2: random d in [2^-96, 2^100], x with |x/d| <= 4096 */
    for (long i = 0; i < 60000000L; ++i) {
        int ed = (int)(next() % 197) - 96;
        float d = ldexpf(1.0f + (float)(next() & 0x7FFFFF) * 0x1p-23f, ed);
        if (d > 0x1p100f) d = 0x1p100f;
        float r = 1.0f / d;
        int ex = (int)(next() % 46) - 33;          /* x/d in about [2^-33, 2^12] */
        float x = ldexpf(1.0f + (float)(next() & 0x7FFFFF) * 0x1p-23f, ex) * d;
        if (!(fabsf(x) <= 4096.0f * d)) continue;
        if (next() & 1) x = -x;
        float y = fast_div(x, d, r);
        ++checked;
        if (fabsf(x) >= 0x1p-100f) {
            float e = x / d;
            if (u_of(y) != u_of(e)) { if (bad < 10) printf("rnd x=%a d=%a y=%a e=%a\n", x, d, y, e); ++bad; }
        } else {
            if (!(fabsf(y) < 0.25f) || (signbit(y) != signbit(x))) { if (bad < 10) printf("tiny x=%a d=%a y=%a\n", x, d, y); ++bad; }
        }
    }
    /* 3: tiny and subnormal x against the smallest fast-path scales */
    for (long i = 0; i < 20000000L; ++i) {
        float d = ldexpf(1.0f + (float)(next() & 0x7FFFFF) * 0x1p-23f, -96 + (int)(next() % 12));
        float r = 1.0f / d;
        float x = f_of((uint32_t)(next() % 0x0C000000u));  /* 0 .. ~2^-103 incl. subnormals */
        if (next() & 1) x = -x;
        float y = fast_div(x, d, r);
        ++checked;
        if (fabsf(x) >= 0x1p-100f) {
            if (u_of(y) != u_of(x / d)) ++bad;
        } else if (!(fabsf(y) < 0.25f) || (signbit(y) != signbit(x))) {
            if (bad < 10) printf("sub x=%a d=%a y=%a\n", x, d, y);
            ++bad;
        }
    }
    /* 4: signed zeros against any scale, including d = 0 (r = 0) */
    for (long i = 0; i < 1000000L; ++i) {
        float d = (i % 7 == 0) ? 0.0f : ldexpf(1.0f + (float)(next() & 0x7FFFFF) * 0x1p-23f, (int)(next() % 197) - 96);
        float r = d > 0.0f ? 1.0f / d : 0.0f;
        float x = (i & 1) ? -0.0f : 0.0f;
        float y = fast_div(x, d, r);
        ++checked;
        if (u_of(y) != u_of(x)) { if (bad < 10) printf("zero x=%a d=%a y=%a\n", x, d, y); ++bad; }
    }
    /* 5: any x against the zero scale (d = 0, r = 0) gives a zero of x's sign */
    for (long i = 0; i < 1000000L; ++i) {
        float x = f_of((uint32_t)(next() & 0xFF7FFFFFu));
        if (!isfinite(x)) continue;
        float y = fast_div(x, 0.0f, 0.0f);
        ++checked;
        if (y != 0.0f || signbit(y) != signbit(x)) { if (bad < 10) printf("d0 x=%a y=%a\n", x, y); ++bad; }
    }
    printf("checked %ld bad %ld\n", checked, bad);
    return bad != 0;
}
"""


def test_fma_corrected_division_is_correctly_rounded(tmp_path):
    src = tmp_path / "div.c"
    exe = tmp_path / "div"
    src.write_text(SRC)
    flags = ["-O2", "-ffp-contract=off", "-fno-fast-math", "-fexcess-precision=standard"]
    if "fma" in open("/proc/cpuinfo").read().split():
        flags.append("-mfma")
    subprocess.run(["gcc", *flags, "-o", str(exe), str(src), "-lm"], check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=600)
    print(r.stdout)
    assert r.returncode == 0, r.stdout
