"""The quantiser's division-free INT8 rounding, checked against IEEE division on the CPU.

Per row the kernels take r = RN(1/(8s)) once; per element, with y = fl32(8x'), they form
q0 = RN(y r) and q1 = RN(q0 + RN-exact(y - q0 (8s)) r) (two fused multiply-adds: Markstein's
correction step), which must equal the correctly rounded quotient fl32(y / (8s)) = fl32(x'/s); then
adding 1.5 * 2^23 rounds q1 half-to-even into the low mantissa bits.  The symmetric INT8 code is the
low byte of that sum and the asymmetric path takes the whole integer (bits minus the bits of 1.5 * 2^23).

A small C program (gcc, fmaf from the C library: a correctly rounded fused multiply-add, no
fast-math, no contraction) runs the recurrence on scales s = fl32(amax / 127), also rounded to
bf16, over amax from 2^-103 (the fast path's lower limit) up to 2^100, and on every quotient tie
k + 1/2 (k = -128..127) with its 3 fp32 neighbours on each side, plus random quotients; every code
must equal rint(IEEE quotient), and q1 must equal the IEEE quotient bit for bit (a zero quotient
may carry either sign: it gives code 0 both ways).  This is an
independent check of the arithmetic the kernels use; it shares no code with them."""
import os
import subprocess
import tempfile

import pytest

SRC = r"""
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

static uint32_t bits(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }
static float from_bits(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint64_t st = 0x9E3779B97F4A7C15ull;
static uint64_t next(void) {   /* SplitMix64 */
    uint64_t z = (st += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}
static float bf16_round(float f) {
    uint32_t u = bits(f);
    u = (u + 0x7fffu + ((u >> 16) & 1u)) & 0xffff0000u;
    return from_bits(u);
}
static long checked = 0, bad_q = 0, bad_code = 0, bad_int = 0;
static void check(float y, float s) {
    const float s8 = s * 8.0f, r8 = 1.0f / s8;
    const float q0 = y * r8;
    const float q1 = fmaf(fmaf(-q0, s8, y), r8, q0);
    const float ref = y / s8;
    ++checked;
    /* equal bit for bit, except that a zero quotient may come out as +0 where IEEE gives -0 */
    if (bits(q1) != bits(ref) && !(q1 == 0.0f && ref == 0.0f)) { if (bad_q++ < 5) printf("q1 %a ref %a y %a s %a\n", q1, ref, y, s); }
    const float magic = 12582912.0f;   /* 1.5 * 2^23 */
    const float t = q1 + magic;
    float rr = rintf(ref);
    if (fabsf(rr) <= 127.0f) {
        const int8_t code = (int8_t)(bits(t) & 0xffu);
        if ((float)code != rr) { if (bad_code++ < 5) printf("code %d ref %a y %a s %a\n", code, ref, y, s); }
    }
    if (fabsf(rr) <= 4096.0f) {
        const int32_t whole = (int32_t)bits(t) - (int32_t)0x4B400000;
        if ((float)whole != rr) { if (bad_int++ < 5) printf("int %d ref %a\n", whole, ref); }
    }
}
int main(int argc, char** argv) {
    const int nscale = argc > 1 ? atoi(argv[1]) : 4096;
    for (int i = 0; i < nscale; ++i) {
        /* amax log-uniform in [2^-103, 2^100) with a random significand */
        const int e = -103 + (int)(next() % 203);
        const float amax = ldexpf(1.0f + (float)(next() >> 41) * 0x1p-23f, e);
        for (int b = 0; b < 2; ++b) {
            float s = amax / 127.0f;
            if (b) s = bf16_round(s);
            if (!(s > 0.0f) || isinf(s)) continue;
            const float s8 = s * 8.0f;
            for (int k = -128; k <= 127; ++k) {
                const float y0 = ((float)k + 0.5f) * s8;
                uint32_t u = bits(y0);
                for (int dlt = -3; dlt <= 3; ++dlt) {
                    const uint32_t v = u + (uint32_t)dlt;
                    const float y = from_bits(v);
                    if (isfinite(y)) check(y, s);
                }
            }
            for (int j = 0; j < 256; ++j) {
                /* a random fp32 y with |y| <= 8 * amax (the row maximum bounds |x'|) */
                const float frac = (float)(next() >> 40) * 0x1p-24f;
                float y = (next() & 1 ? -1.0f : 1.0f) * frac * 8.0f * amax;
                check(y, s);
            }
        }
    }
    printf("checked %ld bad_q %ld bad_code %ld bad_int %ld\n", checked, bad_q, bad_code, bad_int);
    return (bad_q || bad_code || bad_int) ? 1 : 0;
}
"""


def test_division_free_int8_quotient_equals_ieee_division():
    with tempfile.TemporaryDirectory() as tmp:
        src = os.path.join(tmp, "q.c")
        exe = os.path.join(tmp, "q")
        with open(src, "w") as f:
            f.write(SRC.replace("#include <string.h>", "#include <string.h>\n#include <stdlib.h>"))
        r = subprocess.run(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-o", exe, src, "-lm"],
                           capture_output=True, text=True)
        if r.returncode != 0:
            pytest.fail(r.stderr)
        out = subprocess.run([exe, "24000"], capture_output=True, text=True, timeout=300)
        assert out.returncode == 0, out.stdout
        checked = int(out.stdout.split("checked ")[1].split()[0])
        assert checked > 9 * 10**7
