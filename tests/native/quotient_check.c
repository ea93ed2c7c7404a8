/* Host check of the quotient method the quantizer kernels use: for a block
 * scale s >= 2^-80 and |v| <= 448 s, the quotient q2 below (reciprocal
 * r = fl32(1/s), q0 = fl32(v r), two FMA correction steps, sign copied from
 * v) must equal the IEEE quotient fl32(v / s) whenever |v / s| >= 2^-10, and
 * must be a zero or a value below 2^-10 of the same sign otherwise: either way
 * it encodes to the same E4M3 code.  Compiled with contraction off; fmaf is
 * the libm fused multiply-add.
 *
 * usage: quotient_check <random pairs>; prints one line and exits 0 when no
 * pair disagrees. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static uint64_t state = 0x9E3779B97F4A7C15ull;
static uint64_t next(void) { state ^= state << 13; state ^= state >> 7; state ^= state << 17; return state; }
static float from_bits(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t bits(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }
static double unit(void) { return (double)(next() >> 11) / 9007199254740992.0; }

static float quotient(float v, float s)
{
    volatile float r = 1.0f / s;
    float q0 = v * r;
    float q1 = fmaf(fmaf(-q0, s, v), r, q0);
    float q2 = fmaf(fmaf(-q1, s, v), r, q1);
    return copysignf(q2, v);
}

static long checked, bad;

static void check(float v, float s)
{
    float want, got;
    if (!isfinite(v) || !isfinite(s) || s < 0x1p-80f || fabsf(v) > 448.0f * s)
        return;
    want = v / s;
    got = quotient(v, s);
    checked++;
    if (fabsf(want) >= 0x1p-10f ? bits(want) != bits(got)
                                : (fabsf(got) >= 0x1p-10f || signbit(got) != signbit(want))) {
        if (bad < 5)
            printf("mismatch v=%a s=%a ieee=%a fma=%a\n", v, s, want, got);
        bad++;
    }
}

int main(int argc, char **argv)
{
    long pairs = argc > 1 ? atol(argv[1]) : 1000000;
    static const float scales[] = {0x1p-80f, 0x1.000002p-80f, 0x1p-60f, 1.0f / 448, 3.0f / 448, 0.7f, 1.0f,
                                   0x1.fffffep0f, 123.456f, 0x1p100f, 0x1.fffffep127f / 448};
    long i;
    uint32_t h, m;
    size_t k;
    /* every bf16 value against a set of scales */
    for (k = 0; k < sizeof scales / sizeof scales[0]; k++)
        for (h = 0; h < 65536; h++)
            check(from_bits(h << 16), scales[k]);
    /* every scale mantissa at exponent 0, random quotients */
    for (m = 0; m < 0x800000; m += 7)
        check((float)(unit() * 896.0 - 448.0) * from_bits((127u << 23) | m), from_bits((127u << 23) | m));
    /* random scales over the whole range, quotients of several shapes */
    for (i = 0; i < pairs; i++) {
        float s = from_bits(((47u + (uint32_t)(next() % 207)) << 23) | (uint32_t)(next() & 0x7FFFFF));
        switch (next() & 3) {
        case 0: check(from_bits((uint32_t)next()), s); break;
        case 1: check(s * (float)(unit() * 896.0 - 448.0), s); break;
        case 2: check(s * from_bits(0x3F800000u | (uint32_t)(next() & 0x7FFFFF)) * (float)(next() % 448), s); break;
        default: check(from_bits(bits(s * 448.0f) - (uint32_t)(next() % 0x40000000u)), s); break;
        }
    }
    printf("checked %ld quotients, %ld disagree\n", checked, bad);
    return bad != 0;
}
