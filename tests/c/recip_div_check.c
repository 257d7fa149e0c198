/* Checks, on the host's IEEE f32 arithmetic (fused multiply-add exact, round to nearest
 * even, subnormals kept), that the quantizer's reciprocal form of x / s,
 *     q0 = clamp(x * r, -2^100, 2^100),  r = RN(1 / s)
 *     q  = RN(q0 - RN(q0 * s - x) * r)          (two fused multiply-adds)
 * equals the IEEE quotient RN(x / s) for bf16 x and scales s in [2^-80, 2^100]:
 *  1. bit for bit, for every bf16 significand of either sign against every f32 scale
 *     significand in [1, 2) (2^31 pairs; inside the range the exponents only scale both sides);
 *  2. on all 65,536 bf16 bit patterns at scales spread over the range (NaN excluded, which the
 *     kernel selects on x), where what decides the e4m3 code must agree: the sign, the value
 *     bits when |q| lies in [2^-10, 448), and only "saturates" or "rounds to zero" outside.
 * Prints the counts; exits 1 on any mismatch. With argument "neg", checks the uncorrected
 * q0 instead and is expected to fail (the checks are not vacuous). */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

static float f32(uint32_t u) { float x; memcpy(&x, &u, 4); return x; }
static uint32_t bits(float x) { uint32_t v; memcpy(&v, &x, 4); return v; }
static float clampf(float a, float lo, float hi) { return a < lo ? lo : (a > hi ? hi : a); }
static int neg_control;

static float recip_div(float x, float s, float r) {
    const float q0 = clampf(x * r, -0x1p100f, 0x1p100f);
    if (neg_control) return q0;
    return fmaf(fmaf(q0, s, -x), -r, q0);
}

static int code_relevant_equal(float a, float b) {
    if (signbit(a) != signbit(b)) return 0;
    const float A = fabsf(a), B = fabsf(b);
    if (A >= 448.f && B >= 448.f) return 1;
    if (A < 0x1p-10f && B < 0x1p-10f) return 1;
    return bits(A) == bits(B);
}

static uint64_t rng = 88172645463325252ull;
static uint32_t next(void) { rng ^= rng << 13; rng ^= rng >> 7; rng ^= rng << 17; return (uint32_t)rng; }

int main(int argc, char** argv) {
    neg_control = argc > 1 && strcmp(argv[1], "neg") == 0;
    long n1 = 0, bad1 = 0, n2 = 0, bad2 = 0;
    for (uint32_t sm = 0; sm < (1u << 23); ++sm) {
        const float s = f32(0x3f800000u | sm), r = 1.0f / s;
        for (uint32_t xm = 0; xm < 256; ++xm) {
            const float x = f32(((xm & 128 ? 0xbf80u : 0x3f80u) | (xm & 127)) << 16);
            ++n1;
            if (bits(recip_div(x, s, r)) != bits(x / s)) ++bad1;
        }
    }
    for (int ex = -80; ex <= 99; ++ex)
        for (int k = 0; k < 12; ++k) {
            const float s = ldexpf(k == 0 ? 1.0f : f32(0x3f800000u | (next() & 0x7fffffu)), ex), r = 1.0f / s;
            for (uint32_t xb = 0; xb < 65536; ++xb) {
                const float x = f32(xb << 16);
                if (isnan(x)) continue;
                ++n2;
                if (!code_relevant_equal(recip_div(x, s, r), x / s)) ++bad2;
            }
        }
    printf("significand pairs %ld mismatches %ld; bf16 patterns x scales %ld mismatches %ld\n", n1, bad1, n2, bad2);
    return bad1 || bad2;
}
