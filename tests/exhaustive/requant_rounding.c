/* Exhaustive check, on the CPU, of the identity the requantisation kernel
 * relies on: for every finite binary16 scale s > 0 and every finite binary16
 * or bfloat16 weight w,
 *
 *   clamp(rint(fl32(w / s)), -7, 7)                       (the definition)
 *     ==
 *   RNE( snap(clamp(fl32(w * fl32(1 / s)), -7, 7)) )      (the kernel)
 *
 * where snap rounds to a multiple of 2^-14 (adding 768 = 1.5 * 2^9 in
 * binary32) and RNE rounds to an integer by adding 1.5 * 2^23 - 768, whose
 * low four mantissa bits are then the two's-complement code.  Zero and
 * infinite scales give code 0 on both sides.  All arithmetic is binary32 with
 * round-to-nearest-even and no contraction (build with -ffp-contract=off).
 *
 * Returns the number of mismatching pairs (and the first one). */
#include <math.h>
#include <stdint.h>
#include <string.h>

static float f16_to_f32(uint16_t h)
{
    const uint32_t sign = (uint32_t)(h >> 15) << 31;
    const int exp = (h >> 10) & 0x1F;
    const uint32_t man = h & 0x3FF;
    float v;
    if (exp == 0) {
        v = ldexpf((float)man, -24);              /* subnormal (or zero) */
    } else {
        v = ldexpf((float)(man | 0x400), exp - 25);
    }
    uint32_t b;
    memcpy(&b, &v, 4);
    b |= sign;
    memcpy(&v, &b, 4);
    return v;
}

static float bf16_to_f32(uint16_t h)
{
    const uint32_t b = (uint32_t)h << 16;
    float v;
    memcpy(&v, &b, 4);
    return v;
}

static int code_definition(float w, float s)
{
    if (!(s > 0.0f) || isinf(s))
        return 0;
    float q = rintf(w / s);
    if (q > 7.0f) q = 7.0f;
    if (q < -7.0f) q = -7.0f;
    return ((int)q) & 0xF;
}

static int code_kernel(float w, float r, int snap)
{
    float a = w * r;
    if (a > 7.0f) a = 7.0f;
    if (a < -7.0f) a = -7.0f;
    /* volatile: keep each binary32 rounding.  snap = 0 is the same code
     * without the 2^-14 snap (a negative control: it misplaces ties). */
    volatile float u = snap ? a + 768.0f : a;
    volatile float t = snap ? u + 12582144.0f : u + 12582912.0f;
    uint32_t b;
    float tv = t;
    memcpy(&b, &tv, 4);
    return (int)(b & 0xF);
}

/* dtype 0: binary16 weights, 1: bfloat16 weights.  Scales s_lo..s_hi-1
 * (binary16 bit patterns). */
long long count_mismatches(int dtype, int s_lo, int s_hi, int snap, uint32_t *first_w,
                           uint32_t *first_s)
{
    long long bad = 0;
#pragma omp parallel for schedule(dynamic, 64) reduction(+ : bad)
    for (int sb = s_lo; sb < s_hi; ++sb) {
        const float s = f16_to_f32((uint16_t)sb);
        const float r = (s > 0.0f && !isinf(s)) ? 1.0f / s : 0.0f;
        for (int wb = 0; wb < 65536; ++wb) {
            const float w = dtype == 0 ? f16_to_f32((uint16_t)wb) : bf16_to_f32((uint16_t)wb);
            if (!isfinite(w))
                continue;
            if (code_definition(w, s) != code_kernel(w, r, snap)) {
#pragma omp critical
                {
                    if (bad == 0 && *first_w == 0xFFFFFFFFu) {
                        *first_w = (uint32_t)wb;
                        *first_s = (uint32_t)sb;
                    }
                }
                ++bad;
            }
        }
    }
    return bad;
}
