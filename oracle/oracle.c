/*
 * oracle.c -- CPU oracle for speculative-decoding verification through a
 * calibrated int4 output head (lm_head).
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the plain, slow, obviously correct
 * definition that the GPU library is checked against.  Only the test suite,
 * the smoke check and the CPU-baseline leg of the benchmark may load it.  It
 * shares no code, header, table or helper with the GPU library, and the GPU
 * library never calls it.
 *
 * What it computes (one verify block of R independent requests, each of T
 * positions, M = R*T rows of final hidden states):
 *
 *   1. unpack: the head is stored two int4 values per byte, row-major
 *      [V, H/2]; the low nibble holds the even hidden channel, the high
 *      nibble the odd one; each nibble is a two's-complement value and only
 *      [-7, 7] is legal (nibble 0x8 is rejected).
 *      Range and symmetric quantisation: "Qwen3.8-27B on a Single RTX 3090:
 *      How Calibrated Quantization and Speculative Decoding Hit 1,000 tok/s",
 *      Technical Insight (the requantisation listing clamps to [-7, 7] and
 *      keeps one scale per hidden channel).  Nibble order and sign encoding
 *      are not given on any page; the reading above is this project's.
 *   2. dequant and product: p = (f32(x[r,h]) * f32(s[h])) * f32(q[v,h]),
 *      every multiply in IEEE binary32.  x and s are binary16, so the first
 *      product is exact.
 *   3. fixed-order sum: acc = +0.0f, then acc = acc + p for h = 0, 1, ...,
 *      H-1, each add rounded to binary32 (built with -ffp-contract=off, so no
 *      fused multiply-add).  logit[r,v] = acc.
 *   4. greedy argmax per row: the largest logit, lowest vocab index on ties
 *      (strict '>' while scanning v upward; -0.0 and +0.0 compare equal).
 *   5. acceptance per request i: the number of leading draft ids that equal
 *      the argmax at the same position, at most T-1.  Greedy verification of
 *      a drafted block: "Qwen3.8-27B on a Single RTX 3090: ...", Technical
 *      Insight (the split-KV verify listing: compare, keep the accepted
 *      prefix, clear the rejected drafts), and "HyperQwen on one RTX 3090:
 *      a first-time developer's guide to the 381-token claim", section
 *      "What actually became faster?" (a block of up to 16 tokens is
 *      verified in one step).
 *
 * Parallelism: OpenMP over vocab rows only.  Each dot product is one
 * sequential chain, so the result does not depend on the thread count.
 *
 * Build: gcc -O2 -std=c11 -ffp-contract=off -fno-fast-math -fopenmp
 *        -shared -fPIC oracle.c -o liboracle.so -lm
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum {
    ORACLE_OK = 0,
    ORACLE_EINVAL = -1,    /* bad sizes or missing pointers */
    ORACLE_EWEIGHT = -2,   /* a weight nibble equals 0x8 (-8 is not a legal value) */
    ORACLE_ENONFINITE = -3 /* a hidden or scale value is Inf or NaN */
};

/* IEEE 754 binary16 -> double, from the format definition:
 * sign 1 bit, exponent 5 bits (bias 15), fraction 10 bits. */
double oracle_half_to_double(uint16_t bits)
{
    int sign = (bits >> 15) & 1;
    int expo = (bits >> 10) & 0x1F;
    int frac = bits & 0x3FF;
    double v;
    if (expo == 0)
        v = ldexp((double)frac, -24);              /* subnormal: frac * 2^-24 */
    else if (expo == 31)
        v = frac ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + frac), expo - 25); /* (1 + frac/1024) * 2^(expo-15) */
    return sign ? -v : v;
}

/* Two's-complement value of a 4-bit nibble. */
static int sext4(int nib)
{
    return nib >= 8 ? nib - 16 : nib;
}

/* Unpack [V, H/2] bytes to int8 [V, H].  Returns ORACLE_EWEIGHT and the
 * number of illegal nibbles in *n_bad if any nibble is 0x8. */
int oracle_unpack(const uint8_t *packed, int V, int H, int8_t *q_out, int64_t *n_bad)
{
    if (!packed || !q_out || V < 1 || H < 2 || (H & 1))
        return ORACLE_EINVAL;
    int64_t bad = 0;
    size_t half = (size_t)H / 2;
    for (size_t v = 0; v < (size_t)V; ++v) {
        for (size_t j = 0; j < half; ++j) {
            uint8_t b = packed[v * half + j];
            int lo = b & 0xF, hi = b >> 4;
            bad += (lo == 8) + (hi == 8);
            q_out[v * (size_t)H + 2 * j] = (int8_t)sext4(lo);
            q_out[v * (size_t)H + 2 * j + 1] = (int8_t)sext4(hi);
        }
    }
    if (n_bad)
        *n_bad = bad;
    return bad ? ORACLE_EWEIGHT : ORACLE_OK;
}

/* Count nibbles equal to 0x8. */
int64_t oracle_count_bad_nibbles(const uint8_t *packed, int V, int H)
{
    int64_t bad = 0;
    size_t n = (size_t)V * (size_t)H / 2;
    for (size_t i = 0; i < n; ++i)
        bad += ((packed[i] & 0xF) == 8) + ((packed[i] >> 4) == 8);
    return bad;
}

static int check_finite(const uint16_t *h, size_t n)
{
    for (size_t i = 0; i < n; ++i)
        if (((h[i] >> 10) & 0x1F) == 31)
            return ORACLE_ENONFINITE;
    return ORACLE_OK;
}

/* One logit, the definition written out: sequential binary32 sum over h. */
float oracle_logit_one(const uint16_t *hidden_row, const uint8_t *packed_row,
                       const uint16_t *scales, int H)
{
    float acc = 0.0f;
    for (int h = 0; h < H; ++h) {
        uint8_t b = packed_row[h / 2];
        int nib = (h & 1) ? (b >> 4) : (b & 0xF);
        float q = (float)sext4(nib);
        float x = (float)oracle_half_to_double(hidden_row[h]);
        float s = (float)oracle_half_to_double(scales[h]);
        float p = (x * s) * q;
        acc = acc + p;
    }
    return acc;
}

/* All logits [M, V] (row r of the block against every vocab row v). */
int oracle_logits(const uint16_t *hidden, const uint8_t *packed, const uint16_t *scales,
                  int M, int V, int H, float *logits, int n_threads)
{
    if (!hidden || !packed || !scales || !logits || M < 1 || V < 1 || H < 2 || (H & 1))
        return ORACLE_EINVAL;
    if (check_finite(hidden, (size_t)M * H) || check_finite(scales, (size_t)H))
        return ORACLE_ENONFINITE;
    if (oracle_count_bad_nibbles(packed, V, H))
        return ORACLE_EWEIGHT;

    /* x*s is exact in binary32 (11 + 11 significand bits), so forming it once
     * per (r, h) gives the same bits as forming it inside every product. */
    float *xs = (float *)malloc(sizeof(float) * (size_t)M * H);
    if (!xs)
        return ORACLE_EINVAL;
    for (size_t r = 0; r < (size_t)M; ++r)
        for (size_t h = 0; h < (size_t)H; ++h)
            xs[r * H + h] = (float)oracle_half_to_double(hidden[r * H + h]) *
                            (float)oracle_half_to_double(scales[h]);

#ifdef _OPENMP
    if (n_threads > 0)
        omp_set_num_threads(n_threads);
#else
    (void)n_threads;
#endif
    size_t half = (size_t)H / 2;
#pragma omp parallel
    {
        float *q = (float *)malloc(sizeof(float) * (size_t)H);
#pragma omp for schedule(static)
        for (long v = 0; v < (long)V; ++v) {
            const uint8_t *row = packed + (size_t)v * half;
            for (size_t j = 0; j < half; ++j) {
                q[2 * j] = (float)sext4(row[j] & 0xF);
                q[2 * j + 1] = (float)sext4(row[j] >> 4);
            }
            for (size_t r = 0; r < (size_t)M; ++r) {
                const float *x = xs + r * H;
                float acc = 0.0f;
                for (size_t h = 0; h < (size_t)H; ++h) {
                    float p = x[h] * q[h];
                    acc = acc + p;
                }
                logits[r * (size_t)V + (size_t)v] = acc;
            }
        }
        free(q);
    }
    free(xs);
    return ORACLE_OK;
}

/* Per-row argmax (lowest index on ties), the max value, the gap between the
 * best and the second-best logit (+inf when V == 1), and the largest |logit|
 * of the row. */
int oracle_argmax_rows(const float *logits, int M, int V, int32_t *idx, float *maxv,
                       float *gap, float *amax)
{
    if (!logits || !idx || M < 1 || V < 1)
        return ORACLE_EINVAL;
    for (size_t r = 0; r < (size_t)M; ++r) {
        const float *row = logits + r * (size_t)V;
        int best = 0;
        for (int v = 1; v < V; ++v)
            if (row[v] > row[best])
                best = v;
        float second = -INFINITY, am = 0.0f;
        for (int v = 0; v < V; ++v) {
            if (v != best && row[v] > second)
                second = row[v];
            float a = fabsf(row[v]);
            if (a > am)
                am = a;
        }
        idx[r] = best;
        if (maxv)
            maxv[r] = row[best];
        if (gap)
            gap[r] = (V > 1) ? row[best] - second : INFINITY;
        if (amax)
            amax[r] = am;
    }
    return ORACLE_OK;
}

/* Accepted-prefix length per request: drafts [R, T-1] against argmax [R, T]. */
int oracle_accept(const int32_t *argmax_ids, const int32_t *draft_ids, int R, int T,
                  int32_t *n_accepted)
{
    if (!argmax_ids || !n_accepted || R < 1 || T < 1 || (T > 1 && !draft_ids))
        return ORACLE_EINVAL;
    for (int i = 0; i < R; ++i) {
        int n = 0;
        while (n < T - 1 && argmax_ids[i * T + n] == draft_ids[i * (T - 1) + n])
            ++n;
        n_accepted[i] = n;
    }
    return ORACLE_OK;
}

/* The whole verify step.  logits_out may be NULL; gap_out and amax_out may be
 * NULL.  All arrays are host memory owned by the caller. */
int oracle_verify(const uint16_t *hidden, const uint8_t *packed, const uint16_t *scales,
                  const int32_t *draft_ids, int R, int T, int V, int H,
                  float *logits_out, float *logits_max, int32_t *argmax_ids,
                  int32_t *n_accepted, float *gap_out, float *amax_out, int n_threads)
{
    if (R < 1 || T < 1 || T > 16 || !logits_max || !argmax_ids || !n_accepted)
        return ORACLE_EINVAL;
    if (T > 1 && !draft_ids)
        return ORACLE_EINVAL;
    int M = R * T;
    float *lg = logits_out;
    if (!lg) {
        lg = (float *)malloc(sizeof(float) * (size_t)M * (size_t)V);
        if (!lg)
            return ORACLE_EINVAL;
    }
    int st = oracle_logits(hidden, packed, scales, M, V, H, lg, n_threads);
    if (st == ORACLE_OK)
        st = oracle_argmax_rows(lg, M, V, argmax_ids, logits_max, gap_out, amax_out);
    if (st == ORACLE_OK)
        st = oracle_accept(argmax_ids, draft_ids, R, T, n_accepted);
    if (lg != logits_out)
        free(lg);
    return st;
}
