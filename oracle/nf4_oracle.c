/*
 * nf4_oracle.c -- plain, slow, single-threaded CPU reference (test
 * infrastructure only; see nf4_oracle.h for who may use it and for the page
 * key used in the citations below).
 *
 * Build: gcc -O2 -std=c11 -ffp-contract=off -fPIC -shared -lm.
 * fp32 steps use C float arithmetic (SSE, FLT_EVAL_METHOD == 0, no FMA
 * contraction, denormals kept); everything the pages leave in open precision
 * is done in fp64.
 */
#include "nf4_oracle.h"

#include <assert.h>
#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------- */
/* Standard normal CDF and its inverse.                                       */
/* ------------------------------------------------------------------------- */

/* Phi(x) = P(Z <= x) for Z ~ N(0,1), through the C99 complementary error
 * function: Phi(x) = erfc(-x / sqrt 2) / 2. */
static double normal_cdf(double x) { return 0.5 * erfc(-x / sqrt(2.0)); }

/* Inverse of normal_cdf by bisection over doubles: the loop halves [lo, hi]
 * until no double lies strictly between the ends, then returns the end whose
 * CDF is closer to p. */
static double normal_quantile(double p)
{
    assert(p > 0.0 && p < 1.0);
    double lo = -40.0, hi = 40.0;
    for (;;) {
        double mid = lo + 0.5 * (hi - lo);
        if (mid <= lo || mid >= hi) break;
        if (normal_cdf(mid) < p) lo = mid; else hi = mid;
    }
    return (fabs(normal_cdf(lo) - p) < fabs(normal_cdf(hi) - p)) ? lo : hi;
}

/* ------------------------------------------------------------------------- */
/* O1. The 16 NF4 levels.                                                     */
/* ------------------------------------------------------------------------- */
/* [QLoRA page, How It Works, NF4 item]: 16 values, each receiving an equal
 * share of normally distributed weights; [QLoRA explained, NF4]: built around
 * the normal distribution of weights.  So the levels are normal quantiles at
 * evenly spaced probabilities.
 *
 * Reading (the pages give no formula): the format has an exact zero and the
 * endpoints -1 and +1.  An exact zero with 16 levels forces an uneven split:
 * 8 positive and 7 negative quantiles.  The probabilities run evenly from an
 * offset delta down to 1/2 on each side (8 steps on the positive side, 7 on
 * the negative side, 1/2 itself excluded, where zero sits).  delta is the mean
 * of 1 - 1/(2*15) and 1 - 1/(2*16), i.e. 929/960, which keeps the outermost
 * quantile finite.  All levels are divided by the quantile at delta, so the
 * outermost are exactly -1 and +1, and rounded to fp32. */
int nf4o_levels(float out16[16])
{
    const double delta = 929.0 / 960.0;
    const double top = normal_quantile(delta);
    /* negative half: codes 0..6, probabilities delta - k*(delta-1/2)/7 */
    for (int k = 0; k < 7; ++k) {
        double q = delta - (double)k * (delta - 0.5) / 7.0;
        out16[k] = (float)(-normal_quantile(q) / top);
    }
    out16[7] = 0.0f;
    /* positive half: codes 8..15, probabilities delta - k*(delta-1/2)/8,
     * code 15 for k = 0 down to code 8 for k = 7 */
    for (int k = 0; k < 8; ++k) {
        double p = delta - (double)k * (delta - 0.5) / 8.0;
        out16[15 - k] = (float)(normal_quantile(p) / top);
    }
    return 0;
}

/* ------------------------------------------------------------------------- */
/* O2. Decision thresholds.                                                   */
/* ------------------------------------------------------------------------- */
/* Reading: a value takes the nearest level (the plainest reading of mapping a
 * weight onto one of the 16 values); an exact tie goes to the lower code.
 * Threshold t_i is the midpoint of levels i and i+1, computed exactly in fp64
 * (the sum of two fp32 values and a halving are exact there) and rounded
 * toward minus infinity to fp32.  With that rounding, "t_i < s" for an fp32 s
 * holds exactly when s lies above the true midpoint. */
static float round_down_to_f32(double x)
{
    float f = (float)x;                 /* round to nearest */
    if ((double)f > x) f = nextafterf(f, -INFINITY);
    return f;
}

void nf4o_thresholds(float out15[15])
{
    float v[16];
    nf4o_levels(v);
    for (int i = 0; i < 15; ++i)
        out15[i] = round_down_to_f32(((double)v[i] + (double)v[i + 1]) / 2.0);
}

/* ------------------------------------------------------------------------- */
/* 16-bit storage formats.                                                    */
/* ------------------------------------------------------------------------- */
static float bits_to_f32(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }

/* bf16 is the top half of an fp32; fp16 is IEEE binary16 (1, 5, 10). */
float nf4o_from16(uint16_t h, int dtype)
{
    if (dtype == NF4O_BF16) return bits_to_f32((uint32_t)h << 16);
    int sign = h >> 15, e = (h >> 10) & 31, m = h & 1023;
    double v;
    if (e == 0)       v = ldexp((double)m, -24);                 /* subnormal */
    else if (e == 31) v = m ? NAN : INFINITY;
    else              v = ldexp((double)(1024 + m), e - 25);
    return (float)(sign ? -v : v);
}

/* Round an fp32 value to the nearest value of the 16-bit format, ties to the
 * even significand, with gradual underflow and overflow to infinity.  Written
 * from the definition: find the spacing q of the format around |f| (the
 * subnormal spacing below the smallest normal), divide, round to the nearest
 * integer with rint (ties to even under the default rounding mode), multiply
 * back; every step is exact in fp64.  Then encode the bits. */
uint16_t nf4o_to16_rne(float f, int dtype)
{
    const int mant = (dtype == NF4O_BF16) ? 7 : 10;      /* stored fraction bits */
    const int emin = (dtype == NF4O_BF16) ? -126 : -14;  /* smallest normal exponent */
    const int bias = (dtype == NF4O_BF16) ? 127 : 15;
    const int emax = (dtype == NF4O_BF16) ? 127 : 15;
    uint16_t sign = signbit(f) ? 0x8000u : 0u;
    double v = fabs((double)f);
    assert(!isnan(f));
    if (isinf(f)) return sign | (uint16_t)(((1 << (15 - mant)) - 1) << mant);
    if (v == 0.0) return sign;
    int e = ilogb(v);
    if (e < emin) e = emin;
    double q = ldexp(1.0, e - mant);
    double r = rint(v / q) * q;
    if (r >= ldexp(1.0, emax + 1))                       /* overflow -> inf */
        return sign | (uint16_t)(((1 << (15 - mant)) - 1) << mant);
    if (r < ldexp(1.0, emin))                            /* subnormal or zero */
        return sign | (uint16_t)(r / ldexp(1.0, emin - mant));
    int re = ilogb(r);
    uint32_t frac = (uint32_t)(r / ldexp(1.0, re - mant)) - (1u << mant);
    return sign | (uint16_t)(((uint32_t)(re + bias) << mant) | frac);
}

void nf4o_to16_rne_array(const float* f, int64_t n, int dtype, uint16_t* out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = nf4o_to16_rne(f[i], dtype);
}

/* ------------------------------------------------------------------------- */
/* O5. Encode one normalised value.                                           */
/* ------------------------------------------------------------------------- */
/* [QLoRA page, How It Works, NF4 item]: a 4-bit number indexes one of the 16
 * values.  Code order is ascending level order; code = #{i : t_i < s}.  Values
 * slightly beyond +-1 (from rounding of the normalisation) saturate to the end
 * codes by themselves. */
/* The thresholds are computed by the caller and passed in (no static table),
 * so the oracle keeps no state between calls and may run on several threads
 * at once, one matrix per thread. */
static int encode_with(const float t[15], float s)
{
    int c = 0;
    for (int i = 0; i < 15; ++i) if (t[i] < s) ++c;
    return c;
}

int nf4o_encode(float s)
{
    float t[15];
    nf4o_thresholds(t);
    return encode_with(t, s);
}

void nf4o_encode_array(const float* s, int64_t n, uint8_t* out)
{
    float t[15];
    nf4o_thresholds(t);
    for (int64_t i = 0; i < n; ++i) out[i] = (uint8_t)encode_with(t, s[i]);
}

/* ------------------------------------------------------------------------- */
/* O3-O6. Blockwise absmax quantisation and packing.                          */
/* ------------------------------------------------------------------------- */
/* [QLoRA page, The Idea / How It Works]: the frozen base weights are stored
 * as 4-bit values plus quantisation constants; [QLoRA explained, Double
 * Quantization]: the constants map the compressed values back to their
 * numerical range.  Reading: one constant per block of 64 consecutive
 * elements of the flattened (row-major) matrix, the block's largest |x|
 * (blocks may straddle rows; the last block may be partial).
 *
 * Normalisation reading: s = fl32(x * fl32(1/a)).  a = 0: every code is the
 * zero level (7).  For a below the smallest normal fp32 (only subnormal bf16
 * blocks) x and a are first scaled by 2^64, which is exact and keeps 1/a
 * finite.
 *
 * Packing reading: element 2j in the low nibble of byte j, 2j+1 in the high
 * nibble; an odd final element leaves the high nibble 0. */
void nf4o_quantize(const uint16_t* w, int64_t n, int dtype,
                   uint8_t* codes, float* absmax)
{
    const int64_t nb = (n + NF4O_BLOCK - 1) / NF4O_BLOCK;
    float t[15];
    nf4o_thresholds(t);
    memset(codes, 0, (size_t)((n + 1) / 2));
    for (int64_t b = 0; b < nb; ++b) {
        const int64_t lo = b * NF4O_BLOCK;
        const int64_t hi = (lo + NF4O_BLOCK < n) ? lo + NF4O_BLOCK : n;
        float a = 0.0f;
        for (int64_t i = lo; i < hi; ++i) {
            float ax = fabsf(nf4o_from16(w[i], dtype));
            assert(isfinite(ax));
            if (ax > a) a = ax;
        }
        absmax[b] = a;
        float scale = 1.0f, r = 0.0f;
        if (a > 0.0f) {
            if (a < 0x1p-126f) scale = 0x1p64f;
            r = 1.0f / (a * scale);
        }
        for (int64_t i = lo; i < hi; ++i) {
            int c;
            if (a == 0.0f) {
                c = 7;
            } else {
                float x = nf4o_from16(w[i], dtype) * scale;
                float s = x * r;
                c = encode_with(t, s);
            }
            codes[i >> 1] |= (uint8_t)(c << ((i & 1) * 4));
        }
    }
}

/* ------------------------------------------------------------------------- */
/* O7. Double quantisation of the absmax constants.                           */
/* ------------------------------------------------------------------------- */
/* [QLoRA page, How It Works, Double Quantization item]: the quantisation
 * constants are themselves quantised (saving about 0.37 bit per parameter);
 * [QLoRA explained, Double Quantization].  Reading: per matrix, groups of 256
 * consecutive absmax values (the last may be partial); G = the group's
 * largest absmax; scale2 = fl32(G/127); each absmax becomes the int8
 * rint(fl32(a/scale2)) clamped to [-127, 127] (ties to even); G = 0 gives
 * scale2 = 0 and all-zero int8 values.  No mean offset. */
void nf4o_double_quant(const float* absmax, int64_t nb,
                       int8_t* qabsmax, float* scale2)
{
    const int64_t ng = (nb + NF4O_DQ_GROUP - 1) / NF4O_DQ_GROUP;
    for (int64_t g = 0; g < ng; ++g) {
        const int64_t lo = g * NF4O_DQ_GROUP;
        const int64_t hi = (lo + NF4O_DQ_GROUP < nb) ? lo + NF4O_DQ_GROUP : nb;
        float G = 0.0f;
        for (int64_t b = lo; b < hi; ++b) if (absmax[b] > G) G = absmax[b];
        float s2 = (G > 0.0f) ? G / 127.0f : 0.0f;
        scale2[g] = s2;
        for (int64_t b = lo; b < hi; ++b) {
            if (s2 == 0.0f) { qabsmax[b] = 0; continue; }
            float q = rintf(absmax[b] / s2);
            if (q > 127.0f) q = 127.0f;
            if (q < -127.0f) q = -127.0f;
            qabsmax[b] = (int8_t)q;
        }
    }
}

/* ------------------------------------------------------------------------- */
/* O8. Dequantisation.                                                        */
/* ------------------------------------------------------------------------- */
/* [QLoRA page, How It Works]: the 4-bit weights are turned back into 16-bit
 * values for the forward and backward pass; [AQLoRA abstract]: QLoRA does this
 * for every 4-bit weight.  y = RNE16(fl32(level[code] * a')), where a' is the
 * exact absmax, or fl32(q * scale2) when the constants were double-quantised.
 * The 16-bit type is that of the input matrix. */
void nf4o_dequantize(const uint8_t* codes, int64_t n, int dtype,
                     const float* absmax, const int8_t* qabsmax,
                     const float* scale2, uint16_t* out)
{
    float v[16];
    nf4o_levels(v);
    for (int64_t i = 0; i < n; ++i) {
        const int64_t b = i / NF4O_BLOCK;
        float ad = qabsmax ? (float)qabsmax[b] * scale2[b / NF4O_DQ_GROUP]
                           : absmax[b];
        int c = (codes[i >> 1] >> ((i & 1) * 4)) & 15;
        out[i] = nf4o_to16_rne(v[c] * ad, dtype);
    }
}

/* ------------------------------------------------------------------------- */
/* O9. Reconstruction error.                                                  */
/* ------------------------------------------------------------------------- */
/* [AQLoRA abstract]: layers are ranked by NF4 reconstruction error.  Reading:
 * the sum over the matrix of (x - y)^2, x the input and y its dequantised
 * value.  Each difference and square is exact in fp64; the sum uses fp64
 * with Neumaier's compensation. */
double nf4o_sse(const uint16_t* w, const uint16_t* y, int64_t n, int dtype)
{
    double sum = 0.0, comp = 0.0;
    for (int64_t i = 0; i < n; ++i) {
        double d = (double)nf4o_from16(w[i], dtype) - (double)nf4o_from16(y[i], dtype);
        double t = d * d;
        double s = sum + t;
        if (fabs(sum) >= fabs(t)) comp += (sum - s) + t;
        else                      comp += (t - s) + sum;
        sum = s;
    }
    return sum + comp;
}

/* [AQLoRA abstract]: one pass over the weights per matrix -- quantise,
 * (double-quantise), dequantise with the constants the user gets back, and
 * score.  The codes always use the exact absmax; dequantisation and the error
 * use the double-quantised absmax when dq is on. */
double nf4o_layer_error(const uint16_t* w, int64_t n, int dtype, int dq,
                        uint8_t* codes, float* absmax, int8_t* qabsmax,
                        float* scale2, uint16_t* y)
{
    const int64_t nb = (n + NF4O_BLOCK - 1) / NF4O_BLOCK;
    nf4o_quantize(w, n, dtype, codes, absmax);
    if (dq) {
        nf4o_double_quant(absmax, nb, qabsmax, scale2);
        nf4o_dequantize(codes, n, dtype, absmax, qabsmax, scale2, y);
    } else {
        nf4o_dequantize(codes, n, dtype, absmax, NULL, NULL, y);
    }
    return nf4o_sse(w, y, n, dtype);
}

/* ------------------------------------------------------------------------- */
/* O10. Storage and promotion cost.                                           */
/* ------------------------------------------------------------------------- */
/* [AQLoRA abstract]: the quality setting costs 0.2 GiB more memory than
 * QLoRA, i.e. the budget counts the extra bytes of keeping a matrix in 16-bit
 * over its NF4 form.  NF4 form: ceil(n/2) code bytes plus either 4 bytes per
 * block (fp32 absmax) or 1 byte per block plus 4 bytes per group of 256
 * blocks (double-quantised). */
int64_t nf4o_storage_bytes(int64_t n, int dq)
{
    const int64_t nb = (n + NF4O_BLOCK - 1) / NF4O_BLOCK;
    const int64_t ng = (nb + NF4O_DQ_GROUP - 1) / NF4O_DQ_GROUP;
    return (n + 1) / 2 + (dq ? nb + 4 * ng : 4 * nb);
}

int64_t nf4o_promote_cost(int64_t n, int dq) { return 2 * n - nf4o_storage_bytes(n, dq); }

/* ------------------------------------------------------------------------- */
/* O11. Budgeted top-K.                                                       */
/* ------------------------------------------------------------------------- */
/* [AQLoRA abstract]: rank layers by reconstruction error and keep the top-K in
 * 16-bit under a memory budget; [AQLoRA summary, Technical Details]: the
 * budget is configurable.  Reading: order by error descending, equal errors
 * by index ascending; walk that order and stop at the first layer whose cost
 * would take the running total over the budget, or when the count cap is
 * reached. */
typedef struct { double err; int idx; } rank_item;

static int rank_cmp(const void* pa, const void* pb)
{
    const rank_item* a = (const rank_item*)pa;
    const rank_item* b = (const rank_item*)pb;
    if (a->err > b->err) return -1;
    if (a->err < b->err) return 1;
    return (a->idx > b->idx) - (a->idx < b->idx);
}

int nf4o_select_topk(const double* err, const int64_t* cost, int nl,
                     int64_t budget, int kcap, uint8_t* selected)
{
    rank_item* order = (rank_item*)malloc(sizeof(rank_item) * (size_t)(nl > 0 ? nl : 1));
    for (int i = 0; i < nl; ++i) {
        assert(!isnan(err[i]));
        order[i].err = err[i];
        order[i].idx = i;
    }
    qsort(order, (size_t)nl, sizeof(rank_item), rank_cmp);
    int K = 0;
    int64_t total = 0;
    while (K < nl && (kcap < 0 || K < kcap)) {
        int64_t next = total + cost[order[K].idx];
        if (budget >= 0 && next > budget) break;
        total = next;
        ++K;
    }
    memset(selected, 0, (size_t)nl);
    for (int j = 0; j < K; ++j) selected[order[j].idx] = 1;
    free(order);
    return K;
}

/* ------------------------------------------------------------------------- */
/* Selection variants (scores, budget rule, granularity).                     */
/* ------------------------------------------------------------------------- */
/* Squared norm of a matrix, sum of x^2 in fp64 with Neumaier compensation:
 * the denominator of the relative score SSE / ||W||^2.  [AQLoRA abstract]
 * ranks by reconstruction error without saying whether it is normalised;
 * the normalised forms are variants of that score. */
double nf4o_sumsq(const uint16_t* w, int64_t n, int dtype)
{
    double sum = 0.0, comp = 0.0;
    for (int64_t i = 0; i < n; ++i) {
        double x = (double)nf4o_from16(w[i], dtype);
        double t = x * x;
        double s = sum + t;
        if (fabs(sum) >= fabs(t)) comp += (sum - s) + t;
        else                      comp += (t - s) + sum;
        sum = s;
    }
    return sum + comp;
}

/* [AQLoRA abstract] keeps the top-K under a memory budget; a speed setting
 * adapts only the top blocks.  Readings of the variants:
 *   score of layer i = err[i] / denom[i] when denom is given (denom = n gives
 *     the mean squared error, denom = sum of squares the relative error), else
 *     err[i]; the division is IEEE fp64;
 *   units: single layers, or groups of consecutive layers (group g = layers
 *     group_end[g-1] .. group_end[g]-1, group_end[-1] = 0), a group's score
 *     being the sum of its layers' scores in layer order and its cost the sum
 *     of their costs -- a transformer block promoted as a whole;
 *   order: score descending, equal scores by unit index ascending;
 *   rule 0 (prefix): take units in that order, stop at the first that would
 *     take the running cost over the budget;
 *   rule 1 (fill): take every unit, in that order, that still fits, skipping
 *     the ones that do not;
 *   at most kcap units (kcap < 0: no cap); budget < 0: no byte budget.
 * Writes selected[nl] per layer and returns the number of units taken. */
int nf4o_select(const double* err, const double* denom, const int64_t* cost, int nl,
                const int32_t* group_end, int ngroups, int64_t budget, int kcap, int rule,
                uint8_t* selected)
{
    const int nu = group_end ? ngroups : nl;
    rank_item* order = (rank_item*)malloc(sizeof(rank_item) * (size_t)(nu > 0 ? nu : 1));
    int64_t* ucost = (int64_t*)malloc(sizeof(int64_t) * (size_t)(nu > 0 ? nu : 1));
    uint8_t* take = (uint8_t*)calloc((size_t)(nu > 0 ? nu : 1), 1);
    for (int u = 0; u < nu; ++u) {
        int b = group_end ? (u ? group_end[u - 1] : 0) : u;
        int e = group_end ? group_end[u] : u + 1;
        double score = 0.0;
        int64_t c = 0;
        for (int i = b; i < e; ++i) {
            double s = denom ? err[i] / denom[i] : err[i];
            assert(!isnan(s));
            score += s;
            c += cost[i];
        }
        order[u].err = score;
        order[u].idx = u;
        ucost[u] = c;
    }
    qsort(order, (size_t)nu, sizeof(rank_item), rank_cmp);
    int K = 0;
    int64_t total = 0;
    for (int r = 0; r < nu; ++r) {
        if (kcap >= 0 && K >= kcap) break;
        int u = order[r].idx;
        int64_t next = total + ucost[u];
        if (budget >= 0 && next > budget) {
            if (rule == 0) break;
            continue;
        }
        total = next;
        take[u] = 1;
        ++K;
    }
    for (int u = 0; u < nu; ++u) {
        int b = group_end ? (u ? group_end[u - 1] : 0) : u;
        int e = group_end ? group_end[u] : u + 1;
        for (int i = b; i < e; ++i) selected[i] = take[u];
    }
    free(order);
    free(ucost);
    free(take);
    return K;
}

/* ------------------------------------------------------------------------- */
/* Codec variants: block size and the kind of second-level quantisation.      */
/* ------------------------------------------------------------------------- */
/* [QLoRA page, How It Works, Double Quantization item] and [QLoRA explained,
 * Double Quantization] say only that the constants are quantised again.
 * Readings of the variants:
 *   block: 32, 64, 128 or 256 consecutive weights share one absmax (the
 *     encode rule is unchanged);
 *   kind 0: no second level (fp32 absmax);
 *   kind 1: int8, symmetric, per group of 256 blocks (the main reading);
 *   kind 2: int8 of the absmax minus the matrix's mean absmax mu, per group:
 *     c = fl32(a - mu), G = max |c|, s2 = fl32(G/127), q = clamp(rint(fl32(c/s2)),
 *     -127, 127), a' = fl32(fl32(q * s2) + mu);
 *   kind 3: as kind 2 with an 8-bit float (E4M3: 4 exponent bits, bias 7,
 *     3 mantissa bits, largest 448, no infinities) in place of the int8:
 *     s2 = fl32(G/448), q = E4M3 nearest (ties to even) of fl32(c/s2).
 *   mu = fl32(S / nb), S the fp64 sum, in group order, of each group's fp64
 *     sum of its absmax values in block order.
 * Codes always use the exact absmax; dequantisation and the error use a'. */

/* E4M3 byte -> value (the encodings with exponent 15 and mantissa 7 are NaN
 * and never produced here). */
float nf4o_e4m3_decode(uint8_t b)
{
    const int e = (b >> 3) & 15, m = b & 7;
    float v = (e == 0) ? (float)m * 0x1p-9f : ldexpf(1.0f + (float)m / 8.0f, e - 7);
    return (b & 0x80) ? -v : v;
}

/* Nearest E4M3 value of v (|v| <= 448), ties to the even encoding: a plain
 * search over the 127 finite magnitudes; a negative value that rounds to zero
 * gives -0. */
uint8_t nf4o_e4m3_encode(float v)
{
    const float a = fabsf(v);
    assert(a <= 448.0f);
    int best = 0;
    double bd = fabs((double)a - (double)nf4o_e4m3_decode(0));
    for (int c = 1; c <= 0x7e; ++c) {
        const double d = fabs((double)a - (double)nf4o_e4m3_decode((uint8_t)c));
        if (d < bd || (d == bd && (c & 1) == 0 && (best & 1) == 1)) { best = c; bd = d; }
    }
    return (uint8_t)(best | (signbit(v) ? 0x80 : 0));   /* the sign is kept, as IEEE rounding does */
}

int64_t nf4o_storage_bytes_ex(int64_t n, int block, int kind)
{
    const int64_t nb = (n + block - 1) / block;
    const int64_t ng = (nb + NF4O_DQ_GROUP - 1) / NF4O_DQ_GROUP;
    return (n + 1) / 2 + (kind == 0 ? 4 * nb : nb + 4 * ng + (kind >= 2 ? 4 : 0));
}

double nf4o_layer_error_ex(const uint16_t* w, int64_t n, int dtype, int block, int kind,
                           uint8_t* codes, float* absmax, uint8_t* q, float* scale2,
                           float* mean, uint16_t* y)
{
    const int64_t nb = (n + block - 1) / block;
    const int64_t ng = (nb + NF4O_DQ_GROUP - 1) / NF4O_DQ_GROUP;
    float t[15];
    nf4o_thresholds(t);
    /* blockwise absmax and codes, exactly as nf4o_quantize with another block */
    memset(codes, 0, (size_t)((n + 1) / 2));
    for (int64_t b = 0; b < nb; ++b) {
        const int64_t lo = b * block, hi = (lo + block < n) ? lo + block : n;
        float a = 0.0f;
        for (int64_t i = lo; i < hi; ++i) {
            const float ax = fabsf(nf4o_from16(w[i], dtype));
            if (ax > a) a = ax;
        }
        absmax[b] = a;
        float scale = 1.0f, r = 0.0f;
        if (a > 0.0f) {
            if (a < 0x1p-126f) scale = 0x1p64f;
            r = 1.0f / (a * scale);
        }
        for (int64_t i = lo; i < hi; ++i) {
            const int c = (a == 0.0f) ? 7 : encode_with(t, (nf4o_from16(w[i], dtype) * scale) * r);
            codes[i >> 1] |= (uint8_t)(c << ((i & 1) * 4));
        }
    }
    /* the dequantised constants */
    float* ad = (float*)malloc(sizeof(float) * (size_t)(nb > 0 ? nb : 1));
    float mu = 0.0f;
    if (kind >= 2) {
        double S = 0.0;
        for (int64_t g = 0; g < ng; ++g) {
            double sg = 0.0;
            for (int64_t b = g * NF4O_DQ_GROUP; b < nb && b < (g + 1) * NF4O_DQ_GROUP; ++b)
                sg += (double)absmax[b];
            S += sg;
        }
        mu = (float)(S / (double)nb);
    }
    if (mean) *mean = mu;
    for (int64_t g = 0; g < ng; ++g) {
        const int64_t lo = g * NF4O_DQ_GROUP, hi = (lo + NF4O_DQ_GROUP < nb) ? lo + NF4O_DQ_GROUP : nb;
        if (kind == 0) {
            for (int64_t b = lo; b < hi; ++b) ad[b] = absmax[b];
            continue;
        }
        float G = 0.0f;
        for (int64_t b = lo; b < hi; ++b) {
            const float c = kind == 1 ? absmax[b] : absmax[b] - mu;
            if (fabsf(c) > G) G = fabsf(c);
        }
        const float s2 = (G > 0.0f) ? G / (kind == 3 ? 448.0f : 127.0f) : 0.0f;
        scale2[g] = s2;
        for (int64_t b = lo; b < hi; ++b) {
            const float c = kind == 1 ? absmax[b] : absmax[b] - mu;
            if (kind == 3) {
                float v = (s2 > 0.0f) ? c / s2 : 0.0f;
                if (v > 448.0f) v = 448.0f;
                if (v < -448.0f) v = -448.0f;
                q[b] = nf4o_e4m3_encode(v);
                ad[b] = nf4o_e4m3_decode(q[b]) * s2 + mu;
            } else {
                float qf = (s2 > 0.0f) ? rintf(c / s2) : 0.0f;
                if (qf > 127.0f) qf = 127.0f;
                if (qf < -127.0f) qf = -127.0f;
                q[b] = (uint8_t)(int8_t)qf;
                ad[b] = (float)(int8_t)q[b] * s2;
                if (kind == 2) ad[b] = ad[b] + mu;
            }
        }
    }
    /* dequantise and score */
    float v[16];
    nf4o_levels(v);
    for (int64_t i = 0; i < n; ++i) {
        const int c = (codes[i >> 1] >> ((i & 1) * 4)) & 15;
        y[i] = nf4o_to16_rne(v[c] * ad[i / block], dtype);
    }
    free(ad);
    return nf4o_sse(w, y, n, dtype);
}
