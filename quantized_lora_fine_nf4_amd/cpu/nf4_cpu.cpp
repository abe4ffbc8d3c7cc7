/*
 * nf4_cpu.cpp -- the fused NF4 scoring pass on the host CPU, multi-threaded.
 *
 * AQLoRA sets everything with one CPU pass over the weights, taking seconds
 * ("AQLoRA" arXiv listing, English abstract; "AQLoRA: A Zero-Search
 * Recipe...", TL;DR).  This is that pass written for the host cores: the same
 * outputs as nf4_layer_error (codes, block absmax, int8 double-quantised
 * absmax and fp32 scales bit for bit; the per-matrix reconstruction error),
 * computed per 16384-weight tile (one double-quantisation group) on a pool of
 * OpenMP threads, with the loops laid out for the compiler's vectoriser.  It
 * is a separate entry point for comparison with the GPU pass, not a fallback:
 * the GPU calls never reach it.
 *
 * Definitions (same readings as the GPU path):
 *   a = max |x| over a 64-weight block; a = 0 -> codes 7;
 *   a < 2^-126 -> x and a scaled by 2^64 first;
 *   s = fl32(x * fl32(1/a)); code = #{i : t_i < s} over the 15 thresholds;
 *   double quant per 256 blocks: s2 = fl32(G/127), q = rint(fl32(a/s2)),
 *   a' = fl32(q * s2); y = RNE16(fl32(level[code] * a')); err = sum (x - y)^2.
 * The squares are summed in fp64 (exact differences, no over- or underflow),
 * per tile in element order, and the tiles of a matrix in tile order.
 */
#include "nf4_cpu.h"

#include <math.h>
#include <omp.h>
#include <stdlib.h>
#include <string.h>

#include "nf4_format.h"

namespace {

enum { BLOCK = 64, GROUP = 256, TILE = BLOCK * GROUP };

static float bits_f(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t f_bits(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

static float g_lv[16], g_thr[15];

template <int DT>
static float from16(uint16_t h)
{
    if (DT == NF4_BF16) return bits_f((uint32_t)h << 16);
    /* fp16 -> fp32, exact */
    const uint32_t s = (uint32_t)(h & 0x8000u) << 16, e = (h >> 10) & 0x1f, m = h & 0x3ff;
    if (e == 0) {
        const float v = (float)m * 0x1p-24f;   /* subnormal (exact) */
        return s ? -v : v;
    }
    if (e == 31) return bits_f(s | 0x7f800000u | (m << 13));
    return bits_f(s | ((e + 112) << 23) | (m << 13));
}

/* fp32 -> 16-bit, round to nearest even (finite inputs) */
template <int DT>
static uint16_t to16(float f)
{
    const uint32_t u = f_bits(f);
    if (DT == NF4_BF16) return (uint16_t)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
    const uint32_t s = (u >> 16) & 0x8000u;
    const uint32_t a = u & 0x7fffffffu;
    if (a >= 0x477ff000u) return (uint16_t)(s | 0x7c00u);          /* rounds to inf */
    if (a < 0x38800000u) {                                         /* fp16 subnormal or 0 */
        if (a < 0x33000000u) return (uint16_t)s;                   /* below half the smallest */
        const uint32_t e = a >> 23, mant = (a & 0x7fffffu) | 0x800000u;
        const uint32_t shift = 126 - e;                            /* 14..24 */
        uint32_t r = mant >> shift;
        const uint32_t rem = mant & ((1u << shift) - 1u), half = 1u << (shift - 1);
        if (rem > half || (rem == half && (r & 1u))) ++r;
        return (uint16_t)(s | r);
    }
    uint32_t r = a - 0x38000000u;                                  /* rebias exponent */
    r = (r + 0xfffu + ((r >> 13) & 1u)) >> 13;
    return (uint16_t)(s | r);
}

static void init_tables(void)
{
    for (int i = 0; i < 16; ++i) g_lv[i] = bits_f(nf4fmt::kLevelBits[i]);
    for (int i = 0; i < 15; ++i) g_thr[i] = bits_f(nf4fmt::kThresholdBits[i]);
}

/* One tile (up to 256 blocks) of one matrix; returns its squared error. */
template <int DT>
static double tile_pass(const uint16_t* w, int64_t valid, int dq, uint8_t* codes, float* absmax,
                        int8_t* qabs, float* scale2)
{
    const int nbv = (int)((valid + BLOCK - 1) / BLOCK);
    float a[GROUP], adq[GROUP];
    for (int b = 0; b < nbv; ++b) {
        const int64_t e0 = (int64_t)b * BLOCK;
        const int cnt = valid - e0 < BLOCK ? (int)(valid - e0) : BLOCK;
        uint16_t m = 0;
        for (int i = 0; i < cnt; ++i) {
            const uint16_t v = w[e0 + i] & 0x7fffu;
            m = v > m ? v : m;
        }
        a[b] = from16<DT>(m);
        if (absmax) absmax[b] = a[b];
    }
    if (dq) {
        float G = 0.0f;
        for (int b = 0; b < nbv; ++b) G = a[b] > G ? a[b] : G;
        const float s2 = G > 0.0f ? G / 127.0f : 0.0f;
        *scale2 = s2;
        for (int b = 0; b < nbv; ++b) {
            float q = 0.0f;
            if (G > 0.0f) {
                q = rintf(a[b] / s2);
                q = q < -127.0f ? -127.0f : (q > 127.0f ? 127.0f : q);
            }
            qabs[b] = (int8_t)q;
            adq[b] = q * s2;
        }
    } else {
        for (int b = 0; b < nbv; ++b) adq[b] = a[b];
    }

    double err = 0.0;
    for (int b = 0; b < nbv; ++b) {
        const int64_t e0 = (int64_t)b * BLOCK;
        const int cnt = valid - e0 < BLOCK ? (int)(valid - e0) : BLOCK;
        float x[BLOCK];
        uint8_t c[BLOCK];
        for (int i = 0; i < cnt; ++i) x[i] = from16<DT>(w[e0 + i]);
        for (int i = cnt; i < BLOCK; ++i) x[i] = 0.0f;
        if (a[b] == 0.0f) {
            for (int i = 0; i < BLOCK; ++i) c[i] = 7;
        } else {
            float sc = 1.0f, ab = a[b];
            if (ab < 0x1p-126f) { sc = 0x1p64f; ab *= 0x1p64f; }
            const float r = 1.0f / ab;
            for (int i = 0; i < BLOCK; ++i) {
                const float s = (x[i] * sc) * r;
                int k = 0;
                for (int t = 0; t < 15; ++t) k += g_thr[t] < s;
                c[i] = (uint8_t)k;
            }
        }
        for (int i = cnt; i < BLOCK; ++i) c[i] = 0;                /* past the end: 0 */
        for (int j = 0; j < (cnt + 1) / 2; ++j)
            codes[e0 / 2 + j] = (uint8_t)(c[2 * j] | (c[2 * j + 1] << 4));
        /* dequantise with the constant the user gets back, square the differences
           (padding: x = 0, code 7 -> y = 0, nothing added); eight fp64 lanes in a
           fixed order so the loop vectorises and stays deterministic */
        const float k = adq[b];
        int32_t ci[BLOCK];
        for (int i = 0; i < BLOCK; ++i) ci[i] = i < cnt ? c[i] : 7;
        float y[BLOCK];
        for (int i = 0; i < BLOCK; ++i) y[i] = from16<DT>(to16<DT>(g_lv[ci[i]] * k));
        double acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
        for (int i0 = 0; i0 < BLOCK; i0 += 8)
            for (int l = 0; l < 8; ++l) {
                const double d = (double)x[i0 + l] - (double)y[i0 + l];
                acc[l] += d * d;
            }
        err += ((acc[0] + acc[1]) + (acc[2] + acc[3])) + ((acc[4] + acc[5]) + (acc[6] + acc[7]));
    }
    return err;
}

}  // namespace

extern "C" {

nf4_status nf4_cpu_layer_error(const nf4_layer* layers, int32_t nl, nf4_format fmt, double* err,
                               int32_t threads)
{
    if (fmt.blocksize != BLOCK || (fmt.dq_group != 0 && fmt.dq_group != GROUP) ||
        (fmt.dtype != NF4_BF16 && fmt.dtype != NF4_FP16))
        return NF4_E_UNSUPPORTED;
    if (!layers || nl <= 0 || !err) return NF4_E_ARG;
    const int dq = fmt.dq_group != 0;
    int64_t* first = (int64_t*)malloc(sizeof(int64_t) * ((size_t)nl + 1));
    if (!first) return NF4_E_ARG;
    first[0] = 0;
    for (int32_t l = 0; l < nl; ++l) {
        const nf4_layer* L = &layers[l];
        if (L->n <= 0 || L->n >= ((int64_t)1 << 40) || !L->w || !L->codes ||
            (dq ? (!L->qabsmax || !L->scale2) : !L->absmax)) {
            free(first);
            return NF4_E_ARG;
        }
        first[l + 1] = first[l] + (L->n + TILE - 1) / TILE;
    }
    const int64_t ntiles = first[nl];
    double* part = (double*)malloc(sizeof(double) * (size_t)ntiles);
    if (!part) { free(first); return NF4_E_ARG; }
    init_tables();
    if (threads > 0) omp_set_num_threads(threads);
#pragma omp parallel for schedule(dynamic, 8)
    for (int64_t t = 0; t < ntiles; ++t) {
        int32_t lo = 0, hi = nl - 1;                               /* layer of tile t */
        while (lo < hi) {
            const int32_t mid = (lo + hi + 1) / 2;
            if (first[mid] <= t) lo = mid; else hi = mid - 1;
        }
        const nf4_layer* L = &layers[lo];
        const int64_t local = t - first[lo], e0 = local * TILE;
        const int64_t valid = L->n - e0 < TILE ? L->n - e0 : TILE;
        const uint16_t* wt = (const uint16_t*)L->w + e0;
        float* am = L->absmax ? L->absmax + e0 / BLOCK : NULL;
        int8_t* qa = dq ? L->qabsmax + e0 / BLOCK : NULL;
        float* s2 = dq ? L->scale2 + local : NULL;
        part[t] = fmt.dtype == NF4_BF16
                      ? tile_pass<NF4_BF16>(wt, valid, dq, L->codes + e0 / 2, am, qa, s2)
                      : tile_pass<NF4_FP16>(wt, valid, dq, L->codes + e0 / 2, am, qa, s2);
    }
    for (int32_t l = 0; l < nl; ++l) {
        double s = 0.0;
        for (int64_t t = first[l]; t < first[l + 1]; ++t) s += part[t];
        err[l] = s;
    }
    free(part);
    free(first);
    return NF4_OK;
}

int32_t nf4_cpu_max_threads(void) { return omp_get_max_threads(); }

}  // extern "C"
