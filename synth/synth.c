/*
 * synth.c -- seeded synthetic weight matrices (input generation only).
 *
 * Shared by the tests, the smoke check and the benchmark; holds none of the
 * codec's arithmetic.  Every layer is reproducible from (config id, layer
 * index) alone and every chunk of 4096 elements from (layer seed, chunk index),
 * so generation parallelises over chunks and any slice can be regenerated.
 *
 * Generators (published definitions):
 *   SplitMix64  -- Steele, Lea, Flood, "Fast splittable pseudorandom number
 *                  generators" (OOPSLA 2014); used for seeding.
 *   xoshiro256** -- Blackman, Vigna, "Scrambled linear pseudorandom number
 *                  generators" (2018); the per-chunk and per-layer streams.
 *   Normal       -- Marsaglia & Bray polar method (1964), both outputs used.
 *   Student-t(4) -- z * sqrt(4 / chi2), chi2 with 4 degrees of freedom drawn
 *                  as -2 ln u1 - 2 ln u2; scaled by sigma / sqrt(2) so the
 *                  standard deviation is sigma.
 *   Outliers     -- round(frac * n) distinct positions by Floyd's sampling
 *                  algorithm (Bentley & Floyd, CACM 1987) from the layer
 *                  stream; the value there is scaled before rounding.
 * The fp64 draws become 16-bit by rounding to fp32 and then truncating toward
 * zero to bf16 or fp16 -- deliberately not the codec's round-to-nearest.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define SYNTH_CHUNK 4096

static uint64_t splitmix64_next(uint64_t* x)
{
    uint64_t z = (*x += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

typedef struct { uint64_t s[4]; } xoshiro;

static inline uint64_t rotl(uint64_t x, int k) { return (x << k) | (x >> (64 - k)); }

static inline uint64_t xo_next(xoshiro* g)
{
    uint64_t* s = g->s;
    const uint64_t result = rotl(s[1] * 5, 7) * 9;
    const uint64_t t = s[1] << 17;
    s[2] ^= s[0]; s[3] ^= s[1]; s[1] ^= s[2]; s[0] ^= s[3];
    s[2] ^= t;
    s[3] = rotl(s[3], 45);
    return result;
}

static void xo_seed(xoshiro* g, uint64_t seed)
{
    uint64_t x = seed;
    for (int i = 0; i < 4; ++i) g->s[i] = splitmix64_next(&x);
}

/* uniform in [0, 1) with 53 random bits */
static inline double uni(xoshiro* g) { return (double)(xo_next(g) >> 11) * 0x1p-53; }

/* uniform integer in [0, m) (multiply-high; bias below 2^-40 for m < 2^24) */
static inline uint64_t uni_int(xoshiro* g, uint64_t m)
{
    return (uint64_t)(((unsigned __int128)xo_next(g) * m) >> 64);
}

uint64_t synth_layer_seed(uint32_t config_id, uint32_t layer_index)
{
    uint64_t x = ((uint64_t)config_id << 32) | layer_index;
    return splitmix64_next(&x);
}

static void polar_pair(xoshiro* g, double* z0, double* z1)
{
    double u, v, s;
    do {
        u = 2.0 * uni(g) - 1.0;
        v = 2.0 * uni(g) - 1.0;
        s = u * u + v * v;
    } while (s >= 1.0 || s == 0.0);
    double f = sqrt(-2.0 * log(s) / s);
    *z0 = u * f;
    *z1 = v * f;
}

/* Per-layer sigma: sigma_lo when sigma_hi <= sigma_lo, else the first draw of
 * the layer stream mapped onto [sigma_lo, sigma_hi). */
double synth_layer_sigma(uint64_t layer_seed, double sigma_lo, double sigma_hi)
{
    if (!(sigma_hi > sigma_lo)) return sigma_lo;
    xoshiro g;
    xo_seed(&g, layer_seed);
    return sigma_lo + (sigma_hi - sigma_lo) * uni(&g);
}

static int cmp_i64(const void* a, const void* b)
{
    int64_t x = *(const int64_t*)a, y = *(const int64_t*)b;
    return (x > y) - (x < y);
}

/* Outlier positions: m distinct positions in [0, n), sorted ascending.  Drawn
 * from the layer stream after the sigma draw.  Returns m. */
int64_t synth_outlier_positions(uint64_t layer_seed, int64_t n, double frac,
                                double sigma_lo, double sigma_hi, int64_t* out)
{
    int64_t m = (int64_t)llround(frac * (double)n);
    if (m <= 0) return 0;
    if (m > n) m = n;
    xoshiro g;
    xo_seed(&g, layer_seed);
    if (sigma_hi > sigma_lo) (void)uni(&g);
    /* open-addressing hash set for Floyd's algorithm */
    uint64_t cap = 1;
    while (cap < (uint64_t)(4 * m)) cap <<= 1;
    int64_t* tab = (int64_t*)malloc(sizeof(int64_t) * cap);
    for (uint64_t i = 0; i < cap; ++i) tab[i] = -1;
    int64_t k = 0;
    for (int64_t j = n - m; j < n; ++j) {
        int64_t t = (int64_t)uni_int(&g, (uint64_t)j + 1);
        int64_t pick = t;
        /* is t already chosen? */
        uint64_t h = ((uint64_t)t * 0x9E3779B97F4A7C15ull) & (cap - 1);
        int found = 0;
        while (tab[h] >= 0) { if (tab[h] == t) { found = 1; break; } h = (h + 1) & (cap - 1); }
        if (found) {
            pick = j;
            h = ((uint64_t)j * 0x9E3779B97F4A7C15ull) & (cap - 1);
            while (tab[h] >= 0) h = (h + 1) & (cap - 1);
        }
        tab[h] = pick;
        out[k++] = pick;
    }
    free(tab);
    qsort(out, (size_t)m, sizeof(int64_t), cmp_i64);
    return m;
}

static uint16_t trunc_bf16(float f)
{
    uint32_t u;
    memcpy(&u, &f, 4);
    return (uint16_t)(u >> 16);
}

static uint16_t trunc_fp16(float f)
{
    uint16_t sign = signbit(f) ? 0x8000u : 0u;
    double a = fabs((double)f);
    if (a >= 65536.0) return sign | 0x7C00u;
    if (a < 0x1p-24) return sign;
    if (a < 0x1p-14) return sign | (uint16_t)floor(a / 0x1p-24);
    int e;
    double m = frexp(a, &e);          /* a = m * 2^e, m in [0.5, 1) */
    int E = e - 1;                    /* a in [2^E, 2^(E+1)) */
    uint32_t frac = (uint32_t)floor((m * 2.0 - 1.0) * 1024.0);
    if (E > 15) return sign | 0x7C00u;
    return sign | (uint16_t)(((uint32_t)(E + 15) << 10) | frac);
}

/*
 * Generate one layer of n elements into out[n] (16-bit patterns).
 *   dist:    0 = normal, 1 = Student-t(4) scaled to standard deviation sigma
 *   sigma:   from synth_layer_sigma(layer_seed, sigma_lo, sigma_hi)
 *   outliers: m = round(outlier_frac * n) positions scaled by outlier_scale
 *   dtype:   0 = bf16, 1 = fp16
 *   first, count: generate only elements [first, first + count) into
 *            out[0 .. count) (first must be a multiple of 4096), so any
 *            chunk-aligned slice can be regenerated alone.
 */
int synth_generate(uint64_t layer_seed, int64_t n, int dist,
                   double sigma_lo, double sigma_hi,
                   double outlier_frac, double outlier_scale, int dtype,
                   int64_t first, int64_t count, uint16_t* out, int nthreads)
{
    if (first % SYNTH_CHUNK != 0 || first < 0 || count < 0 || first + count > n) return -1;
    const double sigma = synth_layer_sigma(layer_seed, sigma_lo, sigma_hi);
    int64_t m = (int64_t)llround(outlier_frac * (double)n);
    if (m < 0) m = 0;
    if (m > n) m = n;
    int64_t* pos = NULL;
    if (m > 0) {
        pos = (int64_t*)malloc(sizeof(int64_t) * (size_t)m);
        m = synth_outlier_positions(layer_seed, n, outlier_frac, sigma_lo, sigma_hi, pos);
    }
    const int64_t c0 = first / SYNTH_CHUNK;
    const int64_t c1 = (first + count + SYNTH_CHUNK - 1) / SYNTH_CHUNK;
    if (nthreads < 1) nthreads = 1;

#pragma omp parallel for schedule(dynamic, 16) num_threads(nthreads)
    for (int64_t c = c0; c < c1; ++c) {
        xoshiro g;
        xo_seed(&g, layer_seed ^ (0xD1B54A32D192ED03ull * (uint64_t)(c + 1)));
        const int64_t lo = c * SYNTH_CHUNK;
        const int64_t hi = (lo + SYNTH_CHUNK < n) ? lo + SYNTH_CHUNK : n;
        /* first outlier at or after lo */
        int64_t oi = 0, ohi = m;
        while (oi < ohi) { int64_t mid = (oi + ohi) / 2; if (pos[mid] < lo) oi = mid + 1; else ohi = mid; }
        double z[2];
        int zleft = 0;
        for (int64_t i = lo; i < hi; ++i) {
            double v;
            if (zleft == 0) { polar_pair(&g, &z[0], &z[1]); zleft = 2; }
            double zz = z[2 - zleft];
            --zleft;
            if (dist == 1) {
                double chi2;
                do chi2 = -2.0 * log(1.0 - uni(&g)) - 2.0 * log(1.0 - uni(&g));
                while (chi2 <= 0.0);
                v = zz * sqrt(4.0 / chi2) * (sigma / sqrt(2.0));
            } else {
                v = zz * sigma;
            }
            if (oi < m && pos[oi] == i) { v *= outlier_scale; ++oi; }
            if (i >= first && i < first + count) {
                float f = (float)v;
                out[i - first] = (dtype == 0) ? trunc_bf16(f) : trunc_fp16(f);
            }
        }
    }
    free(pos);
    return 0;
}
