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

// The level and threshold values, decoded from their bit patterns once, when
// the library is loaded (namespace-scope initialisation runs before any call),
// and only read afterwards: concurrent calls share them without a race.
struct Tables {
    float lv[16];
    float thr[15];
};

static Tables make_tables(void)
{
    Tables t;
    for (int i = 0; i < 16; ++i) memcpy(&t.lv[i], &nf4fmt::kLevelBits[i], 4);
    for (int i = 0; i < 15; ++i) memcpy(&t.thr[i], &nf4fmt::kThresholdBits[i], 4);
    return t;
}

static const Tables g_tables = make_tables();
static const float* const g_lv = g_tables.lv;
static const float* const g_thr = g_tables.thr;

// The tile pass, compiled twice: for the portable target (x86-64-v3, AVX2)
// and for AVX-512 (x86-64-v4: measured 25% faster per thread on an EPYC
// host); outputs are the same bit for bit (no reassociation, no contraction).
namespace portable {
#include "nf4_cpu_tile.inc"
}  // namespace portable

#pragma GCC push_options
#pragma GCC target("arch=x86-64-v4")
namespace avx512 {
#include "nf4_cpu_tile.inc"
}  // namespace avx512
#pragma GCC pop_options

// The AVX-512 path when the CPU has it, unless NF4_CPU_ISA=avx2 asks for the
// portable one (read at every call; lets both paths be compared on one host).
static bool use_avx512(void)
{
    const char* isa = getenv("NF4_CPU_ISA");
    if (isa && strcmp(isa, "avx2") == 0) return false;
    __builtin_cpu_init();
    return __builtin_cpu_supports("avx512f") && __builtin_cpu_supports("avx512bw") &&
           __builtin_cpu_supports("avx512dq") && __builtin_cpu_supports("avx512vl") &&
           __builtin_cpu_supports("avx512cd");
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
    const bool wide = use_avx512();
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
        uint8_t* cd = L->codes + e0 / 2;
        if (wide)
            part[t] = fmt.dtype == NF4_BF16 ? avx512::tile_pass<NF4_BF16>(wt, valid, dq, cd, am, qa, s2)
                                            : avx512::tile_pass<NF4_FP16>(wt, valid, dq, cd, am, qa, s2);
        else
            part[t] = fmt.dtype == NF4_BF16 ? portable::tile_pass<NF4_BF16>(wt, valid, dq, cd, am, qa, s2)
                                            : portable::tile_pass<NF4_FP16>(wt, valid, dq, cd, am, qa, s2);
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
