// k_variants.hip -- codec variants on gfx950: block sizes 32/64/128/256 and
// the kind of second-level quantisation of the absmax constants.
//
// The pages say that the quantisation constants are quantised again ("QLoRA"
// paper summary page, How It Works, Double Quantization item; "QLoRA
// Explained", Double Quantization) without fixing how.  Kinds:
//   0 none: fp32 absmax;
//   1 int8, symmetric, per group of 256 blocks (the main codec's reading);
//   2 int8 of c = fl32(a - mu), mu the matrix's mean absmax:
//     s2 = fl32(max|c| / 127), q = clamp(rint(fl32(c / s2))), a' = fl32(fl32(q s2) + mu);
//   3 as 2 with an E4M3 8-bit float (4 exponent bits, bias 7, 3 mantissa bits,
//     largest 448): s2 = fl32(max|c| / 448), q = nearest E4M3 (ties to even,
//     sign kept) of fl32(c / s2), a' = fl32(fl32(value(q) s2) + mu).
//   mu = fl32(S / nb), S = the fp64 sum, in group order, of each group's fp64
//   sum of its absmax values in block order.
// Codes use the exact absmax (the encode rule of the main codec, with the
// block size changed); the dequantised values and the error use a'.
//
// Work layout: one 256-thread workgroup (4 waves) per group of 256 blocks of
// B weights.  Wave w owns blocks 64w .. 64w+63; in load j lane L reads the 8
// weights at 64wB + 512j + 8L with one 128-bit load, so every load
// instruction of a wave covers 1 KB contiguously and a block's weights sit in
// B/8 neighbouring lanes of one load (its absmax is a cross-lane maximum over
// those lanes).  Per block, thread t of the group does the second level and
// fills an LDS table with the 16 dequantised values of block t; the weights
// are then encoded through a cell table (one compare per weight) and their
// dequantised values looked up in that table for the error.
//
// Launches of the pass: kinds 0 and 1 need nothing outside the group, so one
// kernel computes the absmax and then encodes (holding the group's weights in
// registers for B = 32, re-reading them, mostly from cache, for larger
// blocks).  Kinds 2 and 3 need every absmax of the matrix before any a': an
// absmax kernel (which also writes the group sums), the per-matrix mean, then
// the encode kernel, which reads the weights a second time.  A last small
// kernel adds the group partials of the error per matrix.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "nf4_format.h"
#include "nf4_internal.h"
#include "nf4_launch.h"

namespace nf4k {
namespace {

constexpr int kVThreads = 256;          // = blocks per group
constexpr int kVWaves = kVThreads / 64;
constexpr int kVCells = 129;            // encode cells, trunc(64 s) in [-64, 64]
constexpr int kVRepl = 16;              // lane-indexed copies of the cell table
constexpr int kVYs = 256 + 17;          // dequant table stride (per code), padded against bank conflicts
constexpr int kVarHold = 32;            // largest block size whose group stays in registers (kinds 0/1)

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned short us2 __attribute__((ext_vector_type(2)));
typedef float f2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
#define GLOBAL __attribute__((address_space(1)))

__device__ __forceinline__ float as_f(uint32_t u) { return __builtin_bit_cast(float, u); }
__device__ __forceinline__ uint32_t as_u(float f) { return __builtin_bit_cast(uint32_t, f); }
__device__ __forceinline__ float opaque(float x) { __asm__ volatile("" : "+v"(x)); return x; }

template <int DT>
__device__ __forceinline__ float from16(uint32_t h)
{
    if constexpr (DT == 0) return as_f(h << 16);
    else return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}

template <int DT>
__device__ __forceinline__ void unpack2(uint32_t d, float& lo, float& hi)
{
    if constexpr (DT == 0) {
        lo = as_f(d << 16);
        hi = as_f(d & 0xffff0000u);
    } else {
        lo = (float)__builtin_bit_cast(_Float16, (uint16_t)(d & 0xffffu));
        hi = (float)__builtin_bit_cast(_Float16, (uint16_t)(d >> 16));
    }
}

// fp32 -> 16-bit, nearest even (the product is rounded to fp32 first)
template <int DT>
__device__ __forceinline__ uint32_t to16(float f)
{
    if constexpr (DT == 0) {
        const uint32_t u = as_u(f);
        return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
    } else {
        return __builtin_bit_cast(uint16_t, (_Float16)opaque(f));
    }
}

// two fp32 values -> packed 16-bit pair, nearest even
template <int DT>
__device__ __forceinline__ uint32_t round_pair(float y0, float y1)
{
    if constexpr (DT == 0) {
        f2 in = {y0, y1};
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(in, bf2));
    } else {
        const _Float16 h0 = (_Float16)opaque(y0), h1 = (_Float16)opaque(y1);
        return (uint32_t)__builtin_bit_cast(uint16_t, h0) |
               ((uint32_t)__builtin_bit_cast(uint16_t, h1) << 16);
    }
}

// E4M3 (finite, |v| <= 448): nearest, ties to even, sign kept.  Below 2^-6 the
// values are multiples of 2^-9; above, 8 mantissa steps per binade.  Every
// scaling below is by a power of two, so rint sees the exact value.
__device__ __forceinline__ uint32_t e4m3_encode(float v)
{
    const float a = __builtin_fabsf(v);
    uint32_t code;
    if (a < 0x1p-6f) {
        code = (uint32_t)__builtin_rintf(a * 0x1p9f);            // 0..8 (8 = smallest normal)
    } else {
        int e = __builtin_amdgcn_frexp_expf(a) - 1;              // a in [2^e, 2^(e+1))
        float m8 = __builtin_rintf(__builtin_amdgcn_ldexpf(a, -e) * 8.0f) - 8.0f;   // 0..8
        if (m8 == 8.0f) { m8 = 0.0f; ++e; }
        code = (uint32_t)((e + 7) << 3) | (uint32_t)m8;
    }
    return code | (__builtin_signbitf(v) ? 0x80u : 0u);
}

__device__ __forceinline__ float e4m3_decode(uint32_t q)
{
    const int e = (q >> 3) & 15, m = q & 7;
    const float v = e == 0 ? (float)m * 0x1p-9f : __builtin_amdgcn_ldexpf((float)(8 + m), e - 10);
    return (q & 0x80u) ? -v : v;
}

// The dequantised constant of a block from its stored form.
template <int KIND>
__device__ __forceinline__ float block_adq(float a, uint32_t q, float s2, float mu)
{
    if constexpr (KIND == 0) return a;
    else if constexpr (KIND == 1) return (float)(int8_t)q * s2;
    else if constexpr (KIND == 2) return (float)(int8_t)q * s2 + mu;
    else return e4m3_decode(q) * s2 + mu;
}

// One encode cell.  u = 64 s is cut into cells by truncation toward zero:
// cell k > 0 holds u in [k, k+1), k < 0 holds (k-1, k], k = 0 holds (-1, 1).
// The level gap (>= 0.0796, >= 5.09 in u) is wider than a cell, so at most one
// threshold lies in a cell: code = base + (u > thr), thr = that threshold
// times 64 (or +inf), base = the thresholds strictly below the cell.  u and
// thr are exact scalings by 64 of s and the threshold, so the comparison is
// exactly "threshold < s".
struct alignas(8) VCell {
    float thr;
    uint32_t base;
};

__device__ void build_vcells(VCell* cells)
{
    for (int idx = threadIdx.x; idx < kVCells * kVRepl; idx += kVThreads) {
        const int k = idx / kVRepl - 64;
        const float lo = (k > 0) ? (float)k : (k < 0 ? (float)(k - 1) : -1.0f);
        const float hi = (k > 0) ? (float)(k + 1) : (k < 0 ? (float)k : 1.0f);
        uint32_t base = 0;
        float thr = __builtin_inff();
        for (int i = 0; i < 15; ++i) {
            const float t64 = as_f(nf4fmt::kThresholdBits[i]) * 64.0f;
            if (t64 < lo) ++base;
            else if (t64 <= hi) thr = t64;
        }
        cells[idx] = VCell{thr, base};
    }
}

// ---- cross-lane reductions -----------------------------------------------

template <int CTRL>
__device__ __forceinline__ uint32_t dpp(uint32_t v)
{
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, true);
}

// Maximum over aligned runs of 2^LOG2 lanes (LOG2 = 2..5); every lane of a
// run ends with it: quad xor 1 and xor 2, then the half-row and row mirrors,
// then xor 16.
template <int LOG2>
__device__ __forceinline__ uint32_t run_max(uint32_t v)
{
    v = max(v, dpp<0xB1>(v));
    if constexpr (LOG2 >= 2) v = max(v, dpp<0x4E>(v));
    if constexpr (LOG2 >= 3) v = max(v, dpp<0x141>(v));
    if constexpr (LOG2 >= 4) v = max(v, dpp<0x140>(v));
    if constexpr (LOG2 >= 5) v = max(v, (uint32_t)__shfl_xor((int)v, 16, 64));
    return v;
}

__device__ __forceinline__ uint32_t wave_max(uint32_t v)
{
    v = max(v, dpp<0xB1>(v));
    v = max(v, dpp<0x4E>(v));
    v = max(v, dpp<0x141>(v));
    v = max(v, dpp<0x140>(v));
    const uint32_t a = max((uint32_t)__builtin_amdgcn_readlane((int)v, 0),
                           (uint32_t)__builtin_amdgcn_readlane((int)v, 16));
    const uint32_t b = max((uint32_t)__builtin_amdgcn_readlane((int)v, 32),
                           (uint32_t)__builtin_amdgcn_readlane((int)v, 48));
    return max(a, b);
}

template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v)
{
    const uint64_t u = __builtin_bit_cast(uint64_t, v);
    const uint32_t lo = dpp<CTRL>((uint32_t)u), hi = dpp<CTRL>((uint32_t)(u >> 32));
    return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

// fp64 sum over a wave in a fixed order; valid in every lane
__device__ __forceinline__ double wave_sum(double v)
{
    v += dpp_f64<0xB1>(v);
    v += dpp_f64<0x4E>(v);
    v += dpp_f64<0x141>(v);
    v += dpp_f64<0x140>(v);
    const uint64_t u = __builtin_bit_cast(uint64_t, v);
    double r[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)u, 16 * i);
        const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), 16 * i);
        r[i] = __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
    }
    return (r[0] + r[1]) + (r[2] + r[3]);
}

// largest |x| bit pattern of 8 packed 16-bit values (sign-magnitude formats:
// for non-negative values the integer order is the numeric order)
__device__ __forceinline__ uint32_t absmax_bits8(const u32x4 v)
{
    const uint32_t m = 0x7fff7fffu;
    us2 a = __builtin_bit_cast(us2, v.x & m), b = __builtin_bit_cast(us2, v.y & m);
    us2 c = __builtin_bit_cast(us2, v.z & m), d = __builtin_bit_cast(us2, v.w & m);
    us2 r = __builtin_elementwise_max(__builtin_elementwise_max(a, b),
                                      __builtin_elementwise_max(c, d));
    return r.x > r.y ? (uint32_t)r.x : (uint32_t)r.y;
}

constexpr int ilog2c(int x) { return x <= 1 ? 0 : 1 + ilog2c(x / 2); }

// ---- a group of one matrix --------------------------------------------------

struct VGroup {
    const LayerDesc* d;
    int l;
    int64_t local;   // group index within the matrix
    int64_t e0;      // first element of the group
    int valid;       // elements of the group inside the matrix
    int nbv;         // blocks of the group inside the matrix
};

// The matrix holding group g (binary search over the running group ends).
__device__ __forceinline__ int group_layer(const LayerDesc* tab, int nl, int64_t g)
{
    int lo = 0, hi = nl - 1;
    while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (tab[mid].tile_end > g) hi = mid; else lo = mid + 1;
    }
    return lo;
}

// Group g of matrix l.
template <int B>
__device__ __forceinline__ VGroup vgroup_of(const LayerDesc* tab, int l, int64_t g)
{
    VGroup r;
    r.d = &tab[l];
    r.l = l;
    r.local = g - (l ? tab[l - 1].tile_end : 0);
    r.e0 = r.local * (int64_t)(kVThreads * B);
    const int64_t rem = r.d->n - r.e0;
    r.valid = rem < kVThreads * B ? (int)rem : kVThreads * B;
    r.nbv = (r.valid + B - 1) / B;
    return r;
}

template <int B>
__device__ __forceinline__ VGroup vgroup(const LayerDesc* tab, int nl, int64_t g)
{
    return vgroup_of<B>(tab, group_layer(tab, nl, g), g);
}

// The thread index behind an opaque barrier: offsets derived from it are
// recomputed where they are used instead of being hoisted out of the group
// loop, where one live register per load would spill.
__device__ __forceinline__ uint32_t lane_tid()
{
    uint32_t t = threadIdx.x;
    __asm__ volatile("" : "+v"(t));
    return t;
}

// Element offset (within the group) of this lane's load j: 64 w B + 512 j + 8 L.
template <int B>
__device__ __forceinline__ uint32_t voff(int j)
{
    const uint32_t t = lane_tid();
    return (t >> 6) * (uint32_t)(64 * B) + (uint32_t)j * 512u + (t & 63u) * 8u;
}

// Block (within the group) of this lane's load j.
template <int B>
__device__ __forceinline__ int vblock(int j)
{
    const int t = (int)lane_tid();
    return (t >> 6) * 64 + j * (512 / B) + (t & 63) / (B / 8);
}

// 8 weights at group offset o; past the end of the matrix they read as 0.
// ONCE: the last read of these weights (a group held in registers, or the
// encode's re-read), so the load is non-temporal; a first read that is read
// again keeps its lines cached.
template <bool FULL, bool ONCE = false>
__device__ __forceinline__ u32x4 vload(const GLOBAL uint16_t* w, uint32_t o, int valid)
{
    if (FULL || (int)o + 8 <= valid) {
        if constexpr (ONCE) return __builtin_nontemporal_load((const GLOBAL u32x4*)(w + o));
        else return *(const GLOBAL u32x4*)(w + o);
    }
    uint32_t h[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) h[k] = ((int)o + k < valid) ? (uint32_t)w[o + k] : 0u;
    return u32x4{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16)};
}

// Block absmax of load j's 8 values: the maximum over the block's B/8 lanes;
// the block's first lane writes it (to memory and to s_a).
template <int DT, int B>
__device__ __forceinline__ void absmax_of_load(const u32x4 v, int j, const VGroup& g, float* s_a)
{
    const uint32_t m = run_max<ilog2c(B / 8)>(absmax_bits8(v));
    const int bg = vblock<B>(j);
    if ((threadIdx.x & (B / 8 - 1)) == 0) {
        const float a = from16<DT>(m);
        s_a[bg] = a;
        if (bg < g.nbv) ((GLOBAL float*)g.d->absmax)[g.local * kVThreads + bg] = a;
    }
}

struct VShared {
    VCell cells[kVCells * kVRepl];
    float ytab[16 * kVYs];         // ytab[c kVYs + b] = RNE16(level c * a' of block b), as fp32
    float a[kVThreads];            // exact absmax of each block
    float r64[kVThreads];          // 64 fl32(1 / (a pre)), 0 for a zero block
    float pre[kVThreads];          // 2^64 for a < 2^-60, else 1
    uint32_t wmax[kVWaves];
    double err[kVWaves];
};

// ---- absmax kernel (kinds with the mean): absmax and the group's fp64 sum -----

template <int DT, int B>
__global__ __launch_bounds__(kVThreads) void k_var_absmax(const LayerDesc* __restrict__ tab, int nl,
                                                          double* __restrict__ gsum)
{
    __shared__ float s_a[kVThreads];
    constexpr int NL = B / 8;
    const VGroup g = vgroup<B>(tab, nl, blockIdx.x);
    const GLOBAL uint16_t* w = (const GLOBAL uint16_t*)g.d->w + g.e0;
    if (g.valid == kVThreads * B) {
        // the encode kernel reads the weights again only after the whole stack has
        // streamed through, so nothing is gained by keeping these lines cached;
        // non-temporal loads measured 4.5% faster at B = 256, even at 64, and
        // 0.5% slower at 32
#pragma unroll 4
        for (int j = 0; j < NL; ++j)
            absmax_of_load<DT, B>(vload<true, (B >= 64)>(w, voff<B>(j), g.valid), j, g, s_a);
    } else {
#pragma unroll 4
        for (int j = 0; j < NL; ++j) absmax_of_load<DT, B>(vload<false>(w, voff<B>(j), g.valid), j, g, s_a);
    }
    __syncthreads();
    if (threadIdx.x == 0) {   // the group's sum in block order, fp64
        double s = 0.0;
        for (int i = 0; i < g.nbv; ++i) s += (double)s_a[i];
        gsum[blockIdx.x] = s;
    }
}

// mu of one matrix per wave (64 threads): its group sums added in group
// order.  The wave loads 64 sums at a time; the additions stay sequential
// (every lane does the same ones, reading the sums through readlane).
__global__ __launch_bounds__(64) void k_var_mean(const LayerDesc* __restrict__ tab, int block,
                                                 const double* __restrict__ gsum,
                                                 float* __restrict__ mean)
{
    const int l = blockIdx.x, lane = threadIdx.x;
    const int64_t g0 = l ? tab[l - 1].tile_end : 0, g1 = tab[l].tile_end;
    double S = 0.0;
    for (int64_t c = g0; c < g1; c += 64) {
        const int cnt = (int)min((int64_t)64, g1 - c);
        const double v = lane < cnt ? gsum[c + lane] : 0.0;
        const uint64_t u = __builtin_bit_cast(uint64_t, v);
        for (int i = 0; i < cnt; ++i) {
            const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)u, i);
            const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), i);
            S += __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
        }
    }
    const int64_t nb = (tab[l].n + block - 1) / block;
    if (lane == 0) mean[l] = (float)(S / (double)nb);
}

// ---- encode kernel ---------------------------------------------------------

// Encode load j's 8 weights, store their codes, return their squared errors
// (the same fp64 difference per weight as the definition; past the end of the
// matrix x = 0 and y = +-0, which adds nothing).
// D32: the difference is taken in fp32, where it is exact for kinds 0 and 1:
// y is 0 (difference x), or y has the sign of x and a' lies within a factor
// 2 of a (kind 0: a' = a; kind 1 with q >= 1: a in [s2/2, 3 s2/2] for q = 1 and
// |a' - a| <= s2/2 above), and every nonzero code has |x| >= 0.03 a, so the two
// 16-bit values are within 2^8 of each other in magnitude and their difference
// fits in 24 bits.  Kinds 2 and 3 give no such bound (a small block's a' comes
// from the matrix mean) and keep the fp64 difference.
template <int DT, int B, bool FULL, bool SPEC, bool D32>
__device__ __forceinline__ double encode_load(const VShared& sh, const u32x4 v, int j, const VGroup& g,
                                              GLOBAL uint8_t* cp)
{
    const int lane = threadIdx.x & 63;
    const VCell* cells = sh.cells + (lane & (kVRepl - 1));
    const int bg = vblock<B>(j);
    const uint32_t o = voff<B>(j);
    const float r64 = sh.r64[bg];
    const float pre = SPEC ? sh.pre[bg] : 1.0f;
    const float* yt = sh.ytab + bg;
    const uint32_t dw[4] = {v.x, v.y, v.z, v.w};
    uint32_t pk = 0;
    double acc = 0.0;
#pragma unroll
    for (int k2 = 0; k2 < 4; ++k2) {
        float x[2];
        unpack2<DT>(dw[k2], x[0], x[1]);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const float u = (SPEC ? x[h] * pre : x[h]) * r64;
            const VCell c = cells[((int)u + 64) * kVRepl];
            const uint32_t code = c.base + (u > c.thr ? 1u : 0u);
            const float y = yt[__umul24(code, (uint32_t)kVYs)];
            const double dd = D32 ? (double)(x[h] - y) : (double)x[h] - (double)y;
            acc = __builtin_fma(dd, dd, acc);
            pk |= code << (8 * k2 + 4 * h);
        }
    }
    if (FULL || (int)o + 8 <= g.valid) {
        __builtin_nontemporal_store(pk, (GLOBAL uint32_t*)(cp + (o >> 1)));   // write-once codes
    } else {
        const int rem = g.valid - (int)o;
        if (rem > 0) {
            pk &= (1u << (4 * rem)) - 1u;
#pragma unroll
            for (int bb = 0; bb < 4; ++bb)
                if (2 * bb < rem) cp[(o >> 1) + bb] = (uint8_t)(pk >> (8 * bb));
        }
    }
    // keep the scheduler from hoisting the next load's lookups (register pressure)
    __builtin_amdgcn_sched_barrier(0);
    return acc;
}

template <int B>
struct Held {
    u32x4 v[(B <= kVarHold) ? B / 8 : 1];
};

template <int DT, int B, bool FULL, bool SPEC, bool HOLD, bool D32>
__device__ __forceinline__ double encode_group(const VShared& sh, const Held<B>& held,
                                               const GLOBAL uint16_t* w, const VGroup& g,
                                               GLOBAL uint8_t* cp)
{
    constexpr int NL = B / 8;
    double acc = 0.0;
    if constexpr (HOLD) {
#pragma unroll
        for (int j = 0; j < NL; ++j) acc += encode_load<DT, B, FULL, SPEC, D32>(sh, held.v[j], j, g, cp);
    } else {
        // last loads first: for the kinds that read the group a second time,
        // what the absmax pass loaded last is the likeliest still in cache
        constexpr int BATCH = 4;
        static_assert(NL % BATCH == 0, "loads come in batches of 4");
#pragma nounroll
        for (int j0 = NL - BATCH; j0 >= 0; j0 -= BATCH) {
            u32x4 v[BATCH];
#pragma unroll
            for (int i = 0; i < BATCH; ++i) v[i] = vload<FULL, true>(w, voff<B>(j0 + i), g.valid);
#pragma unroll
            for (int i = 0; i < BATCH; ++i) acc += encode_load<DT, B, FULL, SPEC, D32>(sh, v[i], j0 + i, g, cp);
        }
    }
    return acc;
}

// Kinds 0/1 compute the absmax here; kinds 2/3 read it (from k_var_absmax).
template <int DT, int B, int KIND, bool FULL>
__device__ __forceinline__ void var_codec_body(VShared& sh, const VGroup& g, int64_t gi,
                                               const float* mean, double* partial)
{
    constexpr bool FUSED = KIND <= 1;
    constexpr bool HOLD = FUSED && B <= kVarHold;
    constexpr int NL = B / 8;
    const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
    const LayerDesc& d = *g.d;
    const GLOBAL uint16_t* w = (const GLOBAL uint16_t*)d.w + g.e0;
    GLOBAL uint8_t* cp = (GLOBAL uint8_t*)d.codes + (g.e0 >> 1);

    // 1. the exact absmax of every block
    Held<B> held;
    if constexpr (FUSED) {
        if constexpr (HOLD) {
#pragma unroll
            for (int j = 0; j < NL; ++j) held.v[j] = vload<FULL, true>(w, voff<B>(j), g.valid);
#pragma unroll
            for (int j = 0; j < NL; ++j) absmax_of_load<DT, B>(held.v[j], j, g, sh.a);
        } else {
#pragma unroll 4
            for (int j = 0; j < NL; ++j) absmax_of_load<DT, B>(vload<FULL>(w, voff<B>(j), g.valid), j, g, sh.a);
        }
        __syncthreads();
    }
    const bool in = t < g.nbv;
    const int64_t b = g.local * kVThreads + t;
    float a;
    if constexpr (FUSED) a = sh.a[t];
    else a = in ? ((const GLOBAL float*)d.absmax)[b] : 0.0f;

    // 2. second level of block t: group maximum of |c|, scale, stored byte, a'
    float adq = a;
    if constexpr (KIND != 0) {
        const float mu = (KIND >= 2) ? mean[g.l] : 0.0f;
        const float c = (KIND >= 2) ? a - mu : a;
        const uint32_t wm = wave_max(in ? as_u(__builtin_fabsf(c)) : 0u);
        if (lane == 0) sh.wmax[wv] = wm;
        __syncthreads();
        uint32_t gm = sh.wmax[0];
#pragma unroll
        for (int i = 1; i < kVWaves; ++i) gm = max(gm, sh.wmax[i]);
        const float G = as_f(gm);
        float s2 = 0.0f;
        uint32_t q = 0;
        if (G > 0.0f) {
            s2 = G / (KIND == 3 ? 448.0f : 127.0f);
            float v = c / s2;
            if constexpr (KIND == 3) {
                v = min(max(v, -448.0f), 448.0f);
                q = e4m3_encode(v);
            } else {
                const float qf = min(max(__builtin_rintf(v), -127.0f), 127.0f);
                q = (uint32_t)(uint8_t)(int8_t)qf;
            }
        }
        adq = block_adq<KIND>(a, q, s2, mu);
        if (in) ((GLOBAL uint8_t*)d.qabsmax)[b] = (uint8_t)q;
        if (t == 0) ((GLOBAL float*)d.scale2)[g.local] = s2;
    }

    // 3. block t's encode scale and its 16 dequantised values.  A prescale
    //    of 2^64 for a < 2^-60 keeps 64 / a finite; (x 2^64)(64 / (a 2^64))
    //    is the same real product as x (64 / a), so the codes do not change.
    float pre = 1.0f, r64 = 0.0f;
    if (a > 0.0f) {
        if (a < 0x1p-60f) pre = 0x1p64f;
        r64 = 64.0f * opaque(1.0f / (a * pre));
    }
    sh.r64[t] = r64;
    sh.pre[t] = pre;
#pragma unroll
    for (int cc = 0; cc < 16; ++cc)
        sh.ytab[cc * kVYs + t] = from16<DT>(to16<DT>(as_f(nf4fmt::kLevelBits[cc]) * adq));
    const bool spec = __syncthreads_or(pre != 1.0f);

    // 4. encode, store codes, squared error
    constexpr bool D32 = KIND <= 1;
    const double acc = spec ? encode_group<DT, B, FULL, true, HOLD, D32>(sh, held, w, g, cp)
                            : encode_group<DT, B, FULL, false, HOLD, D32>(sh, held, w, g, cp);

    // 5. the group's fp64 partial (waves in order)
    const double ws = wave_sum(acc);
    if (lane == 0) sh.err[wv] = ws;
    __syncthreads();
    if (t == 0) partial[gi] = (sh.err[0] + sh.err[1]) + (sh.err[2] + sh.err[3]);
}

// Persistent: each workgroup builds the cell table once and then walks the
// groups gridDim.x apart.  Between two groups the workgroup passes the
// barrier before the partial is written, after which nothing of the previous
// group is read from LDS except that partial (read by thread 0 before its
// next barrier).
template <int DT, int B, int KIND>
__global__ __launch_bounds__(kVThreads, 4) void k_var_codec(const LayerDesc* __restrict__ tab, int nl,
                                                         int64_t ngroups, const float* __restrict__ mean,
                                                         double* __restrict__ partial)
{
    __shared__ VShared sh;
    build_vcells(sh.cells);
    __syncthreads();
    // the walk's groups only increase, so their matrix is found by stepping
    // forward from the previous one: one table read per group where a binary
    // search per group would chain about log2(matrices) dependent reads
    int l = blockIdx.x < ngroups ? group_layer(tab, nl, blockIdx.x) : 0;
    for (int64_t gi = blockIdx.x; gi < ngroups; gi += gridDim.x) {
        while (tab[l].tile_end <= gi) ++l;
        const VGroup g = vgroup_of<B>(tab, l, gi);
        if (g.valid == kVThreads * B) var_codec_body<DT, B, KIND, true>(sh, g, gi, mean, partial);
        else var_codec_body<DT, B, KIND, false>(sh, g, gi, mean, partial);
    }
}

// ---- standalone dequantisation ---------------------------------------------
//
// A prep kernel writes one 64-byte record per group (its codes, output and
// constants, scale2, the matrix's mean, the valid count); then 64-thread
// workgroups each take 2,048 weights of a group (a unit) with four 16-byte
// stores per thread, every load of a whole unit issued at once -- the shape
// that measured fastest for the main dequantisation.

struct alignas(64) VarDqRec {
    const uint8_t* codes;   // the group's first code byte
    uint16_t* out;          // the group's first output element
    const void* cst;        // the group's first stored constant (byte, or fp32 absmax)
    float s2;               // the group's scale2 (kinds 1-3)
    float mu;               // the matrix's mean absmax (kinds 2-3)
    int32_t valid;          // elements of the group inside the matrix
};
constexpr int kVdThreads = 64;                       // 128 over 4,096 weights: 1-3% slower
constexpr int kVdUnit = 2048;                        // weights per workgroup
constexpr int kVdSteps = kVdUnit / (kVdThreads * 8); // 16-byte stores per thread

template <int B, int KIND>
__global__ __launch_bounds__(256) void k_var_dq_prep(const LayerDesc* __restrict__ tab, int nl,
                                                     int64_t ngroups, const float* __restrict__ mean,
                                                     VarDqRec* __restrict__ rec)
{
    const int64_t gi = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (gi >= ngroups) return;
    const VGroup g = vgroup<B>(tab, nl, gi);
    const LayerDesc& d = *g.d;
    VarDqRec r;
    r.codes = d.codes + (g.e0 >> 1);
    r.out = (uint16_t*)d.out + g.e0;
    const int64_t b0 = g.local * kVThreads;
    r.cst = KIND == 0 ? (const void*)(d.absmax + b0) : (const void*)((const uint8_t*)d.qabsmax + b0);
    r.s2 = KIND == 0 ? 0.0f : ((const GLOBAL float*)d.scale2)[g.local];
    r.mu = KIND >= 2 ? mean[g.l] : 0.0f;
    r.valid = g.valid;
    rec[gi] = r;
}

template <int DT, int B, int KIND>
__global__ __launch_bounds__(kVdThreads) void k_var_dequant(const VarDqRec* __restrict__ rec,
                                                            int64_t first_unit)
{
    constexpr int UPG = kVThreads * B / kVdUnit;   // units per group
    __shared__ float s_lv[kVdThreads / 64][16];
    const int t = threadIdx.x, lane = t & 63;
    float* lv = s_lv[t >> 6];
    if (lane < 16) {   // from immediates: no load before the data loads
        float v = as_f(nf4fmt::kLevelBits[0]);
#pragma unroll
        for (int i = 1; i < 16; ++i) v = lane == i ? as_f(nf4fmt::kLevelBits[i]) : v;
        lv[lane] = v;
    }
    const int64_t unit = first_unit + blockIdx.x;
    const int64_t gi = unit / UPG;
    const int sub = (int)(unit - gi * UPG);
    const VarDqRec r = rec[gi];   // uniform: scalar loads
    const int valid = r.valid - sub * kVdUnit;
    if (valid <= 0) return;       // past the end of a ragged last group (the whole workgroup)
    const GLOBAL uint8_t* cp = (const GLOBAL uint8_t*)r.codes + sub * (kVdUnit / 2);
    GLOBAL uint16_t* out = (GLOBAL uint16_t*)r.out + (int64_t)sub * kVdUnit;
    const int bsub = sub * (kVdUnit / B);          // first block of the unit within the group
    const bool full = valid >= kVdUnit;
    uint32_t cw[kVdSteps];
    uint32_t raw[kVdSteps];
    if (full) {
#pragma unroll
        for (int j = 0; j < kVdSteps; ++j) {
            const uint32_t o = 8u * (j * (uint32_t)kVdThreads + t);
            cw[j] = *(const GLOBAL uint32_t*)(cp + (o >> 1));
            const int bl = bsub + (int)(o / B);
            raw[j] = KIND == 0 ? as_u(((const GLOBAL float*)r.cst)[bl])
                               : (uint32_t)((const GLOBAL uint8_t*)r.cst)[bl];
        }
    } else {
#pragma unroll
        for (int j = 0; j < kVdSteps; ++j) {
            const uint32_t o = 8u * (j * (uint32_t)kVdThreads + t);
            uint32_t c = 0;
            for (int bb = 0; bb < 4; ++bb)
                if ((int)o + 2 * bb < valid) c |= (uint32_t)cp[(o >> 1) + bb] << (8 * bb);
            cw[j] = c;
            const int bl = bsub + (int)(o / B);
            raw[j] = (int)o < valid ? (KIND == 0 ? as_u(((const GLOBAL float*)r.cst)[bl])
                                                 : (uint32_t)((const GLOBAL uint8_t*)r.cst)[bl])
                                    : 0u;
        }
    }
    __builtin_amdgcn_wave_barrier();   // the wave's table writes precede its reads (LDS keeps a wave's order)
#pragma unroll
    for (int j = 0; j < kVdSteps; ++j) {
        const uint32_t o = 8u * (j * (uint32_t)kVdThreads + t);
        if (!full && (int)o >= valid) continue;
        const float adq = KIND == 0 ? as_f(raw[j]) : block_adq<KIND>(0.0f, raw[j], r.s2, r.mu);
        uint32_t p[4];
#pragma unroll
        for (int k2 = 0; k2 < 4; ++k2)
            p[k2] = round_pair<DT>(lv[(cw[j] >> (8 * k2)) & 15] * adq, lv[(cw[j] >> (8 * k2 + 4)) & 15] * adq);
        if (full || (int)o + 8 <= valid) {
            // write-once stream: non-temporal (4-7% faster than cached stores here)
            __builtin_nontemporal_store(u32x4{p[0], p[1], p[2], p[3]}, (GLOBAL u32x4*)(out + o));
        } else {
            for (int k = 0; k < 8; ++k)
                if ((int)o + k < valid) out[o + k] = (uint16_t)(p[k >> 1] >> (16 * (k & 1)));
        }
    }
}

// per-matrix sum of the group partials, one workgroup per matrix (a fixed
// order, so the result does not change from run to run)
__global__ __launch_bounds__(kVThreads) void k_var_reduce(const LayerDesc* __restrict__ tab,
                                                          const double* __restrict__ partial,
                                                          double* __restrict__ err)
{
    __shared__ double s_w[kVWaves];
    const int l = blockIdx.x, t = threadIdx.x;
    const int64_t g0 = l ? tab[l - 1].tile_end : 0, g1 = tab[l].tile_end;
    double acc = 0.0;
    for (int64_t g = g0 + t; g < g1; g += kVThreads) acc += partial[g];
    const double ws = wave_sum(acc);
    if ((t & 63) == 0) s_w[t >> 6] = ws;
    __syncthreads();
    if (t == 0) err[l] = (s_w[0] + s_w[1]) + (s_w[2] + s_w[3]);
}

constexpr int64_t kMaxVGrid = 0x7fffffff;

// Workgroups of the persistent encode launch: the resident count per CU
// times the CUs, at most one per group.
template <typename K>
unsigned codec_grid(K kernel, int64_t ngroups)
{
    int dev = 0, cus = 0, per_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
        cus = 256;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, kVThreads, 0) != hipSuccess ||
        per_cu <= 0)
        per_cu = 1;
    const int64_t g = (int64_t)cus * per_cu;
    return (unsigned)(g < ngroups ? g : ngroups);
}

template <int DT, int B, int KIND>
hipError_t variant_go(const LayerDesc* tab, int nl, int64_t ngroups, float* mean, double* gsum,
                      double* partial, double* err, hipStream_t s)
{
    if (ngroups > kMaxVGrid) return hipErrorInvalidValue;
    const unsigned g = (unsigned)ngroups;
    hipError_t e;
    if constexpr (KIND >= 2) {
        hipLaunchKernelGGL((k_var_absmax<DT, B>), dim3(g), dim3(kVThreads), 0, s, tab, nl, gsum);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        hipLaunchKernelGGL(k_var_mean, dim3(nl), dim3(64), 0, s, tab, B, (const double*)gsum, mean);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    hipLaunchKernelGGL((k_var_codec<DT, B, KIND>), dim3(codec_grid(k_var_codec<DT, B, KIND>, ngroups)),
                       dim3(kVThreads), 0, s, tab, nl, ngroups, (const float*)mean, partial);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(k_var_reduce, dim3(nl), dim3(kVThreads), 0, s, tab, (const double*)partial, err);
    return hipGetLastError();
}

template <int DT, int B, int KIND>
hipError_t variant_dq_go(const LayerDesc* tab, int nl, int64_t ngroups, const float* mean,
                         void* rec_ws, hipStream_t s)
{
    if (ngroups > kMaxVGrid) return hipErrorInvalidValue;
    VarDqRec* rec = static_cast<VarDqRec*>(rec_ws);
    hipLaunchKernelGGL((k_var_dq_prep<B, KIND>), dim3((unsigned)((ngroups + 255) / 256)), dim3(256), 0, s,
                       tab, nl, ngroups, mean, rec);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    constexpr int64_t UPG = kVThreads * B / kVdUnit;
    constexpr int64_t kMaxUnits = (int64_t(1) << 32) / kVdThreads - 1;
    const int64_t nunits = ngroups * UPG;
    for (int64_t u0 = 0; u0 < nunits; u0 += kMaxUnits) {
        const int64_t n = nunits - u0 < kMaxUnits ? nunits - u0 : kMaxUnits;
        hipLaunchKernelGGL((k_var_dequant<DT, B, KIND>), dim3((unsigned)n), dim3(kVdThreads), 0, s,
                           (const VarDqRec*)rec, u0);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    return hipSuccess;
}

template <int DT, int B>
hipError_t variant_kind(const LayerDesc* tab, int nl, int64_t ng, int kind, float* mean, double* gsum,
                        double* partial, double* err, hipStream_t s)
{
    switch (kind) {
        case 0: return variant_go<DT, B, 0>(tab, nl, ng, mean, gsum, partial, err, s);
        case 1: return variant_go<DT, B, 1>(tab, nl, ng, mean, gsum, partial, err, s);
        case 2: return variant_go<DT, B, 2>(tab, nl, ng, mean, gsum, partial, err, s);
        default: return variant_go<DT, B, 3>(tab, nl, ng, mean, gsum, partial, err, s);
    }
}

template <int DT, int B>
hipError_t variant_dq_kind(const LayerDesc* tab, int nl, int64_t ng, int kind, const float* mean,
                           void* rec, hipStream_t s)
{
    switch (kind) {
        case 0: return variant_dq_go<DT, B, 0>(tab, nl, ng, mean, rec, s);
        case 1: return variant_dq_go<DT, B, 1>(tab, nl, ng, mean, rec, s);
        case 2: return variant_dq_go<DT, B, 2>(tab, nl, ng, mean, rec, s);
        default: return variant_dq_go<DT, B, 3>(tab, nl, ng, mean, rec, s);
    }
}

template <int DT>
hipError_t variant_block(const LayerDesc* tab, int nl, int64_t ng, int block, int kind, float* mean,
                         double* gsum, double* partial, double* err, hipStream_t s)
{
    switch (block) {
        case 32: return variant_kind<DT, 32>(tab, nl, ng, kind, mean, gsum, partial, err, s);
        case 64: return variant_kind<DT, 64>(tab, nl, ng, kind, mean, gsum, partial, err, s);
        case 128: return variant_kind<DT, 128>(tab, nl, ng, kind, mean, gsum, partial, err, s);
        case 256: return variant_kind<DT, 256>(tab, nl, ng, kind, mean, gsum, partial, err, s);
        default: return hipErrorInvalidValue;
    }
}

template <int DT>
hipError_t variant_dq_block(const LayerDesc* tab, int nl, int64_t ng, int block, int kind,
                            const float* mean, void* rec, hipStream_t s)
{
    switch (block) {
        case 32: return variant_dq_kind<DT, 32>(tab, nl, ng, kind, mean, rec, s);
        case 64: return variant_dq_kind<DT, 64>(tab, nl, ng, kind, mean, rec, s);
        case 128: return variant_dq_kind<DT, 128>(tab, nl, ng, kind, mean, rec, s);
        case 256: return variant_dq_kind<DT, 256>(tab, nl, ng, kind, mean, rec, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_variant_error(const LayerDesc* tab, int nl, int64_t ngroups, int dtype, int block,
                                int kind, float* mean, double* gsum, double* partial, double* err,
                                hipStream_t s)
{
    if (dtype == 0) return variant_block<0>(tab, nl, ngroups, block, kind, mean, gsum, partial, err, s);
    return variant_block<1>(tab, nl, ngroups, block, kind, mean, gsum, partial, err, s);
}

hipError_t launch_variant_dequant(const LayerDesc* tab, int nl, int64_t ngroups, int dtype,
                                  int block, int kind, const float* mean, void* rec_ws, hipStream_t s)
{
    if (dtype == 0) return variant_dq_block<0>(tab, nl, ngroups, block, kind, mean, rec_ws, s);
    return variant_dq_block<1>(tab, nl, ngroups, block, kind, mean, rec_ws, s);
}

}  // namespace nf4k
