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
// Layout of the work: one 256-thread workgroup per group of 256 blocks, one
// thread per block (its weights contiguous, 16-byte loads and stores), three
// launches for the pass -- absmax and group sums; the per-matrix mean;
// second level, encode, dequantise and the error -- and one for the
// standalone dequantisation.  A variant path: the main codec is the fused
// kernel of k_codec.hip.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "nf4_format.h"
#include "nf4_internal.h"

namespace nf4k {
namespace {

constexpr int kVThreads = 256;   // = blocks per group
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
#define GLOBAL __attribute__((address_space(1)))

__device__ __forceinline__ float as_f(uint32_t u) { return __builtin_bit_cast(float, u); }
__device__ __forceinline__ float opaque(float x) { __asm__ volatile("" : "+v"(x)); return x; }

template <int DT>
__device__ __forceinline__ float from16(uint32_t h)
{
    if constexpr (DT == 0) return as_f(h << 16);
    else return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}

// fp32 -> 16-bit, nearest even (the product is rounded to fp32 first)
template <int DT>
__device__ __forceinline__ uint32_t to16(float f)
{
    if constexpr (DT == 0) {
        const uint32_t u = __builtin_bit_cast(uint32_t, f);
        return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
    } else {
        return __builtin_bit_cast(uint16_t, (_Float16)opaque(f));
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

// A group (tile) of one layer: blocks [256 local, 256 local + 255].
struct VRef {
    const LayerDesc* d;
    int l;
    int64_t local, b0, nb;
};

__device__ __forceinline__ VRef vref(const LayerDesc* tab, int nl, int64_t tile, int block)
{
    int lo = 0, hi = nl - 1;
    while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (tab[mid].tile_end > tile) hi = mid; else lo = mid + 1;
    }
    VRef r;
    r.d = &tab[lo];
    r.l = lo;
    const int64_t first = lo ? tab[lo - 1].tile_end : 0;
    r.local = tile - first;
    r.b0 = r.local * kVThreads;
    r.nb = (r.d->n + block - 1) / block;
    return r;
}

// Weights of block b: count and the absolute maximum (bit pattern of |x|).
template <int DT>
__device__ __forceinline__ uint32_t block_absmax(const GLOBAL uint16_t* w, int cnt)
{
    uint32_t m = 0;
    if (cnt == 0) return 0;
    const int full = cnt & ~7;
    for (int i = 0; i < full; i += 8) {
        const u32x4 v = *(const GLOBAL u32x4*)(w + i);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            m = max(m, v[k] & 0x7fffu);
            m = max(m, (v[k] >> 16) & 0x7fffu);
        }
    }
    for (int i = full; i < cnt; ++i) m = max(m, (uint32_t)(w[i] & 0x7fffu));
    return m;
}

template <int DT>
__global__ __launch_bounds__(kVThreads) void k_var_absmax(const LayerDesc* __restrict__ tab, int nl,
                                                          int block, double* __restrict__ gsum)
{
    __shared__ float s_a[kVThreads];
    const VRef r = vref(tab, nl, blockIdx.x, block);
    const int t = threadIdx.x;
    const int64_t b = r.b0 + t;
    float a = 0.0f;
    if (b < r.nb) {
        const int64_t e0 = b * block;
        const int cnt = (int)min((int64_t)block, r.d->n - e0);
        a = from16<DT>(block_absmax<DT>((const GLOBAL uint16_t*)r.d->w + e0, cnt));
        ((GLOBAL float*)r.d->absmax)[b] = a;
    }
    s_a[t] = a;
    __syncthreads();
    if (t == 0) {   // the group's sum in block order, fp64
        double s = 0.0;
        const int nbv = (int)min((int64_t)kVThreads, r.nb - r.b0);
        for (int i = 0; i < nbv; ++i) s += (double)s_a[i];
        gsum[blockIdx.x] = s;
    }
}

// mu of every layer: its group sums in order, over its block count.
__global__ void k_var_mean(const LayerDesc* __restrict__ tab, int nl, int block,
                           const double* __restrict__ gsum, float* __restrict__ mean)
{
    const int l = blockIdx.x * blockDim.x + threadIdx.x;
    if (l >= nl) return;
    const int64_t g0 = l ? tab[l - 1].tile_end : 0;
    double S = 0.0;
    for (int64_t g = g0; g < tab[l].tile_end; ++g) S += gsum[g];
    const int64_t nb = (tab[l].n + block - 1) / block;
    mean[l] = (float)(S / (double)nb);
}

// The dequantised constant of block b from its stored form.
template <int KIND>
__device__ __forceinline__ float block_adq(float a, uint32_t q, float s2, float mu)
{
    if constexpr (KIND == 0) return a;
    else if constexpr (KIND == 1) return (float)(int8_t)q * s2;
    else if constexpr (KIND == 2) return (float)(int8_t)q * s2 + mu;
    else return e4m3_decode(q) * s2 + mu;
}

template <int DT, int KIND, bool ERR>
__global__ __launch_bounds__(kVThreads) void k_var_codec(const LayerDesc* __restrict__ tab, int nl,
                                                         int block, const float* __restrict__ mean,
                                                         double* __restrict__ partial)
{
    __shared__ float s_red[kVThreads];
    __shared__ double s_err[kVThreads];
    __shared__ float s_lv[16];
    const int t = threadIdx.x;
    if (t < 16) s_lv[t] = as_f(nf4fmt::kLevelBits[t]);
    const VRef r = vref(tab, nl, blockIdx.x, block);
    const LayerDesc& d = *r.d;
    const int64_t b = r.b0 + t;
    const bool in = b < r.nb;
    const float a = in ? ((const GLOBAL float*)d.absmax)[b] : 0.0f;
    const float mu = (KIND >= 2) ? mean[r.l] : 0.0f;

    // second level: group maximum of |c|, scale, the stored byte, a'
    const float c = (KIND >= 2) ? a - mu : a;
    s_red[t] = in ? __builtin_fabsf(c) : 0.0f;
    __syncthreads();
    for (int h = kVThreads / 2; h >= 1; h >>= 1) {
        if (t < h) s_red[t] = max(s_red[t], s_red[t + h]);
        __syncthreads();
    }
    const float G = s_red[0];
    float s2 = 0.0f, adq = a;
    uint32_t q = 0;
    if constexpr (KIND != 0) {
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
        } else if constexpr (KIND == 3) {
            q = 0;   // c / s2 is not formed; every c is 0
        }
        adq = block_adq<KIND>(a, q, s2, mu);
        if (in) ((GLOBAL uint8_t*)d.qabsmax)[b] = (uint8_t)q;
        if (t == 0) ((GLOBAL float*)d.scale2)[r.local] = s2;
    }

    // encode (exact absmax), pack, dequantise with a', squared error in fp64
    double acc = 0.0;
    if (in) {
        const int64_t e0 = b * block;
        const int cnt = (int)min((int64_t)block, d.n - e0);
        const GLOBAL uint16_t* w = (const GLOBAL uint16_t*)d.w + e0;
        GLOBAL uint8_t* cp = (GLOBAL uint8_t*)d.codes + (e0 >> 1);
        float sc = 1.0f, r1 = 0.0f;
        if (a > 0.0f) {
            if (a < 0x1p-126f) sc = 0x1p64f;
            r1 = 1.0f / (a * sc);
        }
        for (int i0 = 0; i0 < cnt; i0 += 8) {
            uint16_t h[8];
            if (i0 + 8 <= cnt) {
                const u32x4 v = *(const GLOBAL u32x4*)(w + i0);
#pragma unroll
                for (int k = 0; k < 4; ++k) { h[2 * k] = (uint16_t)v[k]; h[2 * k + 1] = (uint16_t)(v[k] >> 16); }
            } else {
#pragma unroll
                for (int k = 0; k < 8; ++k) h[k] = (i0 + k < cnt) ? w[i0 + k] : (uint16_t)0;
            }
            uint32_t pk = 0;
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const float x = from16<DT>(h[k]);
                uint32_t code = 7;
                if (a > 0.0f) {
                    const float s = (x * sc) * r1;
                    code = 0;
#pragma unroll
                    for (int j = 0; j < 15; ++j) code += as_f(nf4fmt::kThresholdBits[j]) < s ? 1u : 0u;
                }
                if (i0 + k >= cnt) code = 0;
                pk |= code << (4 * k);
                if constexpr (ERR) {
                    if (i0 + k < cnt) {
                        const float y = from16<DT>(to16<DT>(s_lv[code] * adq));
                        const double dd = (double)x - (double)y;
                        acc += dd * dd;
                    }
                }
            }
            if (i0 + 8 <= cnt) {
                *(GLOBAL uint32_t*)(cp + (i0 >> 1)) = pk;
            } else {
#pragma unroll
                for (int k = 0; k < 4; ++k)
                    if (i0 + 2 * k < cnt) cp[(i0 >> 1) + k] = (uint8_t)(pk >> (8 * k));
            }
        }
    }
    if constexpr (ERR) {
        s_err[t] = acc;
        __syncthreads();
        if (t == 0) {   // the group's blocks in order
            double s = 0.0;
            for (int i = 0; i < kVThreads; ++i) s += s_err[i];
            partial[blockIdx.x] = s;
        }
    }
}

template <int DT, int KIND>
__global__ __launch_bounds__(kVThreads) void k_var_dequant(const LayerDesc* __restrict__ tab, int nl,
                                                           int block, const float* __restrict__ mean)
{
    __shared__ float s_lv[16];
    const int t = threadIdx.x;
    if (t < 16) s_lv[t] = as_f(nf4fmt::kLevelBits[t]);
    __syncthreads();
    const VRef r = vref(tab, nl, blockIdx.x, block);
    const LayerDesc& d = *r.d;
    const int64_t b = r.b0 + t;
    if (b >= r.nb) return;
    float adq;
    if constexpr (KIND == 0) {
        adq = ((const GLOBAL float*)d.absmax)[b];
    } else {
        const uint32_t q = ((const GLOBAL uint8_t*)d.qabsmax)[b];
        const float s2 = ((const GLOBAL float*)d.scale2)[r.local];
        adq = block_adq<KIND>(0.0f, q, s2, KIND >= 2 ? mean[r.l] : 0.0f);
    }
    const int64_t e0 = b * block;
    const int cnt = (int)min((int64_t)block, d.n - e0);
    const GLOBAL uint8_t* cp = (const GLOBAL uint8_t*)d.codes + (e0 >> 1);
    GLOBAL uint16_t* out = (GLOBAL uint16_t*)d.out + e0;
    for (int i0 = 0; i0 < cnt; i0 += 8) {
        const uint32_t c = (i0 + 8 <= cnt) ? *(const GLOBAL uint32_t*)(cp + (i0 >> 1)) : 0u;
        uint32_t cc = c;
        if (i0 + 8 > cnt)
            for (int k = 0; k < 4; ++k)
                if (i0 + 2 * k < cnt) cc |= (uint32_t)cp[(i0 >> 1) + k] << (8 * k);
        uint32_t y[4];
#pragma unroll
        for (int k = 0; k < 4; ++k)
            y[k] = to16<DT>(s_lv[(cc >> (8 * k)) & 15] * adq) |
                   (to16<DT>(s_lv[(cc >> (8 * k + 4)) & 15] * adq) << 16);
        if (i0 + 8 <= cnt) {
            *(GLOBAL u32x4*)(out + i0) = u32x4{y[0], y[1], y[2], y[3]};
        } else {
            for (int k = 0; k < 8; ++k)
                if (i0 + k < cnt) out[i0 + k] = (uint16_t)(y[k >> 1] >> (16 * (k & 1)));
        }
    }
}

// per-layer sum of the group partials, in group order
__global__ void k_var_reduce(const LayerDesc* __restrict__ tab, int nl,
                             const double* __restrict__ partial, double* __restrict__ err)
{
    const int l = blockIdx.x * blockDim.x + threadIdx.x;
    if (l >= nl) return;
    double s = 0.0;
    for (int64_t g = l ? tab[l - 1].tile_end : 0; g < tab[l].tile_end; ++g) s += partial[g];
    err[l] = s;
}

constexpr int64_t kMaxVGrid = 0x7fffffff / kVThreads;

template <int DT, int KIND>
hipError_t variant_go(const LayerDesc* tab, int nl, int64_t ngroups, int block, float* mean,
                      double* gsum, double* partial, double* err, hipStream_t s)
{
    if (ngroups > kMaxVGrid) return hipErrorInvalidValue;
    const unsigned g = (unsigned)ngroups, lg = (unsigned)((nl + 255) / 256);
    hipLaunchKernelGGL((k_var_absmax<DT>), dim3(g), dim3(kVThreads), 0, s, tab, nl, block, gsum);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (KIND >= 2) {
        hipLaunchKernelGGL(k_var_mean, dim3(lg), dim3(256), 0, s, tab, nl, block, gsum, mean);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    hipLaunchKernelGGL((k_var_codec<DT, KIND, true>), dim3(g), dim3(kVThreads), 0, s, tab, nl, block,
                       mean, partial);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(k_var_reduce, dim3(lg), dim3(256), 0, s, tab, nl, partial, err);
    return hipGetLastError();
}

template <int DT, int KIND>
hipError_t variant_dq_go(const LayerDesc* tab, int nl, int64_t ngroups, int block, const float* mean,
                         hipStream_t s)
{
    if (ngroups > kMaxVGrid) return hipErrorInvalidValue;
    hipLaunchKernelGGL((k_var_dequant<DT, KIND>), dim3((unsigned)ngroups), dim3(kVThreads), 0, s,
                       tab, nl, block, mean);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_variant_error(const LayerDesc* tab, int nl, int64_t ngroups, int dtype, int block,
                                int kind, float* mean, double* gsum, double* partial, double* err,
                                hipStream_t s)
{
#define NF4_VAR(DT) \
    switch (kind) { \
        case 0: return variant_go<DT, 0>(tab, nl, ngroups, block, mean, gsum, partial, err, s); \
        case 1: return variant_go<DT, 1>(tab, nl, ngroups, block, mean, gsum, partial, err, s); \
        case 2: return variant_go<DT, 2>(tab, nl, ngroups, block, mean, gsum, partial, err, s); \
        default: return variant_go<DT, 3>(tab, nl, ngroups, block, mean, gsum, partial, err, s); \
    }
    if (dtype == 0) { NF4_VAR(0) }
    NF4_VAR(1)
#undef NF4_VAR
}

hipError_t launch_variant_dequant(const LayerDesc* tab, int nl, int64_t ngroups, int dtype,
                                  int block, int kind, const float* mean, hipStream_t s)
{
#define NF4_VDQ(DT) \
    switch (kind) { \
        case 0: return variant_dq_go<DT, 0>(tab, nl, ngroups, block, mean, s); \
        case 1: return variant_dq_go<DT, 1>(tab, nl, ngroups, block, mean, s); \
        case 2: return variant_dq_go<DT, 2>(tab, nl, ngroups, block, mean, s); \
        default: return variant_dq_go<DT, 3>(tab, nl, ngroups, block, mean, s); \
    }
    if (dtype == 0) { NF4_VDQ(0) }
    NF4_VDQ(1)
#undef NF4_VDQ
}

}  // namespace nf4k
