// k_select.hip -- AQLoRA's budgeted top-K on the device.
//
// AQLoRA orders the matrices by their NF4 reconstruction error and keeps the
// leading ones in 16 bits while a memory budget allows (AQLoRA listing,
// arxivdaily.com, English abstract); the budget is a setting ("AQLoRA: A
// Zero-Search Recipe...", aitrending.vip, Technical Details).  Order: error descending, equal errors
// by layer index ascending (a strict total order, so the ranking is unique).
// K = the longest prefix of that order whose running promotion cost stays
// within the budget, capped by k_cap.
//
// Two launches: k_rank gives every layer its rank by counting the layers
// ahead of it (nl <= 65536, so nl^2 compares over the whole GPU is a few
// microseconds and needs no sort); k_take runs in one workgroup, scans the
// costs in rank order and writes selected[] and K.
//
// Variants (the speed setting adapts only the highest-ranked blocks: AQLoRA
// listing, English abstract): the ranked units may be groups of consecutive layers
// (transformer blocks, promoted whole), each layer's error may be divided by
// a per-layer denominator (n: mean squared error; sum of x^2: relative
// error), and the budget may be filled past a unit that does not fit
// (k_fill) instead of stopping there (k_take).  k_units forms the unit
// scores and costs, k_expand writes the units' choice back per layer.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "nf4_internal.h"
#include "nf4_launch.h"

namespace nf4k {
namespace {

constexpr int kRankThreads = 256;
constexpr int kTakeThreads = 1024;
constexpr int kFillThreads = 256;
constexpr int kFillPage = 4096;   // ranks staged in LDS per pass of the fill walk

__global__ __launch_bounds__(kRankThreads) void k_rank(const double* __restrict__ err, int nl,
                                                       int32_t* __restrict__ rank,
                                                       int32_t* __restrict__ perm)
{
    __shared__ double s_e[kRankThreads];
    const int i = blockIdx.x * kRankThreads + threadIdx.x;
    const double ei = (i < nl) ? err[i] : 0.0;
    int r = 0;
    for (int j0 = 0; j0 < nl; j0 += kRankThreads) {
        const int jj = j0 + threadIdx.x;
        s_e[threadIdx.x] = (jj < nl) ? err[jj] : 0.0;
        __syncthreads();
        const int m = (nl - j0) < kRankThreads ? (nl - j0) : kRankThreads;
        for (int k = 0; k < m; ++k) {
            const double ej = s_e[k];
            const int j = j0 + k;
            r += (ej > ei) || (ej == ei && j < i);
        }
        __syncthreads();
    }
    if (i < nl) {
        rank[i] = r;
        perm[r] = i;
    }
}

__global__ __launch_bounds__(kTakeThreads) void k_take(const int64_t* __restrict__ cost, int nl,
                                                       int64_t budget, int kcap,
                                                       const int32_t* __restrict__ rank,
                                                       const int32_t* __restrict__ perm,
                                                       uint8_t* __restrict__ selected,
                                                       int32_t* __restrict__ k_out)
{
    __shared__ int64_t s_sum[kTakeThreads];
    __shared__ int s_first[kTakeThreads];
    const int t = threadIdx.x;
    const int chunk = (nl + kTakeThreads - 1) / kTakeThreads;
    const int r0 = t * chunk;
    const int r1 = (r0 + chunk < nl) ? r0 + chunk : nl;

    // perm is a permutation for finite scores; the clamp keeps NaN scores
    // (unsupported, unspecified result) from reading outside cost[]
    auto at = [&](int r) { const int p = perm[r]; return cost[(unsigned)p < (unsigned)nl ? p : 0]; };
    int64_t local = 0;
    for (int r = r0; r < r1; ++r) local += at(r);
    s_sum[t] = local;
    __syncthreads();
    // inclusive scan over the per-thread sums (Hillis-Steele, fixed order)
    for (int off = 1; off < kTakeThreads; off <<= 1) {
        const int64_t add = (t >= off) ? s_sum[t - off] : 0;
        __syncthreads();
        s_sum[t] += add;
        __syncthreads();
    }
    int64_t run = s_sum[t] - local;   // exclusive prefix: cost of ranks < r0
    int first = nl;                   // first rank that does not fit
    if (budget >= 0) {
        for (int r = r0; r < r1; ++r) {
            run += at(r);
            if (run > budget) { first = r; break; }
        }
    }
    s_first[t] = first;
    __syncthreads();
    for (int h = kTakeThreads / 2; h >= 1; h >>= 1) {
        if (t < h) s_first[t] = min(s_first[t], s_first[t + h]);
        __syncthreads();
    }
    int K = s_first[0];
    if (kcap >= 0 && kcap < K) K = kcap;
    for (int i = t; i < nl; i += kTakeThreads) selected[i] = (rank[i] < K) ? 1 : 0;
    if (t == 0) *k_out = K;
}

// Unit u: layer u, or layers group_end[u-1] .. group_end[u]-1 (group_end[-1]
// = 0).  Score = sum over its layers, in layer order, of err (divided by denom
// when given, IEEE fp64); cost = sum of the layers' costs.
__global__ __launch_bounds__(kRankThreads) void k_units(const double* __restrict__ err,
                                                        const double* __restrict__ denom,
                                                        const int64_t* __restrict__ cost,
                                                        const int32_t* __restrict__ group_end,
                                                        int nu, double* __restrict__ uscore,
                                                        int64_t* __restrict__ ucost)
{
    const int u = blockIdx.x * kRankThreads + threadIdx.x;
    if (u >= nu) return;
    const int b = group_end ? (u ? group_end[u - 1] : 0) : u;
    const int e = group_end ? group_end[u] : u + 1;
    double sc = 0.0;
    int64_t c = 0;
    for (int i = b; i < e; ++i) {
        sc += denom ? err[i] / denom[i] : err[i];
        c += cost[i];
    }
    uscore[u] = sc;
    ucost[u] = c;
}

// Fill rule: walk the ranking and take every unit that still fits (and while
// fewer than kcap are taken).  The walk is sequential by definition; the
// workgroup gathers each page of costs in rank order into LDS and one thread
// walks it, the running total staying in its registers across pages.
__global__ __launch_bounds__(kFillThreads) void k_fill(const int64_t* __restrict__ cost, int nu,
                                                       int64_t budget, int kcap,
                                                       const int32_t* __restrict__ perm,
                                                       uint8_t* __restrict__ flag,
                                                       int32_t* __restrict__ k_out)
{
    __shared__ int64_t s_c[kFillPage];
    __shared__ int32_t s_u[kFillPage];
    __shared__ uint8_t s_take[kFillPage];
    const int t = threadIdx.x;
    int64_t total = 0;
    int K = 0;
    for (int p0 = 0; p0 < nu; p0 += kFillPage) {
        const int m = (nu - p0) < kFillPage ? (nu - p0) : kFillPage;
        for (int r = t; r < m; r += kFillThreads) {
            const int p = perm[p0 + r];
            const int u = (unsigned)p < (unsigned)nu ? p : 0;   // NaN scores: stay in bounds
            s_u[r] = u;
            s_c[r] = cost[u];
        }
        __syncthreads();
        if (t == 0) {
            for (int r = 0; r < m; ++r) {
                uint8_t take = 0;
                if (kcap < 0 || K < kcap) {
                    const int64_t next = total + s_c[r];
                    if (budget < 0 || next <= budget) {
                        total = next;
                        ++K;
                        take = 1;
                    }
                }
                s_take[r] = take;
            }
        }
        __syncthreads();
        for (int r = t; r < m; r += kFillThreads) flag[s_u[r]] = s_take[r];
        __syncthreads();
    }
    if (t == 0) *k_out = K;
}

__global__ __launch_bounds__(kRankThreads) void k_expand(const uint8_t* __restrict__ flag,
                                                         const int32_t* __restrict__ group_end,
                                                         int nu, uint8_t* __restrict__ selected)
{
    const int u = blockIdx.x * kRankThreads + threadIdx.x;
    if (u >= nu) return;
    const int b = u ? group_end[u - 1] : 0;
    for (int i = b; i < group_end[u]; ++i) selected[i] = flag[u];
}

}  // namespace

hipError_t launch_select(const double* err, const int64_t* cost, int nl, int64_t budget, int kcap,
                         uint8_t* selected, int32_t* k_out, int32_t* rank, int32_t* perm,
                         hipStream_t s)
{
    const unsigned grid = (unsigned)((nl + kRankThreads - 1) / kRankThreads);
    hipLaunchKernelGGL(k_rank, dim3(grid), dim3(kRankThreads), 0, s, err, nl, rank, perm);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_take, dim3(1), dim3(kTakeThreads), 0, s, cost, nl, budget, kcap, rank,
                       perm, selected, k_out);
    return hipGetLastError();
}

hipError_t launch_select_ex(const double* err, const double* denom, const int64_t* cost,
                            const int32_t* group_end, int nu, int64_t budget, int kcap, int rule,
                            uint8_t* selected, int32_t* k_out, SelectScratch w, hipStream_t s)
{
    const unsigned grid = (unsigned)((nu + kRankThreads - 1) / kRankThreads);
    const double* score = err;
    const int64_t* ucost = cost;
    hipError_t e;
    if (denom || group_end) {
        hipLaunchKernelGGL(k_units, dim3(grid), dim3(kRankThreads), 0, s, err, denom, cost,
                           group_end, nu, w.uscore, w.ucost);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        score = w.uscore;
        ucost = w.ucost;
    }
    hipLaunchKernelGGL(k_rank, dim3(grid), dim3(kRankThreads), 0, s, score, nu, w.rank, w.perm);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    uint8_t* flag = group_end ? w.flag : selected;
    if (rule == 0)
        hipLaunchKernelGGL(k_take, dim3(1), dim3(kTakeThreads), 0, s, ucost, nu, budget, kcap,
                           w.rank, w.perm, flag, k_out);
    else
        hipLaunchKernelGGL(k_fill, dim3(1), dim3(kFillThreads), 0, s, ucost, nu, budget, kcap,
                           w.perm, flag, k_out);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (group_end) {
        hipLaunchKernelGGL(k_expand, dim3(grid), dim3(kRankThreads), 0, s, flag, group_end, nu,
                           selected);
        e = hipGetLastError();
    }
    return e;
}

}  // namespace nf4k
