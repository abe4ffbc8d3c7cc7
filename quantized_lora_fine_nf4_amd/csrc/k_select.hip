// k_select.hip -- AQLoRA's budgeted top-K on the device.
//
// "The pass ranks layers by NF4 reconstruction error and keeps the top-K in
// fp16 under a memory budget" (AQLoRA listing, arxivdaily.com, English
// abstract); the budget is configurable ("AQLoRA: A Zero-Search Recipe...",
// aitrending.vip, Technical Details).  Order: error descending, equal errors
// by layer index ascending (a strict total order, so the ranking is unique).
// K = the longest prefix of that order whose running promotion cost stays
// within the budget, capped by k_cap.
//
// Two launches: k_rank gives every layer its rank by counting the layers
// ahead of it (nl <= 65536, so nl^2 compares over the whole GPU is a few
// microseconds and needs no sort); k_take runs in one workgroup, scans the
// costs in rank order and writes selected[] and K.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "nf4_internal.h"

namespace nf4k {
namespace {

constexpr int kRankThreads = 256;
constexpr int kTakeThreads = 1024;

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

}  // namespace nf4k
