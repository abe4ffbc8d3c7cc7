// nf4_api.cpp -- the C entry points of include/nf4.h: argument validation
// (all on the host, before anything is enqueued), workspace layout, staging
// of the layer table, and the kernel launches.
#include "nf4.h"

#include <hip/hip_runtime.h>

#include <cstring>
#include <vector>

#include "nf4_format.h"
#include "nf4_internal.h"
#include "nf4_launch.h"

using nf4k::LayerDesc;

namespace {

thread_local int32_t g_last_hip = 0;

constexpr int64_t kMaxN = int64_t(1) << 40;
constexpr int32_t kMaxLayers = 1 << 24;
// tiles of 16,384 weights over all matrices of one call: the fused kernel's
// persistent walk counts them in 32 bits, tile index plus grid size included
// (2^31 tiles are 3.5e13 weights)
constexpr int64_t kMaxTiles = (int64_t(1) << 31) - (int64_t(1) << 20);
constexpr int32_t kMaxSelectLayers = 65536;

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }
inline bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

nf4_status check_format(const nf4_format& f)
{
    if (f.blocksize != nf4fmt::kBlock) return NF4_E_UNSUPPORTED;
    if (f.dq_group != 0 && f.dq_group != nf4fmt::kGroup) return NF4_E_UNSUPPORTED;
    if (f.dtype != NF4_BF16 && f.dtype != NF4_FP16) return NF4_E_UNSUPPORTED;
    return NF4_OK;
}

// Which pointers of a layer a call needs.
enum Need : unsigned {
    NEED_W = 1, NEED_CODES = 2, NEED_ABSMAX = 4, NEED_Q = 8, NEED_S2 = 16, NEED_OUT = 32,
    OPT_ABSMAX = 64
};

nf4_status check_layers(const nf4_layer* L, int32_t nl, unsigned need, int64_t* ntiles_out)
{
    if (!L || nl <= 0 || nl > kMaxLayers) return NF4_E_ARG;
    int64_t ntiles = 0;
    for (int32_t i = 0; i < nl; ++i) {
        const nf4_layer& x = L[i];
        if (x.n <= 0 || x.n >= kMaxN) return NF4_E_ARG;
        if ((need & NEED_W) && !x.w) return NF4_E_ARG;
        if ((need & NEED_CODES) && !x.codes) return NF4_E_ARG;
        if ((need & NEED_ABSMAX) && !x.absmax) return NF4_E_ARG;
        if ((need & NEED_Q) && !x.qabsmax) return NF4_E_ARG;
        if ((need & NEED_S2) && !x.scale2) return NF4_E_ARG;
        if ((need & NEED_OUT) && !x.out) return NF4_E_ARG;
        if ((need & NEED_W) && !aligned(x.w, 16)) return NF4_E_ALIGN;
        if ((need & NEED_CODES) && !aligned(x.codes, 16)) return NF4_E_ALIGN;
        if ((need & (NEED_ABSMAX | OPT_ABSMAX)) && x.absmax && !aligned(x.absmax, 4)) return NF4_E_ALIGN;
        if ((need & NEED_S2) && !aligned(x.scale2, 4)) return NF4_E_ALIGN;
        if ((need & NEED_OUT) && !aligned(x.out, 16)) return NF4_E_ALIGN;
        ntiles += nf4k::tiles_of(x.n);
    }
    if (ntiles >= kMaxTiles) return NF4_E_UNSUPPORTED;
    *ntiles_out = ntiles;
    return NF4_OK;
}

// Some matrix ends in a partial tile (the fused pass then adds its tail launch).
bool any_ragged(const nf4_layer* L, int32_t nl)
{
    for (int32_t i = 0; i < nl; ++i)
        if (L[i].n % nf4k::kTileElems) return true;
    return false;
}

size_t table_bytes(int32_t nl) { return align256(size_t(nl) * sizeof(LayerDesc)); }
size_t partial_bytes(int64_t ntiles)
{
    return align256(size_t(ntiles) * nf4k::kPartsPerTile * sizeof(double));
}
// The fused pass's per-tile records (where each tile lies), after the table.
size_t record_bytes(int64_t ntiles) { return align256(size_t(ntiles) * nf4k::kRecordBytes); }

nf4_status check_ws(const void* ws, size_t ws_bytes, size_t need)
{
    if (!ws || !aligned(ws, 256) || ws_bytes < need) return NF4_E_WORKSPACE;
    return NF4_OK;
}

nf4_status hip_fail(hipError_t e)
{
    g_last_hip = static_cast<int32_t>(e);
    return NF4_E_HIP;
}

// Build the device layer table in host memory and copy it into the workspace
// on the stream.  The copy is from pageable memory, which the runtime stages
// before the call returns, so the host vector may die right after.
nf4_status stage_table(const nf4_layer* L, int32_t nl, void* ws, hipStream_t s)
{
    std::vector<LayerDesc> tab(static_cast<size_t>(nl));
    int64_t run = 0;
    for (int32_t i = 0; i < nl; ++i) {
        run += nf4k::tiles_of(L[i].n);
        tab[i] = LayerDesc{L[i].w, L[i].codes, L[i].absmax, L[i].qabsmax, L[i].scale2, L[i].out,
                           L[i].n, run};
    }
    hipError_t e = hipMemcpyAsync(ws, tab.data(), sizeof(LayerDesc) * size_t(nl),
                                  hipMemcpyHostToDevice, s);
    if (e != hipSuccess) return hip_fail(e);
    return NF4_OK;
}

// Table for the codec variants: tile_end counts groups of 256 blocks of the
// variant's block size.
nf4_status stage_table_variant(const nf4_layer* L, int32_t nl, int block, void* ws, hipStream_t s)
{
    std::vector<LayerDesc> tab(static_cast<size_t>(nl));
    int64_t run = 0;
    for (int32_t i = 0; i < nl; ++i) {
        const int64_t nb = (L[i].n + block - 1) / block;
        run += (nb + nf4fmt::kGroup - 1) / nf4fmt::kGroup;
        tab[i] = LayerDesc{L[i].w, L[i].codes, L[i].absmax, L[i].qabsmax, L[i].scale2, L[i].out,
                           L[i].n, run};
    }
    hipError_t e = hipMemcpyAsync(ws, tab.data(), sizeof(LayerDesc) * size_t(nl),
                                  hipMemcpyHostToDevice, s);
    if (e != hipSuccess) return hip_fail(e);
    return NF4_OK;
}

nf4_status check_variant(const nf4_variant& v)
{
    if (v.blocksize != 32 && v.blocksize != 64 && v.blocksize != 128 && v.blocksize != 256)
        return NF4_E_UNSUPPORTED;
    if (v.dq_kind < NF4_DQ_NONE || v.dq_kind > NF4_DQ_E4M3_MEAN) return NF4_E_UNSUPPORTED;
    if (v.dtype != NF4_BF16 && v.dtype != NF4_FP16) return NF4_E_UNSUPPORTED;
    return NF4_OK;
}

// Workspace after the table for the variant calls: two fp64 per group (error
// pass) or one 64-byte record per group (dequantisation), whichever is larger.
size_t variant_scratch_bytes(int64_t ng)
{
    const size_t two = 2 * align256(size_t(ng) * sizeof(double)), rec = align256(size_t(ng) * 64);
    return two > rec ? two : rec;
}

int64_t variant_groups(const nf4_layer* L, int32_t nl, int block)
{
    int64_t g = 0;
    for (int32_t i = 0; i < nl; ++i) g += ((L[i].n + block - 1) / block + nf4fmt::kGroup - 1) / nf4fmt::kGroup;
    return g;
}

// The fused pass; with sumsq also the per-layer sum of x^2 (partials for it
// follow the error partials in the workspace).
nf4_status layer_error_impl(const nf4_layer* layers, int32_t nl, nf4_format fmt, double* err,
                            double* sumsq, void* ws, size_t ws_bytes, hipStream_t stream)
{
    nf4_status st = check_format(fmt);
    if (st != NF4_OK) return st;
    const bool dq = fmt.dq_group != 0;
    if (!err) return NF4_E_ARG;
    int64_t ntiles = 0;
    st = check_layers(layers, nl,
                      NEED_W | NEED_CODES | (dq ? NEED_Q | NEED_S2 | OPT_ABSMAX : NEED_ABSMAX),
                      &ntiles);
    if (st != NF4_OK) return st;
    if (!aligned(err, 8) || (sumsq && !aligned(sumsq, 8))) return NF4_E_ALIGN;
    const size_t need = table_bytes(nl) + record_bytes(ntiles) + (sumsq ? 2 : 1) * partial_bytes(ntiles);
    if ((st = check_ws(ws, ws_bytes, need)) != NF4_OK) return st;
    hipStream_t s = stream;
    if ((st = stage_table(layers, nl, ws, s)) != NF4_OK) return st;
    const LayerDesc* tab = static_cast<const LayerDesc*>(ws);
    char* rec = static_cast<char*>(ws) + table_bytes(nl);
    double* partial = reinterpret_cast<double*>(rec + record_bytes(ntiles));
    double* partial_sq = sumsq ? reinterpret_cast<double*>(reinterpret_cast<char*>(partial) +
                                                           partial_bytes(ntiles))
                               : nullptr;
    hipError_t e = nf4k::launch_codec(tab, nl, ntiles, any_ragged(layers, nl), fmt.dtype, dq,
                                      rec, partial, partial_sq, s);
    if (e != hipSuccess) return hip_fail(e);
    e = nf4k::launch_reduce(tab, nl, partial, err, s);
    if (e == hipSuccess && sumsq) e = nf4k::launch_reduce(tab, nl, partial_sq, sumsq, s);
    return e == hipSuccess ? NF4_OK : hip_fail(e);
}

// Selection workspace: rank, perm (as aqlora_select_topk uses them), then the
// staged group boundaries, unit scores, unit costs and unit flags.
struct SelectLayout {
    size_t rank, perm, groups, uscore, ucost, flag, total;
};

SelectLayout select_layout(int32_t nl)
{
    SelectLayout L;
    const size_t i4 = align256(size_t(nl) * 4), i8 = align256(size_t(nl) * 8);
    L.rank = 0;
    L.perm = L.rank + i4;
    L.groups = L.perm + i4;
    L.uscore = L.groups + i4;
    L.ucost = L.uscore + i8;
    L.flag = L.ucost + i8;
    L.total = L.flag + align256(size_t(nl));
    return L;
}

nf4_status check_matmul(const nf4_layer* w, int64_t rows, int64_t cols, nf4_format fmt,
                        int32_t backward, const void* x, int64_t m, void* out, int32_t out_fp32)
{
    nf4_status st = check_format(fmt);
    if (st != NF4_OK) return st;
    if (!w || !x || !out) return NF4_E_ARG;
    if (rows <= 0 || cols <= 0 || m <= 0 || m >= (int64_t(1) << 31)) return NF4_E_ARG;
    if (rows > kMaxN / cols || w->n != rows * cols) return NF4_E_ARG;
    if (rows % 128 || cols % 128) return NF4_E_UNSUPPORTED;
    if (backward != 0 && backward != 1) return NF4_E_ARG;
    if (out_fp32 != 0 && out_fp32 != 1) return NF4_E_ARG;
    const bool dq = fmt.dq_group != 0;
    if (!w->codes || (dq ? (!w->qabsmax || !w->scale2) : !w->absmax)) return NF4_E_ARG;
    if (!aligned(w->codes, 16) || !aligned(x, 16) || !aligned(out, 16)) return NF4_E_ALIGN;
    if (dq ? !aligned(w->scale2, 4) : !aligned(w->absmax, 4)) return NF4_E_ALIGN;
    return NF4_OK;
}

nf4_status run_matmul(const nf4_layer* w, int64_t rows, int64_t cols, nf4_format fmt, int32_t backward,
                      const void* x, int64_t m, void* out, int32_t out_fp32, float* part, int nsplit,
                      int tail_split, hipStream_t stream)
{
    const bool dq = fmt.dq_group != 0;
    hipError_t e = nf4k::launch_nf4_matmul(fmt.dtype, w->codes, dq ? w->qabsmax : nullptr,
                                           dq ? w->scale2 : nullptr, dq ? nullptr : w->absmax,
                                           rows, cols, backward == 0, x, m, out, out_fp32 == 1,
                                           part, nsplit, tail_split, stream);
    return e == hipSuccess ? NF4_OK : hip_fail(e);
}

// Bytes of fp32 partials for nsplit splits (0 without a split).
size_t matmul_part_bytes(int64_t rows, int64_t cols, int32_t backward, int64_t m, int nsplit)
{
    if (nsplit <= 1) return 0;
    const int64_t ncol = backward ? cols : rows;
    return align256(size_t(nsplit) * size_t(m) * size_t(ncol) * sizeof(float));
}

// Bytes of fp32 partials of the leftover tiles' splits: one 256 x 256 block per
// (split, tile); 0 when the shape has no such split.
size_t matmul_tail_bytes(int64_t rows, int64_t cols, int32_t backward, int64_t m, int* tail_split)
{
    int64_t rem = 0;
    const int ts = nf4k::nf4_matmul_tail_splits(rows, cols, backward == 0, m, &rem);
    if (tail_split) *tail_split = ts;
    if (ts <= 1) return 0;
    return align256(size_t(ts) * size_t(rem) * size_t(256 * 256) * sizeof(float));
}

// nf4_dequantize, with the device skip mask of nf4_dequantize_masked (or null).
nf4_status dequantize_impl(const nf4_layer* layers, int32_t nl, nf4_format fmt, const uint8_t* skip,
                           void* ws, size_t ws_bytes, hipStream_t stream)
{
    nf4_status st = check_format(fmt);
    if (st != NF4_OK) return st;
    const bool dq = fmt.dq_group != 0;
    int64_t ntiles = 0;
    st = check_layers(layers, nl, NEED_CODES | NEED_OUT | (dq ? NEED_Q | NEED_S2 : NEED_ABSMAX),
                      &ntiles);
    if (st != NF4_OK) return st;
    // the table, then one 32-byte record per tile (where the fused pass keeps its partials)
    if ((st = check_ws(ws, ws_bytes, table_bytes(nl) + partial_bytes(ntiles))) != NF4_OK) return st;
    hipStream_t s = stream;
    if ((st = stage_table(layers, nl, ws, s)) != NF4_OK) return st;
    hipError_t e = nf4k::launch_dequant(static_cast<const LayerDesc*>(ws), nl, ntiles, fmt.dtype,
                                        dq, skip, static_cast<char*>(ws) + table_bytes(nl), s);
    return e == hipSuccess ? NF4_OK : hip_fail(e);
}

}  // namespace

extern "C" {

int32_t nf4_abi_version(void) { return NF4_ABI_VERSION; }
int32_t nf4_last_hip_error(void) { return g_last_hip; }

const char* nf4_status_str(nf4_status s)
{
    switch (s) {
        case NF4_OK: return "ok";
        case NF4_E_ARG: return "invalid argument";
        case NF4_E_ALIGN: return "misaligned pointer";
        case NF4_E_UNSUPPORTED: return "unsupported format";
        case NF4_E_WORKSPACE: return "workspace missing, misaligned or too small";
        case NF4_E_HIP: return "HIP runtime error";
    }
    return "unknown status";
}

void nf4_levels(float out16[16])
{
    for (int i = 0; i < 16; ++i) std::memcpy(&out16[i], &nf4fmt::kLevelBits[i], 4);
}

void nf4_thresholds(float out15[15])
{
    for (int i = 0; i < 15; ++i) std::memcpy(&out15[i], &nf4fmt::kThresholdBits[i], 4);
}

int64_t nf4_storage_bytes(int64_t n, nf4_format f)
{
    if (n <= 0 || n >= kMaxN || check_format(f) != NF4_OK) return -1;
    const int64_t nb = (n + nf4fmt::kBlock - 1) / nf4fmt::kBlock;
    const int64_t ng = (nb + nf4fmt::kGroup - 1) / nf4fmt::kGroup;
    return (n + 1) / 2 + (f.dq_group ? nb + 4 * ng : 4 * nb);
}

int64_t aqlora_promote_cost(int64_t n, nf4_format f)
{
    const int64_t s = nf4_storage_bytes(n, f);
    return s < 0 ? -1 : 2 * n - s;
}

size_t nf4_workspace_bytes(int32_t nl, const int64_t* n_per_layer, nf4_format f)
{
    if (!n_per_layer || nl <= 0 || nl > kMaxLayers || check_format(f) != NF4_OK) return 0;
    int64_t ntiles = 0;
    for (int32_t i = 0; i < nl; ++i) {
        if (n_per_layer[i] <= 0 || n_per_layer[i] >= kMaxN) return 0;
        ntiles += nf4k::tiles_of(n_per_layer[i]);
    }
    if (ntiles >= kMaxTiles) return 0;
    // tile records, then error and sum-of-squares partials
    return table_bytes(nl) + record_bytes(ntiles) + 2 * partial_bytes(ntiles);
}

size_t aqlora_workspace_bytes(int32_t nl)
{
    if (nl <= 0 || nl > kMaxSelectLayers) return 0;
    return select_layout(nl).total;
}

nf4_status nf4_quantize(const nf4_layer* layers, int32_t nl, nf4_format fmt, void* ws,
                        size_t ws_bytes, hipStream_t stream)
{
    nf4_status st = check_format(fmt);
    if (st != NF4_OK) return st;
    const bool dq = fmt.dq_group != 0;
    int64_t ntiles = 0;
    st = check_layers(layers, nl, NEED_W | NEED_CODES | NEED_ABSMAX | (dq ? NEED_Q | NEED_S2 : 0u),
                      &ntiles);
    if (st != NF4_OK) return st;
    if ((st = check_ws(ws, ws_bytes, table_bytes(nl) + record_bytes(ntiles))) != NF4_OK) return st;
    hipStream_t s = stream;
    if ((st = stage_table(layers, nl, ws, s)) != NF4_OK) return st;
    hipError_t e = nf4k::launch_codec(static_cast<const LayerDesc*>(ws), nl, ntiles,
                                      any_ragged(layers, nl), fmt.dtype, dq,
                                      static_cast<char*>(ws) + table_bytes(nl), nullptr, nullptr, s);
    return e == hipSuccess ? NF4_OK : hip_fail(e);
}

nf4_status nf4_double_quant(const nf4_layer* layers, int32_t nl, nf4_format fmt, void* ws,
                            size_t ws_bytes, hipStream_t stream)
{
    nf4_status st = check_format(fmt);
    if (st != NF4_OK) return st;
    if (fmt.dq_group != nf4fmt::kGroup) return NF4_E_UNSUPPORTED;
    int64_t ntiles = 0;
    st = check_layers(layers, nl, NEED_ABSMAX | NEED_Q | NEED_S2, &ntiles);
    if (st != NF4_OK) return st;
    if ((st = check_ws(ws, ws_bytes, table_bytes(nl))) != NF4_OK) return st;
    hipStream_t s = stream;
    if ((st = stage_table(layers, nl, ws, s)) != NF4_OK) return st;
    hipError_t e = nf4k::launch_double_quant(static_cast<const LayerDesc*>(ws), nl, ntiles, s);
    return e == hipSuccess ? NF4_OK : hip_fail(e);
}

nf4_status nf4_dequantize(const nf4_layer* layers, int32_t nl, nf4_format fmt, void* ws,
                          size_t ws_bytes, hipStream_t stream)
{
    return dequantize_impl(layers, nl, fmt, nullptr, ws, ws_bytes, stream);
}

nf4_status nf4_dequantize_masked(const nf4_layer* layers, int32_t nl, nf4_format fmt,
                                 const uint8_t* skip, void* ws, size_t ws_bytes, hipStream_t stream)
{
    if (!skip) return NF4_E_ARG;
    return dequantize_impl(layers, nl, fmt, skip, ws, ws_bytes, stream);
}

nf4_status nf4_layer_error(const nf4_layer* layers, int32_t nl, nf4_format fmt, double* err,
                           void* ws, size_t ws_bytes, hipStream_t stream)
{
    return layer_error_impl(layers, nl, fmt, err, nullptr, ws, ws_bytes, stream);
}

nf4_status nf4_layer_error_noalloc(const nf4_layer* layers, int32_t nl, nf4_format fmt,
                                   double* err, hipStream_t stream)
{
    // the same checks as nf4_layer_error, then the size check against the
    // fixed scratch, all before anything is looked up or enqueued
    nf4_status st = check_format(fmt);
    if (st != NF4_OK) return st;
    const bool dq = fmt.dq_group != 0;
    if (!err) return NF4_E_ARG;
    int64_t ntiles = 0;
    st = check_layers(layers, nl,
                      NEED_W | NEED_CODES | (dq ? NEED_Q | NEED_S2 | OPT_ABSMAX : NEED_ABSMAX),
                      &ntiles);
    if (st != NF4_OK) return st;
    if (!aligned(err, 8)) return NF4_E_ALIGN;
    if (table_bytes(nl) + record_bytes(ntiles) + partial_bytes(ntiles) > nf4k::kScratchBytes)
        return NF4_E_WORKSPACE;
    void* scratch = nullptr;
    const hipError_t e = nf4k::scratch_pointer(&scratch);
    if (e != hipSuccess) return hip_fail(e);
    return layer_error_impl(layers, nl, fmt, err, nullptr, scratch, nf4k::kScratchBytes, stream);
}

size_t nf4_noalloc_scratch_bytes(void) { return nf4k::kScratchBytes; }

nf4_status nf4_layer_error_norm(const nf4_layer* layers, int32_t nl, nf4_format fmt, double* err,
                                double* sumsq, void* ws, size_t ws_bytes, hipStream_t stream)
{
    if (!sumsq) return NF4_E_ARG;
    return layer_error_impl(layers, nl, fmt, err, sumsq, ws, ws_bytes, stream);
}

nf4_status aqlora_select_topk(const double* err, const int64_t* cost, int32_t nl,
                              int64_t budget_bytes, int32_t k_cap, uint8_t* selected,
                              int32_t* k_out, void* ws, size_t ws_bytes, hipStream_t stream)
{
    if (!err || !cost || !selected || !k_out) return NF4_E_ARG;
    if (nl <= 0 || nl > kMaxSelectLayers) return NF4_E_ARG;
    if (!aligned(err, 8) || !aligned(cost, 8) || !aligned(k_out, 4)) return NF4_E_ALIGN;
    nf4_status st = check_ws(ws, ws_bytes, aqlora_workspace_bytes(nl));
    if (st != NF4_OK) return st;
    int32_t* rank = static_cast<int32_t*>(ws);
    int32_t* perm = reinterpret_cast<int32_t*>(static_cast<char*>(ws) +
                                               align256(size_t(nl) * sizeof(int32_t)));
    hipError_t e = nf4k::launch_select(err, cost, nl, budget_bytes, k_cap, selected, k_out, rank,
                                       perm, stream);
    return e == hipSuccess ? NF4_OK : hip_fail(e);
}

nf4_status aqlora_select(const double* err, const double* denom, const int64_t* cost, int32_t nl,
                         const int32_t* group_end, int32_t ngroups, int64_t budget_bytes,
                         int32_t k_cap, int32_t rule, uint8_t* selected, int32_t* k_out,
                         void* ws, size_t ws_bytes, hipStream_t stream)
{
    if (!err || !cost || !selected || !k_out) return NF4_E_ARG;
    if (nl <= 0 || nl > kMaxSelectLayers) return NF4_E_ARG;
    if (rule != AQLORA_PREFIX && rule != AQLORA_FILL) return NF4_E_ARG;
    if (group_end) {
        if (ngroups <= 0 || ngroups > nl || group_end[ngroups - 1] != nl) return NF4_E_ARG;
        int32_t prev = 0;
        for (int32_t g = 0; g < ngroups; ++g) {
            if (group_end[g] <= prev) return NF4_E_ARG;
            prev = group_end[g];
        }
    }
    if (!aligned(err, 8) || !aligned(cost, 8) || !aligned(k_out, 4) || (denom && !aligned(denom, 8)))
        return NF4_E_ALIGN;
    const SelectLayout L = select_layout(nl);
    nf4_status st = check_ws(ws, ws_bytes, L.total);
    if (st != NF4_OK) return st;
    char* w = static_cast<char*>(ws);
    hipStream_t s = stream;
    int32_t* ge = nullptr;
    if (group_end) {
        // pageable source: staged by the runtime before the call returns
        ge = reinterpret_cast<int32_t*>(w + L.groups);
        hipError_t e = hipMemcpyAsync(ge, group_end, sizeof(int32_t) * size_t(ngroups),
                                      hipMemcpyHostToDevice, s);
        if (e != hipSuccess) return hip_fail(e);
    }
    nf4k::SelectScratch scr{reinterpret_cast<int32_t*>(w + L.rank),
                            reinterpret_cast<int32_t*>(w + L.perm),
                            reinterpret_cast<double*>(w + L.uscore),
                            reinterpret_cast<int64_t*>(w + L.ucost),
                            reinterpret_cast<uint8_t*>(w + L.flag)};
    hipError_t e = nf4k::launch_select_ex(err, denom, cost, ge, group_end ? ngroups : nl,
                                          budget_bytes, k_cap, rule, selected, k_out, scr, s);
    return e == hipSuccess ? NF4_OK : hip_fail(e);
}


nf4_status nf4_matmul(const nf4_layer* w, int64_t rows, int64_t cols, nf4_format fmt,
                      int32_t backward, const void* x, int64_t m, void* out, int32_t out_fp32,
                      hipStream_t stream)
{
    nf4_status st = check_matmul(w, rows, cols, fmt, backward, x, m, out, out_fp32);
    if (st != NF4_OK) return st;
    return run_matmul(w, rows, cols, fmt, backward, x, m, out, out_fp32, nullptr, 1, 0, stream);
}

size_t nf4_matmul_workspace_bytes(int64_t rows, int64_t cols, int32_t backward, int64_t m)
{
    if (rows <= 0 || cols <= 0 || m <= 0 || m >= (int64_t(1) << 31) || rows % 128 || cols % 128)
        return 0;
    if (rows > kMaxN / cols || (backward != 0 && backward != 1)) return 0;
    const int gv = nf4k::nf4_gemv_parts(rows, cols, backward == 0, m);
    if (gv > 0) return align256(size_t(gv) * size_t(m) * size_t(rows) * sizeof(float));
    const size_t split = matmul_part_bytes(rows, cols, backward, m, nf4k::nf4_matmul_splits(rows, cols, backward == 0, m));
    return split > 0 ? split : matmul_tail_bytes(rows, cols, backward, m, nullptr);
}

nf4_status nf4_matmul_ws(const nf4_layer* w, int64_t rows, int64_t cols, nf4_format fmt,
                         int32_t backward, const void* x, int64_t m, void* out, int32_t out_fp32,
                         void* ws, size_t ws_bytes, hipStream_t stream)
{
    nf4_status st = check_matmul(w, rows, cols, fmt, backward, x, m, out, out_fp32);
    if (st != NF4_OK) return st;
    const int gv = nf4k::nf4_gemv_parts(rows, cols, backward == 0, m);
    if (gv > 0) {
        st = check_ws(ws, ws_bytes, nf4_matmul_workspace_bytes(rows, cols, backward, m));
        if (st != NF4_OK) return st;
        const bool dq = fmt.dq_group != 0;
        hipError_t e = nf4k::launch_nf4_gemv(fmt.dtype, w->codes, dq ? w->qabsmax : nullptr,
                                             dq ? w->scale2 : nullptr, dq ? nullptr : w->absmax, rows, cols,
                                             x, m, out, out_fp32 == 1, static_cast<float*>(ws), gv,
                                             stream);
        return e == hipSuccess ? NF4_OK : hip_fail(e);
    }
    const int nsplit = nf4k::nf4_matmul_splits(rows, cols, backward == 0, m);
    const size_t need = matmul_part_bytes(rows, cols, backward, m, nsplit);
    if (need == 0) {
        int tail = 0;
        const size_t tneed = matmul_tail_bytes(rows, cols, backward, m, &tail);
        if (tneed == 0)
            return run_matmul(w, rows, cols, fmt, backward, x, m, out, out_fp32, nullptr, 1, 0, stream);
        st = check_ws(ws, ws_bytes, tneed);
        if (st != NF4_OK) return st;
        return run_matmul(w, rows, cols, fmt, backward, x, m, out, out_fp32, static_cast<float*>(ws), 1, tail,
                          stream);
    }
    st = check_ws(ws, ws_bytes, need);
    if (st != NF4_OK) return st;
    return run_matmul(w, rows, cols, fmt, backward, x, m, out, out_fp32, static_cast<float*>(ws), nsplit, 0,
                      stream);
}

size_t nf4_workspace_bytes_variant(int32_t nl, const int64_t* n_per_layer, nf4_variant v)
{
    if (!n_per_layer || nl <= 0 || nl > kMaxLayers || check_variant(v) != NF4_OK) return 0;
    int64_t g = 0;
    for (int32_t i = 0; i < nl; ++i) {
        if (n_per_layer[i] <= 0 || n_per_layer[i] >= kMaxN) return 0;
        g += ((n_per_layer[i] + v.blocksize - 1) / v.blocksize + nf4fmt::kGroup - 1) / nf4fmt::kGroup;
    }
    return table_bytes(nl) + variant_scratch_bytes(g);
}

int64_t nf4_storage_bytes_variant(int64_t n, nf4_variant v)
{
    if (n <= 0 || n >= kMaxN || check_variant(v) != NF4_OK) return -1;
    const int64_t nb = (n + v.blocksize - 1) / v.blocksize;
    const int64_t ng = (nb + nf4fmt::kGroup - 1) / nf4fmt::kGroup;
    return (n + 1) / 2 + (v.dq_kind == NF4_DQ_NONE ? 4 * nb : nb + 4 * ng) +
           (v.dq_kind >= NF4_DQ_INT8_MEAN ? 4 : 0);
}

nf4_status nf4_layer_error_variant(const nf4_layer* layers, int32_t nl, nf4_variant v,
                                   float* mean, double* err, void* ws, size_t ws_bytes,
                                   hipStream_t stream)
{
    nf4_status st = check_variant(v);
    if (st != NF4_OK) return st;
    if (!err) return NF4_E_ARG;
    const bool second = v.dq_kind != NF4_DQ_NONE, with_mean = v.dq_kind >= NF4_DQ_INT8_MEAN;
    if (with_mean && !mean) return NF4_E_ARG;
    int64_t ntiles = 0;
    st = check_layers(layers, nl, NEED_W | NEED_CODES | NEED_ABSMAX | (second ? NEED_Q | NEED_S2 : 0u),
                      &ntiles);
    if (st != NF4_OK) return st;
    if (!aligned(err, 8) || (with_mean && !aligned(mean, 4))) return NF4_E_ALIGN;
    const int64_t ng = variant_groups(layers, nl, v.blocksize);
    const size_t part = align256(size_t(ng) * sizeof(double));
    if ((st = check_ws(ws, ws_bytes, table_bytes(nl) + 2 * part)) != NF4_OK) return st;
    hipStream_t s = stream;
    if ((st = stage_table_variant(layers, nl, v.blocksize, ws, s)) != NF4_OK) return st;
    char* w = static_cast<char*>(ws);
    hipError_t e = nf4k::launch_variant_error(
        reinterpret_cast<const LayerDesc*>(w), nl, ng, v.dtype, v.blocksize, v.dq_kind,
        with_mean ? mean : nullptr, reinterpret_cast<double*>(w + table_bytes(nl)),
        reinterpret_cast<double*>(w + table_bytes(nl) + part), err, s);
    return e == hipSuccess ? NF4_OK : hip_fail(e);
}

nf4_status nf4_dequantize_variant(const nf4_layer* layers, int32_t nl, nf4_variant v,
                                  const float* mean, void* ws, size_t ws_bytes, hipStream_t stream)
{
    nf4_status st = check_variant(v);
    if (st != NF4_OK) return st;
    const bool second = v.dq_kind != NF4_DQ_NONE, with_mean = v.dq_kind >= NF4_DQ_INT8_MEAN;
    if (with_mean && !mean) return NF4_E_ARG;
    int64_t ntiles = 0;
    st = check_layers(layers, nl, NEED_CODES | NEED_OUT | (second ? NEED_Q | NEED_S2 : NEED_ABSMAX),
                      &ntiles);
    if (st != NF4_OK) return st;
    if (with_mean && !aligned(mean, 4)) return NF4_E_ALIGN;
    const int64_t ng = variant_groups(layers, nl, v.blocksize);
    if ((st = check_ws(ws, ws_bytes, table_bytes(nl) + align256(size_t(ng) * 64))) != NF4_OK) return st;
    hipStream_t s = stream;
    if ((st = stage_table_variant(layers, nl, v.blocksize, ws, s)) != NF4_OK) return st;
    hipError_t e = nf4k::launch_variant_dequant(static_cast<const LayerDesc*>(ws), nl, ng, v.dtype,
                                                v.blocksize, v.dq_kind, with_mean ? mean : nullptr,
                                                static_cast<char*>(ws) + table_bytes(nl), s);
    return e == hipSuccess ? NF4_OK : hip_fail(e);
}

}  // extern "C"
