// nf4_launch.h -- the kernel launchers the C entry points in nf4_api.cpp call
// after validating their arguments (not part of the public ABI).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "nf4_internal.h"

namespace nf4k {

// Fused blockwise quantisation (+ int8 double quantisation when dq) and, when
// err_partial != nullptr, in-register dequantisation and the fp64 squared
// error, written as kPartsPerTile partials per tile to err_partial; with
// sq_partial != nullptr too, also the sum of x^2, laid out the same way.
// rec_ws: device scratch for one 8-byte tile record per tile (kRecordBytes).
// ragged: some layer's n is not a multiple of kTileElems (adds the tail launch).
constexpr int kRecordBytes = 8;
hipError_t launch_codec(const LayerDesc* tab, int nl, int64_t ntiles, bool ragged, int dtype,
                        bool dq, void* rec_ws, double* err_partial, double* sq_partial,
                        hipStream_t s);
// Per-layer fixed-order sum of the per-tile partials into err[nl].
hipError_t launch_reduce(const LayerDesc* tab, int nl, const double* partial, double* err,
                         hipStream_t s);
// Standalone dequantisation (qabsmax/scale2 when dq, else absmax); desc_ws:
// device scratch for one 32-byte record per tile (kPartsPerTile doubles);
// skip: null, or device uint8[nl] (layers with a nonzero byte are left alone).
hipError_t launch_dequant(const LayerDesc* tab, int nl, int64_t ntiles, int dtype, bool dq,
                          const uint8_t* skip, void* desc_ws, hipStream_t s);
// Standalone double quantisation of absmax.
hipError_t launch_double_quant(const LayerDesc* tab, int nl, int64_t ntiles, hipStream_t s);
// Budgeted top-K; rank/perm are int32[nl] workspace arrays.
// Codec variants (block 32/64/128/256; second-level kind 0 none, 1 int8,
// 2 int8 minus the mean absmax, 3 E4M3 minus the mean absmax).  The table's
// tile_end counts groups of 256 blocks of the variant's block size.
// gsum and partial: one fp64 per group.
hipError_t launch_variant_error(const LayerDesc* tab, int nl, int64_t ngroups, int dtype, int block,
                                int kind, float* mean, double* gsum, double* partial, double* err,
                                hipStream_t s);
// rec_ws: device scratch for one 64-byte record per group.
hipError_t launch_variant_dequant(const LayerDesc* tab, int nl, int64_t ngroups, int dtype,
                                  int block, int kind, const float* mean, void* rec_ws, hipStream_t s);
// NF4 weight dequantised into the matmul that consumes it (bf16 MFMA):
// forward out[m x rows] = x[m x cols] * W^T, backward out[m x cols] =
// x[m x rows] * W; W [rows x cols] given by its codes and constants
// (qabsmax + scale2 when qabsmax != nullptr, else absmax).  rows and cols
// multiples of 128; x and the dequantised W in the 16-bit type dtype (0 bf16,
// 1 fp16); out fp32 or that 16-bit type.  With part != nullptr and nsplit > 1
// the reduction is split nsplit ways into fp32 partials at part
// ([nsplit][m x (rows | cols)]), then added in split order into out.  With
// part != nullptr, nsplit == 1 and tail_split > 1 (the value
// nf4_matmul_tail_splits gives for the shape), the tiles left over after the
// whole rounds are split tail_split ways into [tail_split][rem][256 x 256]
// fp32 blocks at part, then added in split order into out.
hipError_t launch_nf4_matmul(int dtype, const uint8_t* codes, const int8_t* qabsmax, const float* scale2,
                             const float* absmax, int64_t rows, int64_t cols, bool forward,
                             const void* x, int64_t m, void* out, bool out_f32, float* part, int nsplit,
                             int tail_split, hipStream_t s);
// The split count the split-reduction matmul uses for a shape (1: none); a
// function of the shape only.
int nf4_matmul_splits(int64_t rows, int64_t cols, bool forward, int64_t m);
// Where the large-tile kernels take a shape whole: the split count of its
// leftover tiles with a workspace (0: none) and, when > 0, their number in
// *rem_out; a function of the shape only.
int nf4_matmul_tail_splits(int64_t rows, int64_t cols, bool forward, int64_t m, int64_t* rem_out);
// Few-token forward (m <= 32): the part count of the wave-per-16-rows path
// (0 when it does not apply); a function of the shape only.
int nf4_gemv_parts(int64_t rows, int64_t cols, bool forward, int64_t m);
// That path: fp32 partials at part ([parts][m x rows]), then added in part
// order into out (fp32 or the 16-bit type dtype).
hipError_t launch_nf4_gemv(int dtype, const uint8_t* codes, const int8_t* qabsmax, const float* scale2,
                           const float* absmax, int64_t rows, int64_t cols, const void* x, int64_t m,
                           void* out, bool out_f32, float* part, int parts, hipStream_t s);
hipError_t launch_select(const double* err, const int64_t* cost, int nl, int64_t budget,
                         int kcap, uint8_t* selected, int32_t* k_out, int32_t* rank,
                         int32_t* perm, hipStream_t s);
// Selection variants: unit = layer, or group of consecutive layers when
// group_end (device, nu entries) is given; score = err (/ denom when given);
// rule 0 = longest prefix within the budget, 1 = fill past what does not fit.
struct SelectScratch {
    int32_t* rank;    // [nu]
    int32_t* perm;    // [nu]
    double* uscore;   // [nu]
    int64_t* ucost;   // [nu]
    uint8_t* flag;    // [nu]
};
// The fixed device scratch of nf4_layer_error_noalloc (nf4_scratch.hip):
// kScratchBytes per device.  scratch_pointer returns the current device's
// copy, looked up once per device with hipGetSymbolAddress (thread-safe).
constexpr size_t kScratchBytes = size_t(32) << 20;
hipError_t scratch_pointer(void** out);

hipError_t launch_select_ex(const double* err, const double* denom, const int64_t* cost,
                            const int32_t* group_end, int nu, int64_t budget, int kcap, int rule,
                            uint8_t* selected, int32_t* k_out, SelectScratch w, hipStream_t s);

}  // namespace nf4k
