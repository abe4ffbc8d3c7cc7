/*
 * nf4.h -- C ABI of the MI355X (gfx950) NF4 weight codec and AQLoRA layer
 * selector.
 *
 * What the calls compute, and where the pages define it:
 *   - NF4: 4-bit NormalFloat, 16 values placed so that each gets an equal share
 *     of normally distributed weights ("QLoRA" paper summary page,
 *     ai360xpert.com, How It Works, NF4 item; "QLoRA Explained",
 *     devtoolshub.net, section NF4).
 *   - Quantisation constants and their double quantisation (same QLoRA page,
 *     How It Works, Double Quantization item; "QLoRA Explained", section
 *     Double Quantization).
 *   - Dequantisation of every 4-bit weight back to 16-bit (QLoRA page, How It
 *     Works; AQLoRA paper listing, arxivdaily.com, English abstract).
 *   - AQLoRA's single pass: rank layers by NF4 reconstruction error and keep
 *     the top-K in 16-bit under a memory budget, from the weights alone
 *     (AQLoRA listing, English abstract; "AQLoRA: A Zero-Search Recipe for
 *     Fast Quantized LoRA Fine-Tuning", aitrending.vip, Technical Details).
 *
 * Format (the readings taken where the pages are silent):
 *   - blocks of 64 consecutive elements of the flattened row-major matrix
 *     (the last block may be partial); constant = the block's largest |x| in
 *     fp32 ("absmax");
 *   - code of x = number of the 15 nearest-level thresholds strictly below
 *     s = fl32(x * fl32(1/absmax)); ascending level order, code 7 = 0.0;
 *     an all-zero block encodes to 7 (for a subnormal absmax the oracle
 *     scales x and absmax by 2^64 first, the kernels do so below 2^-100: an
 *     exact power-of-two scaling that changes no code);
 *   - codes packed two per byte, element 2j in the low nibble of byte j, an
 *     odd final element leaves the high nibble 0;
 *   - double quantisation (dq_group = 256): per matrix, groups of 256
 *     consecutive absmax values; scale2 = fl32(G/127) with G the group's
 *     largest absmax; qabsmax = rint(fl32(absmax/scale2)) as int8 (ties to
 *     even); the dequantised constant is fl32(qabsmax * scale2).  Codes
 *     always use the exact absmax;
 *   - dequantised value = round-to-nearest-even to the input's 16-bit type of
 *     fl32(level[code] * constant);
 *   - reconstruction error of a matrix = sum over its elements of
 *     (x - dequantised x)^2.  The kernels accumulate it in fp32 over each
 *     lane's 64 weights (8 consecutive weights from each of 8 blocks of one
 *     wave's 64), then in fp64 across the lanes of a wave, the waves of a
 *     16,384-weight tile and the tiles of the matrix, in a fixed order
 *     (bitwise reproducible); in a wave where a block's absmax is below
 *     2^-40 or at least 2^40 each difference is scaled by an exact power of
 *     two before squaring and the lane's fp32 sum per block is unscaled in
 *     fp64, so the squares neither underflow nor overflow.  Within 1e-5
 *     relative of the oracle's exact fp64 sum (observed <= 2e-8);
 *   - promotion cost = 2n - NF4 bytes; ranking by error descending, equal
 *     errors by index ascending; K = the longest prefix of that order whose
 *     running cost stays within the budget (and within the count cap).
 *
 * Conventions for every call:
 *   - Buffers named "device" are device pointers the caller allocated and
 *     owns; the library never allocates or frees device memory and keeps no
 *     pointer after it returns (nf4_layer_error_noalloc uses a fixed device
 *     array of the library instead of a workspace).  `stream` is a
 *     hipStream_t (NULL = the null stream); calls only enqueue work on it
 *     and return -- the caller synchronises.  Every device buffer must stay alive until that work is
 *     done.  The nf4_layer array is host memory, copied into the workspace
 *     before the call returns; the caller may reuse it at once.
 *   - `ws` is caller-provided device scratch of at least the size the matching
 *     *_workspace_bytes helper returns (256-byte aligned).  Calls on one stream
 *     may share a workspace; concurrent calls on different streams need their
 *     own.
 *   - All argument checks run on the host before anything is enqueued; on an
 *     error nothing is enqueued and no output is touched.  No call prints,
 *     throws or aborts.  A failed HIP call returns NF4_E_HIP and its code is
 *     kept per thread for nf4_last_hip_error().  Faults inside kernels surface
 *     at the caller's next synchronisation.
 *   - Inputs must be finite; NaN/Inf weights or errors give unspecified
 *     (but memory-safe) results.
 *   - Outputs are bitwise deterministic run to run.
 */
#ifndef NF4_H
#define NF4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* The HIP stream handle, declared as hip_runtime_api.h declares it, so that
 * this header needs no HIP include. */
typedef struct ihipStream_t* hipStream_t;

#define NF4_ABI_VERSION 5

typedef enum {
    NF4_OK = 0,
    NF4_E_ARG = 1,          /* NULL where required, nl <= 0, n <= 0, sizes out of range   */
    NF4_E_ALIGN = 2,        /* a pointer violates its alignment                           */
    NF4_E_UNSUPPORTED = 3,  /* blocksize != 64, dq_group not in {0, 256}, bad dtype       */
    NF4_E_WORKSPACE = 4,    /* ws NULL, misaligned, or ws_bytes too small                 */
    NF4_E_HIP = 5           /* a HIP runtime call or launch failed                        */
} nf4_status;

typedef enum { NF4_BF16 = 0, NF4_FP16 = 1 } nf4_dtype;

/* Codec variants: kind of the second-level quantisation of the constants. */
typedef enum {
    NF4_DQ_NONE = 0,       /* fp32 absmax per block                                       */
    NF4_DQ_INT8 = 1,       /* int8 per block + fp32 scale per 256 blocks, symmetric        */
    NF4_DQ_INT8_MEAN = 2,  /* as INT8, of the absmax minus the matrix's mean absmax        */
    NF4_DQ_E4M3_MEAN = 3   /* 8-bit float E4M3 of the absmax minus the mean, fp32 scale    */
} nf4_dq_kind;

typedef struct {
    int32_t dtype;      /* nf4_dtype                                   */
    int32_t blocksize;  /* 32, 64, 128 or 256                          */
    int32_t dq_kind;    /* nf4_dq_kind; groups of 256 blocks           */
} nf4_variant;

/* Budget rules of aqlora_select. */
typedef enum {
    AQLORA_PREFIX = 0,  /* take units in rank order, stop at the first that does not fit */
    AQLORA_FILL = 1     /* take every unit, in rank order, that still fits               */
} aqlora_rule;

typedef struct {
    int32_t dtype;      /* nf4_dtype of the 16-bit weights (and of dequantised output)  */
    int32_t blocksize;  /* must be 64                                                   */
    int32_t dq_group;   /* 0 = no double quantisation, 256 = int8 + fp32 per 256 blocks */
} nf4_format;

/* One weight matrix ("layer"), flattened row-major, n elements, nb = ceil(n/64)
 * blocks, ng = ceil(nb/256) groups.  Which fields a call reads or writes is
 * listed at each call; unused fields may be NULL.  The codec calls take
 * fewer than 2^31 - 2^20 tiles of 16,384 weights in total (sum of
 * ceil(n/16384) over the matrices of one call), else NF4_E_UNSUPPORTED. */
typedef struct {
    int64_t     n;        /* elements, 1 <= n < 2^40                                   */
    const void* w;        /* device [n] 16-bit weights, 16-byte aligned                */
    uint8_t*    codes;    /* device [ceil(n/2)] packed codes, 16-byte aligned          */
    float*      absmax;   /* device [nb] exact fp32 block absmax, 4-byte aligned       */
    int8_t*     qabsmax;  /* device [nb] int8 double-quantised absmax                  */
    float*      scale2;   /* device [ng] fp32 second-level scales, 4-byte aligned      */
    void*       out;      /* device [n] 16-bit dequantised output, 16-byte aligned     */
} nf4_layer;

/* Blockwise NF4 quantisation of nl matrices in one grouped launch: the
 * 4-bit NormalFloat codes and their per-block constants ("QLoRA" paper
 * summary page, ai360xpert.com, How It Works, NF4 item; "QLoRA Explained",
 * devtoolshub.net, NF4).  Reads w; writes codes and absmax; with
 * dq_group == 256 also writes qabsmax and scale2 (double quantisation fused
 * into the same pass).  Required: w, codes, absmax; qabsmax and scale2 when
 * dq_group == 256.  ws: the descriptor table and an 8-byte record per
 * 16,384-weight tile (nf4_workspace_bytes is enough). */
nf4_status nf4_quantize(const nf4_layer* layers, int32_t nl, nf4_format fmt,
                        void* ws, size_t ws_bytes, hipStream_t stream);

/* Double quantisation of existing absmax constants: the quantisation
 * constants quantised again (QLoRA page, How It Works, Double Quantization
 * item; "QLoRA Explained", Double Quantization); dq_group must be 256.
 * Reads absmax; writes qabsmax and scale2.  ws: the descriptor table. */
nf4_status nf4_double_quant(const nf4_layer* layers, int32_t nl, nf4_format fmt,
                            void* ws, size_t ws_bytes, hipStream_t stream);

/* Dequantisation to the 16-bit type fmt.dtype: the 4-bit weight turned back
 * into 16 bits, as QLoRA does on the fly for the forward and backward pass
 * (QLoRA page, How It Works) and as every non-promoted layer still needs
 * under AQLoRA (AQLoRA paper listing, arxivdaily.com, English abstract).
 * Reads codes and either absmax (dq_group == 0) or qabsmax + scale2
 * (dq_group == 256); writes out.  ws: at least the table and one 32-byte
 * record per tile of these layers (nf4_workspace_bytes of them, or of any
 * superset, is enough). */
nf4_status nf4_dequantize(const nf4_layer* layers, int32_t nl, nf4_format fmt,
                          void* ws, size_t ws_bytes, hipStream_t stream);

/* nf4_dequantize of the matrices a selection left in NF4 form, with the
 * selection on the device: matrix i is dequantised iff skip[i] == 0, and the
 * out buffer of a matrix with skip[i] != 0 is not touched.  Passing
 * aqlora_select_topk's (or aqlora_select's) `selected` array as skip gives
 * AQLoRA's step: the promoted matrices keep their 16-bit weights and skip
 * dequantisation (AQLoRA listing, English abstract), with no host round trip
 * between the selection and the dequantisation.  skip: device uint8[nl], read
 * in stream order (NULL: NF4_E_ARG).  Every matrix needs its out pointer and
 * constants as for nf4_dequantize; ws as for nf4_dequantize over all nl
 * matrices. */
nf4_status nf4_dequantize_masked(const nf4_layer* layers, int32_t nl, nf4_format fmt,
                                 const uint8_t* skip, void* ws, size_t ws_bytes,
                                 hipStream_t stream);

/* The fused single pass: quantise (+ double-quantise), dequantise in
 * registers with the constants the user gets back, and score each matrix by
 * its NF4 reconstruction error -- AQLoRA's one pass over the weights, from
 * the weights alone (AQLoRA listing, English abstract; "AQLoRA: A
 * Zero-Search Recipe for Fast Quantized LoRA Fine-Tuning", aitrending.vip,
 * Technical Details).
 * Reads w; writes codes, qabsmax and scale2 (dq_group == 256), absmax
 * (required when dq_group == 0, optional -- NULL skips it -- when 256), and
 * err[nl] (device fp64, the reconstruction error of each matrix).  out is not
 * touched. */
nf4_status nf4_layer_error(const nf4_layer* layers, int32_t nl, nf4_format fmt,
                           double* err, void* ws, size_t ws_bytes, hipStream_t stream);

/* nf4_layer_error without a workspace argument, for callers that cannot
 * allocate device memory (code that must not call hipMalloc: graph capture,
 * tight serving loops, harnesses that forbid it).  Same arguments, checks and
 * results as nf4_layer_error (the same kernels); its workspace is a fixed
 * file-scope device array of nf4_noalloc_scratch_bytes() (32 MiB) that each
 * GPU holds from the first call on it until the process ends.  That bounds
 * the call to its workspace within 32 MiB: 64 bytes per matrix plus 8 bytes
 * of tile record and 32 bytes of partials per 16,384-weight tile (each part
 * rounded up to 256 bytes), about 8.4e5 tiles or 1.37e10 weights; a larger
 * call returns NF4_E_WORKSPACE before anything is enqueued.  Nothing is allocated or freed: no hipMalloc,
 * hipFree or allocating library routine.  The scratch needs no clearing (the
 * table is copied in and every partial is written before it is read).  Every
 * call on one GPU shares that GPU's array, so calls that overlap on one GPU
 * (different streams, or host threads, without ordering between them) race
 * and give undefined results; calls ordered on one stream are safe. */
nf4_status nf4_layer_error_noalloc(const nf4_layer* layers, int32_t nl, nf4_format fmt,
                                   double* err, hipStream_t stream);
/* Size in bytes of nf4_layer_error_noalloc's fixed per-device scratch. */
size_t nf4_noalloc_scratch_bytes(void);

/* nf4_layer_error plus sumsq[nl] (device fp64): the sum of x^2 over each
 * matrix, the denominator of the relative score err / sumsq.  The pages rank
 * by reconstruction error without fixing a normalisation ("AQLoRA" arXiv
 * listing, English abstract); the normalised scores are variants of that
 * score.  Same precision and order as err (fp32 over each lane's 64 weights,
 * fp64 beyond); err is bitwise the same as nf4_layer_error's.  The same pass,
 * about one more instruction per weight.  sumsq must be non-NULL, 8-byte
 * aligned. */
nf4_status nf4_layer_error_norm(const nf4_layer* layers, int32_t nl, nf4_format fmt,
                                double* err, double* sumsq, void* ws, size_t ws_bytes,
                                hipStream_t stream);

/* Budgeted top-K over per-layer scores, on the device: rank the matrices by
 * reconstruction error and keep the leading ones in 16 bits while the memory
 * budget allows (AQLoRA listing, English abstract; aitrending page,
 * Technical Details: the budget is a setting).
 *   err[nl]   device fp64 scores (finite, as written by nf4_layer_error)
 *   cost[nl]  device int64 promotion costs (aqlora_promote_cost)
 *   budget_bytes  < 0: no byte budget;  k_cap < 0: no count cap
 *   selected[nl]  device uint8, 1 for promoted layers, 0 otherwise
 *   k_out         device int32, K
 * 1 <= nl <= 65536. */
nf4_status aqlora_select_topk(const double* err, const int64_t* cost, int32_t nl,
                              int64_t budget_bytes, int32_t k_cap,
                              uint8_t* selected, int32_t* k_out,
                              void* ws, size_t ws_bytes, hipStream_t stream);

/* Selection variants on the device.  The pages keep the top-K layers under a
 * memory budget, and their speed setting adapts only the top blocks
 * ("AQLoRA" arXiv listing, English abstract; "AQLoRA: A Zero-Search
 * Recipe...", Technical Details); the options read those words:
 *   denom[nl]   device fp64 or NULL: layer i scores err[i] / denom[i] (IEEE
 *               fp64), e.g. n for the mean squared error, sumsq from
 *               nf4_layer_error_norm for the relative error; each > 0 and
 *               finite, else the scores are unspecified.  NULL: err[i].
 *   group_end   HOST int32[ngroups] or NULL: units are groups of consecutive
 *               layers (group g = layers group_end[g-1] .. group_end[g]-1,
 *               group_end[-1] = 0; strictly increasing, last == nl), e.g. the
 *               matrices of each transformer block, scored by the sum of their
 *               layers' scores in layer order and costed by the sum of their
 *               costs, and promoted whole.  Copied before the call returns.
 *               NULL: units are single layers (ngroups ignored).
 *   rule        AQLORA_PREFIX or AQLORA_FILL.
 * Units are ranked by score descending, equal scores by unit index ascending;
 * k_cap (< 0: none) caps the number of units, budget_bytes (< 0: none) their
 * total cost.  Writes selected[nl] per layer (1 = promoted) and k_out = the
 * number of units taken.  With denom and group_end NULL and AQLORA_PREFIX
 * this is aqlora_select_topk.  1 <= nl <= 65536; bad group_end or rule:
 * NF4_E_ARG; ws of aqlora_workspace_bytes(nl). */
nf4_status aqlora_select(const double* err, const double* denom, const int64_t* cost,
                         int32_t nl, const int32_t* group_end, int32_t ngroups,
                         int64_t budget_bytes, int32_t k_cap, int32_t rule,
                         uint8_t* selected, int32_t* k_out,
                         void* ws, size_t ws_bytes, hipStream_t stream);

/* Codec variants ("QLoRA" paper summary page, How It Works, Double
 * Quantization item; "QLoRA Explained", Double Quantization: the constants
 * are quantised again, without saying how).  Block size 32/64/128/256 and:
 *   NF4_DQ_NONE      a' = a;
 *   NF4_DQ_INT8      s2 = fl32(G/127) per 256 blocks (G their largest absmax),
 *                    q = clamp(rint(fl32(a/s2))), a' = fl32(q s2);
 *   NF4_DQ_INT8_MEAN c = fl32(a - mu), s2 = fl32(max|c|/127), q as above of
 *                    fl32(c/s2), a' = fl32(fl32(q s2) + mu);
 *   NF4_DQ_E4M3_MEAN as INT8_MEAN with s2 = fl32(max|c|/448) and q the nearest
 *                    E4M3 value (ties to even, sign kept) of fl32(c/s2);
 *   mu = fl32(S/nb), S the fp64 sum in group order of each group's fp64 sum of
 *   its absmax values in block order.
 * Codes use the exact absmax (the encode rule of the main codec with the block
 * size changed); y = RNE16(fl32(level[code] a')); err = sum (x - y)^2 (fp64).
 * layers: w (read, 16-byte aligned), codes (16-byte aligned), absmax (written:
 * [ceil(n/block)] fp32), and for kinds 1-3 qabsmax (one byte per block: the
 * int8, or the E4M3 encoding) and scale2 ([ceil(nb/256)] fp32).  mean: device
 * fp32 [nl], written for kinds 2-3 (may be NULL otherwise).  err: device fp64
 * [nl].  ws: nf4_workspace_bytes_variant.  The main codec (nf4_layer_error)
 * is the fused fast path; this one takes three launches (absmax; mean;
 * second level + encode + dequantise + error). */
nf4_status nf4_layer_error_variant(const nf4_layer* layers, int32_t nl, nf4_variant v,
                                   float* mean, double* err, void* ws, size_t ws_bytes,
                                   hipStream_t stream);

/* Dequantisation of a variant's codes: reads codes, absmax (kind 0) or
 * qabsmax + scale2 (+ mean for kinds 2-3); writes out (16-byte aligned).
 * ws: at least the table and one 64-byte record per group of these layers
 * (nf4_workspace_bytes_variant of them, or of any superset, is enough). */
nf4_status nf4_dequantize_variant(const nf4_layer* layers, int32_t nl, nf4_variant v,
                                  const float* mean, void* ws, size_t ws_bytes, hipStream_t stream);

/* NF4 dequantisation fused into the 16-bit matmul that consumes the weight,
 * on the matrix cores.  QLoRA dequantises the 4-bit weight on the fly for the
 * forward and the backward pass ("QLoRA" paper summary page, How It Works);
 * AQLoRA names that as where quantised fine-tuning loses its time ("AQLoRA"
 * arXiv listing, English abstract).  The weight tile is dequantised into
 * on-chip memory, to exactly the 16-bit values nf4_dequantize writes, and
 * multiplied there; the 16-bit weight never goes to memory.
 *   w        one matrix W [rows x cols] (w->n == rows * cols), row-major, in
 *            its NF4 form: codes, and qabsmax + scale2 (dq_group 256) or absmax
 *   backward 0: out[m x rows] = x[m x cols] * W^T   (forward, y = x W^T)
 *            1: out[m x cols] = x[m x rows] * W     (input gradient, dx = dy W)
 *   x        device [m x (cols | rows)] in fmt.dtype (bf16 or fp16),
 *            row-major, 16-byte aligned
 *   out      device [m x (rows | cols)], row-major, 16-byte aligned:
 *            fp32 (out_fp32 = 1) or fmt.dtype rounded to nearest even (0)
 * Products of two bf16 or two fp16 values are exact in fp32; the sums are
 * fp32 (matrix core accumulation).  rows, cols must be multiples of 128
 * (else NF4_E_UNSUPPORTED); 1 <= m < 2^31; codes 16-byte aligned.  No
 * workspace; enqueues only.  Deterministic run to run. */
nf4_status nf4_matmul(const nf4_layer* w, int64_t rows, int64_t cols, nf4_format fmt,
                      int32_t backward, const void* x, int64_t m, void* out,
                      int32_t out_fp32, hipStream_t stream);

/* nf4_matmul with a caller workspace, for shapes whose output tiles alone do
 * not fill the GPU (few tokens m): the reduction is then split into up to 16
 * parts, each workgroup multiplies one output tile over one part into fp32
 * partials in ws, and a second kernel adds the parts in part order (fixed, so
 * the result is deterministic run to run) and rounds as nf4_matmul does.  The
 * split count is a function of (rows, cols, backward, m) only.  Same
 * arguments and results as nf4_matmul except the summation order; ws: device,
 * 256-byte aligned, at least nf4_matmul_workspace_bytes(rows, cols, backward,
 * m) bytes (NF4_E_WORKSPACE otherwise); when that is 0 the call is
 * nf4_matmul and ws may be NULL.  Error bound as for nf4_matmul:
 * (K/parts + parts) fp32 additions per output instead of K.  Forward with
 * m <= 32 takes a kernel of its own with the same contract: one wave per 16
 * weight rows and part of the reduction (parts of at most 1024 k, 512 k
 * above 16 tokens), fp32 partials in ws added in part order by the same
 * second kernel.  Where the output tiles fill the GPU but leave a last round
 * at most half full (e.g. 4096 tokens through a 13824 x 5120 weight: 320
 * tiles of 256 x 256 on 256 compute units), the whole rounds run unsplit and
 * each leftover tile's reduction is split floor(256 / leftover) ways (at most
 * 16, each part at least 1024 k), into one 256 x 256 fp32 block per (part,
 * tile) in ws, added in part order into out. */
nf4_status nf4_matmul_ws(const nf4_layer* w, int64_t rows, int64_t cols, nf4_format fmt,
                         int32_t backward, const void* x, int64_t m, void* out,
                         int32_t out_fp32, void* ws, size_t ws_bytes, hipStream_t stream);

/* ---- host-only helpers (pure; no HIP calls) ---- */

/* Workspace of nf4_matmul_ws for this shape: parts * m * (rows | cols) fp32
 * partials when the whole reduction is split, parts * leftover tiles * 256 *
 * 256 fp32 when only the leftover tiles' is, rounded up to 256 bytes; 0 when
 * the shape is not split or on bad input. */
size_t      nf4_matmul_workspace_bytes(int64_t rows, int64_t cols, int32_t backward, int64_t m);

/* Workspace for every codec call above over these matrices (the descriptor
 * table, an 8-byte record per 16384-weight tile, and two arrays of 4 fp64
 * partials per tile); 0 on bad input. */
size_t      nf4_workspace_bytes(int32_t nl, const int64_t* n_per_layer, nf4_format fmt);
/* Workspace for aqlora_select_topk and aqlora_select; 0 on bad input. */
size_t      aqlora_workspace_bytes(int32_t nl);
/* Workspace for the variant calls (the table, then the larger of two fp64 per
 * group and one 64-byte record per group); 0 on bad input. */
size_t      nf4_workspace_bytes_variant(int32_t nl, const int64_t* n_per_layer, nf4_variant v);
/* ceil(n/2) + (kind 0 ? 4 nb : nb + 4 ng) + (kinds 2-3 ? 4 : 0); -1 on bad input. */
int64_t     nf4_storage_bytes_variant(int64_t n, nf4_variant v);
/* ceil(n/2) + (dq_group ? nb + 4*ng : 4*nb); -1 on bad input. */
int64_t     nf4_storage_bytes(int64_t n, nf4_format fmt);
/* 2n - nf4_storage_bytes(n, fmt): extra bytes of keeping the matrix 16-bit. */
int64_t     aqlora_promote_cost(int64_t n, nf4_format fmt);
/* The 16 NF4 levels in code order (ascending), as embedded in the kernels. */
void        nf4_levels(float out16[16]);
/* The 15 decision thresholds (fp32), as embedded in the kernels. */
void        nf4_thresholds(float out15[15]);
const char* nf4_status_str(nf4_status s);
int32_t     nf4_abi_version(void);
/* HIP error code (hipError_t value) of the last NF4_E_HIP on this thread. */
int32_t     nf4_last_hip_error(void);

#ifdef __cplusplus
}
#endif
#endif /* NF4_H */
