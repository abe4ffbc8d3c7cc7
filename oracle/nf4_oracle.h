/*
 * nf4_oracle.h -- plain, slow, single-threaded CPU reference for the NF4 weight
 * codec and the AQLoRA layer ranking.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the CPU
 * baseline leg of the benchmark may load this library.  The product path (the
 * HIP library and its Python binding) never calls it, and the two share no
 * code, header, table or constant.
 *
 * Sources (cited by page title and section throughout):
 *   [QLoRA page]      "QLoRA" paper summary (ai360xpert.com), sections
 *                     "The Idea" and "How It Works".
 *   [QLoRA explained] "QLoRA Explained" (devtoolshub.net), sections
 *                     "4-Bit Quantization in QLoRA", "NF4", "Double Quantization".
 *   [AQLoRA abstract] arXiv listing of the AQLoRA paper (arxivdaily.com),
 *                     English abstract.
 *   [AQLoRA summary]  "AQLoRA: A Zero-Search Recipe for Fast Quantized LoRA
 *                     Fine-Tuning" (aitrending.vip), TL;DR and Technical Details.
 *
 * Where the pages leave a step open the plainest reading is taken; every such
 * reading is listed in the design notes and in the comment of the function that
 * applies it.  Parity of the NF4 level construction (the quantile offset and the
 * 8-positive / 7-negative split) is not fixed by the pages: "parity unpinned"
 * as far as the pages go; it is pinned to library normal quantiles in the tests.
 */
#ifndef NF4_ORACLE_H
#define NF4_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define NF4O_BLOCK    64   /* elements per absmax block                        */
#define NF4O_DQ_GROUP 256  /* absmax values per second-level (int8) group      */

enum { NF4O_BF16 = 0, NF4O_FP16 = 1 };

/* 16 NF4 levels, ascending, as fp32.  Returns 0. */
int      nf4o_levels(float out16[16]);
/* 15 decision thresholds between neighbouring levels, fp32. */
void     nf4o_thresholds(float out15[15]);
/* 16-bit storage value -> fp32 (exact). */
float    nf4o_from16(uint16_t h, int dtype);
/* fp32 -> 16-bit storage value, round to nearest, ties to even. */
uint16_t nf4o_to16_rne(float f, int dtype);
void     nf4o_to16_rne_array(const float* f, int64_t n, int dtype, uint16_t* out);
/* code of one normalised value s: the number of thresholds strictly below s. */
int      nf4o_encode(float s);
void     nf4o_encode_array(const float* s, int64_t n, uint8_t* out);

/* Blockwise absmax quantisation of one flattened matrix of n elements.
 * codes: ceil(n/2) bytes, element 2j in the low nibble of byte j.
 * absmax: ceil(n/64) exact fp32 block maxima of |x|. */
void     nf4o_quantize(const uint16_t* w, int64_t n, int dtype,
                       uint8_t* codes, float* absmax);
/* Second-level quantisation of the absmax values of one matrix:
 * int8 per block plus one fp32 scale per group of 256 blocks. */
void     nf4o_double_quant(const float* absmax, int64_t nb,
                           int8_t* qabsmax, float* scale2);
/* Dequantise to 16-bit.  If qabsmax is NULL the exact absmax is used,
 * otherwise the double-quantised constant qabsmax*scale2. */
void     nf4o_dequantize(const uint8_t* codes, int64_t n, int dtype,
                         const float* absmax, const int8_t* qabsmax,
                         const float* scale2, uint16_t* out);
/* Sum of squared differences between two 16-bit arrays, in fp64. */
double   nf4o_sse(const uint16_t* w, const uint16_t* y, int64_t n, int dtype);
/* The whole per-matrix scoring pass: quantise (+ double-quantise when dq),
 * dequantise, and return the reconstruction error.  Every intermediate is
 * written to the caller's buffers (qabsmax/scale2 may be NULL when !dq). */
double   nf4o_layer_error(const uint16_t* w, int64_t n, int dtype, int dq,
                          uint8_t* codes, float* absmax, int8_t* qabsmax,
                          float* scale2, uint16_t* y);

/* Bytes of the NF4 form of an n-element matrix, and the extra bytes that
 * keeping it in 16-bit costs over that form. */
int64_t  nf4o_storage_bytes(int64_t n, int dq);
int64_t  nf4o_promote_cost(int64_t n, int dq);
/* Budgeted top-K.  budget < 0: no byte budget; kcap < 0: no count cap.
 * Writes selected[nl] (0/1) and returns K. */
int      nf4o_select_topk(const double* err, const int64_t* cost, int nl,
                          int64_t budget, int kcap, uint8_t* selected);

/* Selection variants.  Sum of x^2 over a matrix in fp64 (the relative score's
 * denominator), and the general selection: optional per-layer divisor of the
 * error, optional groups of consecutive layers (group_end[g] = one past the
 * group's last layer), rule 0 = stop at the first unit that does not fit,
 * rule 1 = skip it and keep filling.  Returns the number of units taken. */
double   nf4o_sumsq(const uint16_t* w, int64_t n, int dtype);

/* Codec variants: block size 32/64/128/256 and the second-level kind (0 none,
 * 1 int8 symmetric, 2 int8 with the matrix's mean absmax subtracted, 3 E4M3
 * 8-bit float with the mean subtracted), groups of 256 blocks.  q holds the
 * int8 or E4M3 byte per block; mean (may be NULL) receives mu (0 for kinds
 * 0 and 1).  Returns the reconstruction error; y receives the dequantised
 * values. */
float    nf4o_e4m3_decode(uint8_t b);
uint8_t  nf4o_e4m3_encode(float v);
int64_t  nf4o_storage_bytes_ex(int64_t n, int block, int kind);
double   nf4o_layer_error_ex(const uint16_t* w, int64_t n, int dtype, int block, int kind,
                             uint8_t* codes, float* absmax, uint8_t* q, float* scale2,
                             float* mean, uint16_t* y);
int      nf4o_select(const double* err, const double* denom, const int64_t* cost, int nl,
                     const int32_t* group_end, int ngroups, int64_t budget, int kcap,
                     int rule, uint8_t* selected);

#ifdef __cplusplus
}
#endif
#endif
