/*
 * nf4_cpu.h -- the fused NF4 scoring pass on the host CPU (libnf4cpu.so).
 *
 * AQLoRA sets everything with one CPU pass over the weights, in seconds
 * ("AQLoRA" arXiv listing, English abstract; "AQLoRA: A Zero-Search
 * Recipe...", TL;DR).  This library is that pass on the host cores, for
 * comparison with the GPU pass of nf4.h; it is a separate entry point, never
 * a fallback of the GPU calls.  Types and status codes are those of nf4.h.
 */
#ifndef NF4_CPU_H
#define NF4_CPU_H

#include "nf4.h"

#ifdef __cplusplus
extern "C" {
#endif

/* nf4_layer_error on HOST memory: every pointer of layers[] and err point to
 * host memory.  Reads w; writes codes, qabsmax and scale2 (dq_group 256),
 * absmax (required without double quant, optional -- NULL skips it -- with),
 * and err[nl] (fp64 reconstruction error per matrix).  Codes and constants
 * equal the GPU pass's bit for bit; err is summed in fp64 (per 16384-weight
 * tile in element order, then the tiles in order).  threads <= 0: the OpenMP
 * default.  Synchronous.  NF4_E_ARG on NULL/size errors, NF4_E_UNSUPPORTED on
 * formats other than block 64 with dq_group 0 or 256, bf16 or fp16.  Uses an
 * AVX-512 code path when the CPU has it (same outputs bit for bit); the
 * environment variable NF4_CPU_ISA=avx2 selects the AVX2 path instead. */
nf4_status nf4_cpu_layer_error(const nf4_layer* layers, int32_t nl, nf4_format fmt,
                               double* err, int32_t threads);

/* Threads an unrestricted call would use. */
int32_t nf4_cpu_max_threads(void);

#ifdef __cplusplus
}
#endif
#endif /* NF4_CPU_H */
