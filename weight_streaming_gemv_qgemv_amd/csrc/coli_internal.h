/* coli_internal.h -- declarations shared by libcoli's own translation units
 * (host checks in coli_validate.c, launches in the .hip files).  Not part of
 * the public ABI. */
#ifndef COLI_INTERNAL_H
#define COLI_INTERNAL_H

#include <stddef.h>
#include <stdint.h>

#include "coli.h"

#define COLI_MAX_E 1024 /* 16 scores per lane of a 64-wide wave */
/* slots per chunk of the chunked grouping (batches of more than one chunk) */
#define COLI_GROUP_CHUNK 1024
#define COLI_MAX_K 64
/* rows per pass of the matrix-core expert kernels: in fp32 precision 8, as
 * bf16 hi/lo column pairs of one 16-column MFMA tile; in bf16 precision 64,
 * one column each over four tiles */
#define COLI_MM_TPP_FP32 16
#define COLI_MM_TPP_BF16 64

/* input width of the matrix-core products, rounded up to whole 1024-element
 * k-block groups (the activations are zero past the real width) */
static inline int64_t coli__kpad(int64_t I) { return (I + 1023) / 1024 * 1024; }

#ifdef __cplusplus
extern "C" {
#endif

int coli__check_qgemv(int fmt, const void *W, const float *scale,
                      const float *x, const float *y, int S, int I, int O);
int coli__check_router(const float *Wr, const float *bias, const float *x,
                       int S, int E, int D, int K, int norm_topk,
                       const int32_t *idx, const float *w, const float *sig,
                       const void *ws, size_t ws_bytes);
/* Router logits are summed over d in `splits` slices of `*slice` elements
 * (a multiple of 16), chosen so the fp64 matrix-core grid of
 * coli__router_token_tile(S) x 64 tiles fills the chip; the partial sums
 * need coli__router_partial_bytes() of scratch. */
int coli__router_token_tile(int S);
int coli__router_splits(int S, int E, int D, int *slice);
int64_t coli__router_partial_bytes(int S, int E, int D);

int coli__check_pack(int fmt, const void *W, int64_t count, int O, int I, const void *dst);
int coli__check_pack_scales(const float *S, int64_t count, int O, int I, int gs, const float *dst);
int coli__check_moe(const coli_experts *ex, const coli_mlp *sh, const float *x,
                    int S, int K, const int32_t *idx, const float *w,
                    const float *out, int prec, const void *ws, size_t ws_bytes,
                    int need_routing);

#ifdef __cplusplus
}
#endif

#endif
