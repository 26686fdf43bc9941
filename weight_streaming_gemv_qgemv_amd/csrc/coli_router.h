// coli_router.h -- host interface of the router kernels (coli_router.hip).
#ifndef COLI_ROUTER_H
#define COLI_ROUTER_H

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "coli_internal.h"

namespace coli {

// part: fp64 scratch of coli__router_partial_bytes(S, E, D) bytes.
hipError_t router_launch(const float *Wr, const float *bias, const float *x, int S, int E,
                         int D, int K, int norm_topk, float routed_scale, float topp,
                         int32_t *idx, float *w, int32_t *keff, float *sig, double *part,
                         hipStream_t st);

}  // namespace coli

#endif
