// coli_mfma.h -- host interface of the matrix-core grouped kernels (coli_mfma.hip).
#ifndef COLI_MFMA_H
#define COLI_MFMA_H

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace coli {

// Groups as in GemvArgs (coli_gemv.h); activations come prepared: hi/lo bf16
// planes xq[row][2][xld] in the weights' slot order, and sum(hi + lo) per row
// as the sum of xsum_parts partial arrays (stride xsum_stride).
struct MmArgs {
    const uint8_t *w[2];
    const float *s[2];
    int64_t w_gstride, s_gstride;
    int ngroups, O;
    const uint8_t *xw[2];
    const float *xs[2];
    int has_extra, xO, x_rows, x_row0;
    int I;
    int64_t rb;
    const int *offsets;
    const int *row_pair;
    int K, xrow_token;
    const uint16_t *xq;
    int64_t xld;
    const float *xsum;
    int xsum_parts;
    int64_t xsum_stride;
    const int *work;     // (g | pass << 11) per group-pass, NULL = one group
    const int *n_work;
    float *out;
    int64_t ldo;
    // M == 2 only: the result also as hi/lo planes for the next product
    uint16_t *hq;
    int64_t hq_ld;
    int hq_rows;         // rows of hq written per output row (zeros past O)
    int hq_fmt;          // slot order of the next product's weights
    float *hsum_part;    // [tiles][hsum_stride] partial sums of hi + lo
    int64_t hsum_stride;
    int tiles;           // set by mm_launch
};

int mm_kblock(int fmt);
int mm_rows_per_block();
hipError_t xprep_launch(int fmt, const float *x, int64_t ldx, int rows, int I, int ld,
                        uint16_t *xq, float *xsum, hipStream_t st);
hipError_t mm_launch(MmArgs a, int fmt, int M, int64_t max_group_passes, hipStream_t st);
hipError_t build_work_launch(const int32_t *offsets, int E, int extra_rows, int32_t *work,
                             int32_t *n_work, hipStream_t st);

}  // namespace coli

#endif
