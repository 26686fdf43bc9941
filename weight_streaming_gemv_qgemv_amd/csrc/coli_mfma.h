// coli_mfma.h -- host interface of the matrix-core grouped kernels (coli_mfma.hip).
#ifndef COLI_MFMA_H
#define COLI_MFMA_H

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace coli {

// Groups as in GemvArgs (coli_gemv.h).  Work is a list of (group, pass)
// entries, a pass being up to `tpp` rows of one group: 8 in fp32 precision
// (bf16 hi/lo column pairs), 16 in bf16 precision (one column each).  Every
// pass has its activations prepared fragment-major in xf (xf_stride elements
// per pass, kpad = input width rounded up to 1024) and the sum of the stored
// values per token in xsum (indexed pass * 16 + token).
struct MmArgs {
    const uint8_t *w[2];
    const float *s[2];
    int64_t w_gstride, s_gstride;
    int ngroups, O;
    const uint8_t *xw[2];
    const float *xs[2];
    int has_extra, xO, x_rows, x_row0;
    int I, kpad;
    int64_t rb;
    const int *offsets;
    const int *row_pair;
    int K, xrow_token;
    uint16_t *xf;
    int64_t xf_stride;
    float *xsum;         // [group-pass * 16 + token] sum(hi + lo) of the activations
    int tpp;             // rows per pass: 8 (fp32, hi/lo) or 32 (bf16)
    int bf16;            // activations rounded once to bf16 (no lo part)
    const int *work;     // (g | pass << 11) per group-pass, NULL = one group
    const int *n_work;
    float *out;
    int64_t ldo;
    int out_vec4;        // out rows may be written with 16-byte stores
    // M == 2 only: the result also prepared as the next product's activations
    uint16_t *hf;
    int64_t hf_stride;
    int hf_rows;         // outputs written per token (zeros past O), = next kpad;
                         // laid out for a product of the same weight format
    float *hsum;         // [tiles][hsum_stride] partial sums per pass * 16 + token
    int64_t hsum_stride;
    int tiles;           // set by mm_launch
};

// Output rows per item of the paired (M = 2) or single (M = 1) product.
int mm_rows_per_block(int M, int bf16);
// Columns (token slots) per pass: the stride of xsum/hsum per group-pass.
int mm_pass_slots(int bf16);
int64_t mm_kpad(int64_t I);
// One block per possible group-pass (blocks past the device count exit).
hipError_t xprep_launch(int fmt, const MmArgs &a, const float *x, int64_t ldx,
                        int64_t max_group_passes, hipStream_t st);
hipError_t mm_launch(MmArgs a, int fmt, int M, int64_t max_group_passes, hipStream_t st);
// out[i] = sum_p parts[p * stride + i] in p order, i < n.
hipError_t sum_parts_launch(const float *parts, int nparts, int64_t stride, int64_t n, float *out,
                           hipStream_t st);


}  // namespace coli

#endif
