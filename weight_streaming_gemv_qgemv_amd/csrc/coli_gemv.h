// coli_gemv.h -- host interface of the grouped VALU GEMV kernel (coli_gemv.hip).
#ifndef COLI_GEMV_H
#define COLI_GEMV_H

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace coli {

// One launch covers `ngroups` routed groups (+1 extra group when has_extra).
// Group g's activation rows are the grouped rows offsets[g]..offsets[g+1]-1
// (offsets == NULL: one group of x_rows rows starting at row 0); the extra
// group's rows are x_row0 .. x_row0 + x_rows - 1.  The output row of grouped
// row r is out + r * ldo.  M = 2 computes silu(matrix0 . x) * (matrix1 . x).
struct GemvArgs {
    const uint8_t *w[2];
    const float *s[2];
    int64_t w_gstride;   // bytes between consecutive groups' matrices
    int64_t s_gstride;   // floats between consecutive groups' scale vectors
    int ngroups;
    int O;
    const uint8_t *xw[2];
    const float *xs[2];
    int has_extra, xO, x_rows, x_row0;
    int I;
    int64_t rb;
    const int *offsets;
    const int *row_pair;
    int K;
    int xrow_token;      // x row of grouped row r is row_pair[r] / K (extra group: its token)
    const float *x;
    int64_t ldx;
    int x_vec4;          // x rows may be read with 16-byte loads
    float *out;
    int64_t ldo;
    int aligned;         // every weight row starts on a 16-byte boundary
    // filled by gemv_launch
    int tiles, lpr, ich;
};

// max_rows_per_group: an upper bound of the rows any group has in the common
// case (it picks the token-pass width, up to 8; larger groups take several
// passes).
hipError_t gemv_launch(GemvArgs a, int fmt, int M, int max_rows_per_group, hipStream_t st);

}  // namespace coli

#endif
