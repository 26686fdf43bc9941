// coli_idot.h -- host interface of the integer-dot qgemv (coli_idot.hip).
#ifndef COLI_IDOT_H
#define COLI_IDOT_H

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace coli {

// Quantised activation rows: kq = I rounded up to 256 int8 values per row in
// the product's fragment order, then the per-row scales (fp32) and the sums of
// the quantised values (int32, four partial sums per row -- one per
// 4096-element part -- added in order where int4 weights need them).
inline int64_t idot_row_bytes(int64_t I) { return (I + 255) / 256 * 256; }
int64_t idot_workspace_bytes(int S, int I);

struct IdotArgs {
    const uint8_t *W;     // [O, rb] packed rows, rb % 16 == 0
    const float *scale;   // [O]
    const float *x;       // [S, I]
    float *y;             // [S, O]
    int S, I, O;
    int64_t rb;
    int nkb;              // k-blocks per row (set by idot_launch)
    int64_t kq;           // quantised row length (bytes)
    int8_t *table;        // [S, kq] quantised rows
    float *sx;            // [S]
    int *sq;              // [S, 4]: partial sums of the quantised values per 4096-element part
    int y_vec4;
};

// fmt: kI8 or kI4.  Returns hipErrorInvalidValue for shapes outside the
// kernels' range (checked by the caller first).
hipError_t idot_launch(IdotArgs a, int fmt, hipStream_t st);
int idot_max_kblocks_per_wave();
int idot_kblock(int fmt);

// rows rows of x [rows, I] quantised into table [rows, kq] (fragment order
// of fmt, zeros past I), sx [rows] and sq [rows, 4]; I <= kq <= 16384, kq a
// multiple of 256.
hipError_t qrow_launch(int fmt, const float *x, int rows, int I, int64_t kq, int8_t *table, float *sx,
                       int *sq, hipStream_t st);

// Integer-dot grouped expert products for prefill batches (tiled weights):
// the same groups, passes, classes and items as the bf16 prefill kernels
// (coli_pre.h), with the activations quantised to int8 per row.
//   M = 2: h[r, o] = silu(g) * u, g = ((float)dot_g * sg[o]) * sx_r, u alike
//   M = 1: y[r, o] = ((float)dot_d * sd[o]) * sx_r
// dot: the exact int32 dot of the weight values with the row's int8 values.
struct PreIdArgs {
    const uint8_t *w[2];
    const float *s[2];
    int64_t w_gstride, s_gstride;   // tiled bytes of one matrix; scales per group
    int ngroups, O;
    const uint8_t *xw[2];           // the extra (shared) group's matrices
    const float *xs[2];
    int has_extra, xO, x_rows, x_row0;
    int I;                          // product width (elements)
    int64_t rb;                     // packed row bytes
    int64_t kq;                     // quantised row bytes (idot_row_bytes(I))
    const int *offsets;
    const int *work;
    const int *n_work;
    const int *act_row;             // table row of grouped row r (NULL: r)
    const float *row_sx;            // [grouped row] its row's scale
    const int *row_sq;              // [grouped row] its row's sum of int8 values
    const int8_t *act;              // quantised table
    float *out;                     // fp32 result rows (grouped row r at out + r * ldo)
    int64_t ldo;
    int out_vec4;
    int tiles;                      // set by preid_launch
};
// Per grouped row r: the table row t (gate/up: the token of slot
// row_pair[r] for r < P, then the shared expert's tokens; down: r itself,
// act_row NULL), row_sx[r] = sx[t], row_sq[r] = the sum of t's four partial
// sums in order.
hipError_t idrows_launch(const int32_t *row_pair, int P, int K, int S, int rows, const float *sx,
                         const int *sq, int32_t *act_row, float *row_sx, int *row_sq, hipStream_t st);
hipError_t preid_launch(PreIdArgs a, int fmt, int M, int64_t max_group_passes, hipStream_t st);

}  // namespace coli

#endif
