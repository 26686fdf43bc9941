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

}  // namespace coli

#endif
