// coli_qmv.h -- host interface of the dense matrix-core qgemv (coli_qmv.hip).
#ifndef COLI_QMV_H
#define COLI_QMV_H

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace coli {

struct QmvArgs {
    const uint8_t *W;     // [O, rb] packed rows
    const float *scale;   // [O] (NULL: 1)
    const float *x;       // [S, I]
    float *y;             // [S, O]
    int S, I, O;
    int64_t rb;
    int nkb;              // set by qmv_launch
    int y_vec4;           // set by qmv_launch
    int gs, ng;           // grouped int4: elements per scale group, groups per row
};

// Formats int8 / int4 / int2 with 16-byte row segments, I a multiple of 4,
// W and x 16-byte aligned and the matrix under 4 GB (32-bit row offsets).
bool qmv_supported(int fmt, int64_t rb, int I, int O, const void *W, const float *x);
hipError_t qmv_launch(QmvArgs a, int fmt, hipStream_t st);

// fp32 rows (fmt f32) on the fp32 matrix cores: I a multiple of 4, W and x
// 16-byte aligned (64-bit row offsets: any matrix size).
bool qmv_f32_supported(int I, const void *W, const float *x);
hipError_t qmv_f32_launch(QmvArgs a, hipStream_t st);

// Grouped-scale int4 (scale [O, ceil(I / gs)]): gs 32, 64 or a multiple of
// 128; 16-byte row segments, 16-byte aligned W, scale and x, I <= 12288.
bool qmv_grouped_supported(int64_t rb, int I, int gs, const void *W, const float *scale, const float *x);
hipError_t qmv_grouped_launch(QmvArgs a, hipStream_t st);

}  // namespace coli

#endif
