// coli_dec.h -- host interface of the decode expert kernels (coli_dec.hip).
#ifndef COLI_DEC_H
#define COLI_DEC_H

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace coli {

// Activation "row tables": one row per activation row, kpad elements (the
// input width rounded up to 1024, zeros past it) stored as bf16 hi/lo pairs
// in fragment order -- chunk c (8 elements) is the 32-byte run of its hi unit
// and its lo unit, so a row is 4 * kpad bytes.
inline int64_t dec_row_bytes(int64_t kpad) { return 4 * kpad; }

// Rows per pass of the decode kernels (two MFMA N-tiles of 8 rows, each row
// a bf16 hi/lo column pair).
constexpr int kDecTpp = 16;

// Groups: group g < ngroups is expert g, whose rows are the grouped rows
// offsets[g] .. offsets[g+1]-1; group ngroups (when has_extra) is the shared
// expert, rows x_row0 .. x_row0 + x_rows - 1.  The work list (built on the
// device) holds one entry g | pass << 11 per group-pass, a pass being up to
// kDecTpp rows of one group; *n_work is the number of entries.
struct DecArgs {
    const uint8_t *w[2];
    const float *s[2];
    int64_t w_gstride, s_gstride;
    int ngroups, O;
    const uint8_t *xw[2];   // the extra (shared) group's matrices
    const float *xs[2];
    int has_extra, xO, x_rows, x_row0;
    int I, kpad;
    int64_t rb;
    const int *offsets;
    const int *row_pair;
    int K;
    // activation row of grouped row r: its token (row_pair[r] / K; the extra
    // group's rows are tokens 0..x_rows-1) when act_by_token, else r itself
    int act_by_token;
    const uint16_t *act;     // row table of the activations
    const int *work;
    const int *n_work;
    float *out;              // fp32 result rows (grouped row r at out + r * ldo)
    int64_t ldo;
    int out_vec4;            // out rows may be written with 16-byte stores
    // M == 2 only: the result also written as the next product's row table
    // (rows = grouped rows, kpad = hf_kpad, same weight format)
    uint16_t *hf;
    int hf_kpad;
    int tiled;               // weights in the tiled layout (coli_pack_tiled); w_gstride
                             // is then the tiled bytes of one matrix
    // grouped-scale int4 (0: one scale per row): steps of 32 elements per
    // group, and groups per row of the packed scales ([row tile][gs_ngp][16]
    // floats per matrix, s_gstride floats apart); weights in the grouped tiled
    // layout (coli_pack_tiled_grouped)
    int gs_spg, gs_ngp;
    int tiles;               // set by dec_launch
};

// x [rows, ldx] fp32 -> row table (rows x 4 kpad bytes) for weight format fmt.
hipError_t xrows_launch(int fmt, const float *x, int64_t ldx, int rows, int I, int kpad,
                        uint16_t *table, hipStream_t st);
// M = 2: h = silu(gate . x) * (up . x); M = 1: y = down . h.
hipError_t dec_launch(DecArgs a, int fmt, int M, int64_t max_group_passes, hipStream_t st);
int dec_rows_per_block(int M);

}  // namespace coli

#endif
