// coli_pre.h -- host interface of the prefill expert kernels (coli_pre.hip).
#ifndef COLI_PRE_H
#define COLI_PRE_H

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace coli {

// Rows per pass of the prefill kernels (4 MFMA N-tiles of 16 columns).
constexpr int kPreTpp = 64;
// Weight rows per item of the paired (M = 2: 8 waves x 32) and single
// (M = 1: 8 waves x 64) product: the single product, with half the
// accumulators, gives each wave more rows, so that each staged activation
// unit meets as many weight rows.
// Grouped-scale int4 (gs > 0) keeps a running total per output beside the
// group's sums, so a wave takes half the rows: 128 and 256.
constexpr int pre_rows_per_item(int M, bool gs = false) { return (M == 2 ? 256 : 512) >> (gs ? 1 : 0); }

// bf16 row tables: one row per activation row, kpad elements rounded once to
// bf16 in fragment order (16-byte units of 8 elements), 2 * kpad bytes a row.
//
// Groups, passes and work list as for the decode kernels (coli_dec.h), with
// passes of kPreTpp rows.
struct PreArgs {
    const uint8_t *w[2];
    const float *s[2];
    int64_t w_gstride, s_gstride;
    int ngroups, O;
    const uint8_t *xw[2];   // the extra (shared) group's matrices
    const float *xs[2];
    int has_extra, xO, x_rows, x_row0;
    int kpad;
    int64_t rb;
    const int *offsets;
    const int *work;
    const int *n_work;
    const int *act_row;     // row-table row of grouped row r (NULL: r itself)
    const float *row_sum;   // [grouped row] sum of that row's stored activations
    const uint16_t *act;    // bf16 row table of the activations
    float *out;             // result rows (grouped row r at out + r * ldo elements); gate/up:
                            // NULL for none (the down product reads the row table hf)
    int64_t ldo;
    int out_vec4;           // 16-byte aligned rows (fp32) / 8-byte aligned rows (bf16)
    int out_bf16;           // down: the result rows rounded to bf16 (uint16_t elements)
    // M == 2 only: the result as the next product's bf16 row table (rows =
    // grouped rows, hf_kpad elements) and its partial sums per row:
    // hpart[r * nparts + p], p = tile * 8 + wave
    uint16_t *hf;
    int hf_kpad;
    float *hpart;
    int nparts;
    int tiled;               // weights in the tiled layout (coli_pack_tiled); w_gstride
                             // is then the tiled bytes of one matrix
    // grouped-scale int4 (0: one scale per row): 32-element MFMA steps per
    // group (gs / 32) and groups per row (kpad / gs); weights in the grouped
    // tiled layout, scales [row tile][group][16 rows] (coli_pack_scales_grouped,
    // s_gstride floats per matrix)
    int gs_spg, gs_ngp;
    int tiles;               // set by pre_launch
};

// x [rows, ldx] -> bf16 row table (rows x 2 kpad bytes) and per-row sums of
// the stored values (fixed order).
hipError_t xrows_bf16_launch(int fmt, const float *x, int64_t ldx, int rows, int I, int kpad,
                             uint16_t *table, float *sums, hipStream_t st);
// act_row / row_sum of the gate/up product: grouped row r < P is slot
// row_pair[r] (token row_pair[r] / K), rows P..P+extra-1 are the shared
// expert's tokens 0..extra-1 (extra: S with a shared expert, else 0).
hipError_t pre_rows_launch(const int32_t *row_pair, int P, int K, int S, int extra, const float *token_sum,
                           int32_t *act_row, float *row_sum, hipStream_t st);
// row_sum[r] = sum_p hpart[r * nparts + p] in p order.
hipError_t pre_sum_launch(const float *hpart, int nparts, int rows, float *row_sum, hipStream_t st);
hipError_t pre_launch(PreArgs a, int fmt, int M, int64_t max_group_passes, hipStream_t st);
int pre_parts(int hf_kpad, bool gs = false);

}  // namespace coli

#endif
