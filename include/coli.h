/*
 * coli.h -- C ABI of libcoli: dequant-on-use quantized GEMV and the batched
 * MoE block (router, expert-grouped SwiGLU experts, shared expert) on AMD
 * MI355X (gfx950).
 *
 * Conventions shared by every entry point
 *   - Every array argument is a DEVICE pointer (memory the caller allocated
 *     on the current HIP device, e.g. a torch tensor's data_ptr()), unless the
 *     argument says "host".  The library never allocates, frees or keeps any
 *     caller memory and holds no state between calls, apart from the
 *     optional stage timer (coli_stage_timing).
 *   - Arrays are dense, row-major (C-contiguous).  A packed weight matrix
 *     [O, I] is stored as O rows of coli_row_bytes(fmt, I) bytes each.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Calls only enqueue work on it and return; nothing synchronises except
 *     coli_check_device_flags().
 *   - Outputs are overwritten, never accumulated into.
 *   - Return value: COLI_OK (0) or a negative coli_status.  All argument
 *     checks run on the host before anything is enqueued; on an error nothing
 *     is launched and no output is touched.  The library never aborts or exits.
 *   - Sizes of 0 are allowed where stated (an empty batch enqueues nothing).
 *
 * Typical use (one MoE layer per call, decode or prefill):
 *   size_t nb = coli_moe_workspace_bytes(S, K, E, D, F, F_shared, prec);
 *   (allocate nb device bytes, 256-byte aligned, once per shape)
 *   coli_moe_layer(&router, &experts, &shared, x, S, NULL, NULL, out,
 *                  idx_out, w_out, prec, ws, nb, stream);
 *   coli_check_device_flags(ws, stream, NULL);   (optional: bad routing ids)
 * and for a single quantized matrix: coli_qgemv(fmt, W, scale, x, y, S, I, O,
 * stream), which needs no workspace.
 *
 * Sources (page title -- section):
 *   glm.c@98759bf  colibri-strix c/glm.c, commit 98759bf
 *   glm.c@97c756a  colibri-strix c/glm.c, commit 97c756a
 *   metal@93cde63  colibri c/backend_metal.mm, commit 93cde63
 *   docs-quickstart  colibri compare main...docs-quickstart (qt_resolve_fmt)
 */
#ifndef COLI_H
#define COLI_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Weight row formats: the QT tensor's fmt codes [glm.c@98759bf -- typedef QT].
 *   COLI_F32 : fp32 values, 4*I bytes per row.
 *   COLI_I8  : signed int8 values, I bytes per row   [glm.c@98759bf -- matmul_q]
 *   COLI_I4  : two values per byte, (I+1)/2 bytes per row; element 2k is the
 *              low nibble of byte k, 2k+1 the high nibble; value = nibble - 8
 *              [glm.c@98759bf -- matmul_i4, pack_int4]
 *   COLI_I2  : four values per byte, (I+3)/4 bytes per row; element i is bits
 *              2*(i%4)..2*(i%4)+1 of byte i/4; value = crumb - 2
 *              [glm.c@98759bf -- matmul_i2, pack_int2]
 * Padding nibbles / crumbs past I in a row's last byte are never read. */
enum coli_fmt { COLI_F32 = 0, COLI_I8 = 1, COLI_I4 = 2, COLI_I2 = 3 };

enum coli_status {
    COLI_OK = 0,
    COLI_EINVAL = -1,     /* a required pointer is NULL, or a flag is out of its range */
    COLI_ESHAPE = -2,     /* a size is negative, or a byte count overflows int64 */
    COLI_EFMT = -3,       /* unknown weight format, or one this call does not take */
    COLI_EALIGN = -4,     /* a pointer is not aligned as the call requires */
    COLI_ERANGE = -5,     /* K, E or another count outside its supported range */
    COLI_EWORKSPACE = -6, /* workspace NULL or smaller than the size query says */
    COLI_EDEVICE = -7,    /* the HIP runtime reported an error */
    COLI_EIDX = -8        /* coli_check_device_flags: bad routing ids were seen */
};

/* Precision of the MoE expert products.
 *   COLI_PREC_FP32: fp32 activations, fp32 accumulation; every float output
 *     meets |y - y_ref| <= 1e-4 * (scale * sum |v * x|) + 1e-6.
 *     (The matrix cores take x as bf16 hi + lo, 16 rows per pass.)
 *   COLI_PREC_BF16: activations -- x, and h for the down product -- rounded
 *     once to bf16, int weights converted exactly to bf16 for the matrix
 *     cores, fp32 accumulation, scale applied in fp32 after the sum, 64 rows
 *     per pass; bound 2e-2 of the same magnitude.  Meant for prefill-sized
 *     batches.  Shapes that take the vector-ALU kernels (rows that are not
 *     whole 16-byte segments) compute in fp32 under either value.
 *   COLI_PREC_IDOT: the pages' integer-dot path [glm.c@98759bf -- qrow_i8,
 *     dot_i4i8, dot_i8i8, matmul_q_idot; the moe block's expert matmuls]:
 *     x per token, and h per grouped row, quantised to int8 by its absolute
 *     maximum (s = max|v| / 127, at least 1e-12, q = round-half-even(v / s)
 *     with 1/s in fp32), the dot with the int weight values exact in int32
 *     (v_mfma_i32_16x16x64_i8), then ((float)dot * scale[o]) * s, rounded
 *     in fp32 in that order; gate/up give h = silu(g) * u in fp32.  Lossy
 *     by design (int8 activations, about 0.3% RMS per product on the
 *     pages' measurements): every integer dot and its epilogue equal the
 *     definition's bit for bit.  int8 or int4 experts in the tiled layout
 *     only (and a shared expert of the same format, F and layout), D and F
 *     at most 16384; else COLI_EFMT / COLI_EINVAL / COLI_ERANGE.  64 rows
 *     per pass, as COLI_PREC_BF16. */
enum coli_prec { COLI_PREC_FP32 = 0, COLI_PREC_BF16 = 1, COLI_PREC_IDOT = 2 };

/* Bytes in one packed row of I elements, or -1 for an unknown fmt / I < 0
 * [glm.c@98759bf -- qt_bytes].  Host only; no device work. */
int64_t coli_row_bytes(int fmt, int64_t I);

/* Quantized matrix-vector product, dequantised on use
 *     y[s, o] = scale[o] * sum_{i<I} v(o, i) * x[s, i]
 * [glm.c@98759bf -- matmul_q, matmul_i4, matmul_i2, matmul_qt;
 *  metal@93cde63 -- mm_gemv].  The per-row scale multiplies the finished sum.
 *   fmt    COLI_F32 / I8 / I4 / I2.
 *   W      [O, coli_row_bytes(fmt, I)] bytes, 4-byte aligned.
 *   scale  [O] fp32.  May be NULL only for COLI_F32 (then 1), since glm.c's
 *          f32 rows carry no scale while the Metal kernel applies one.
 *   x      [S, I] fp32, 4-byte aligned.
 *   y      [S, O] fp32, overwritten.
 *   S, I, O >= 0.  S == 0 or O == 0 enqueues nothing; I == 0 writes zeros.
 * Errors: COLI_EFMT, COLI_EINVAL (NULL array), COLI_ESHAPE, COLI_EALIGN,
 * COLI_EDEVICE. */
int coli_qgemv(int fmt, const void *W, const float *scale, const float *x,
               float *y, int S, int I, int O, void *stream);

/* Integer-dot quantized matrix-vector product (IDOT), a lossy variant of
 * coli_qgemv [glm.c@98759bf -- qrow_i8, dot_i8i8, dot_i4i8, matmul_q_idot,
 * matmul_i4_idot]: each row of x is quantised to int8 by its absolute
 * maximum,
 *     s_s = max(max_i |x[s,i]| / 127, 1e-12),  q[s,i] = rint(x[s,i] * (1/s_s)),
 * (fp32, round half to even), the dot product with the weight values is
 * exact integer arithmetic, and
 *     y[s, o] = ((float)dot(v(o, .), q[s, .]) * scale[o]) * s_s
 * with each operation rounded in fp32 in that order.  The result is the
 * definition's bit for bit; against coli_qgemv it differs by the int8
 * rounding of x (about 0.3% RMS on the pages' measurements).
 *   fmt    COLI_I8 or COLI_I4 (the pages' integer-dot formats).
 *   W      [O, coli_row_bytes(fmt, I)] bytes, 16-byte aligned, the row a
 *          whole number of 16-byte segments (I a multiple of 16 for int8,
 *          of 32 for int4), I <= 8192 (int8) / 16384 (int4).
 *   scale  [O] fp32 (required).   x [S, I] fp32.   y [S, O] fp32, overwritten.
 *   ws     device workspace of ws_bytes >= coli_qgemv_idot_workspace_bytes(S, I)
 *          bytes, 256-byte aligned: the quantised rows.
 * Errors: COLI_EFMT, COLI_EINVAL, COLI_ESHAPE, COLI_EALIGN, COLI_ERANGE,
 * COLI_EWORKSPACE, COLI_EDEVICE. */
size_t coli_qgemv_idot_workspace_bytes(int S, int I);
int coli_qgemv_idot(int fmt, const void *W, const float *scale, const float *x, float *y,
                    int S, int I, int O, void *ws, size_t ws_bytes, void *stream);

/* Grouped-scale int4 matrix-vector product (the pages' fmt 4,
 * "int4-grouped": int4 rows with one fp32 scale per group of gs consecutive
 * elements along I instead of one per row) [docs-quickstart --
 * qt_resolve_fmt; glm.c@98759bf -- qt_from_disk]:
 *     y[s, o] = sum_g scale[o, g] * sum_{i in group g} v(o, i) * x[s, i],
 * group g = elements g*gs .. min((g+1)*gs, I) - 1, v = nibble - 8.  Bound as
 * coli_qgemv: |y - y_ref| <= 1e-4 * sum_g |scale[o,g]| sum |v x| + 1e-6.
 *   W      [O, coli_row_bytes(COLI_I4, I)] bytes, 16-byte aligned, rows a
 *          whole number of 16-byte segments (I a multiple of 32), I <= 12288.
 *   scale  [O, ceil(I / gs)] fp32, 16-byte aligned.   gs: 32, 64 or a multiple
 *          of 128.
 *   x      [S, I] fp32, 16-byte aligned.   y [S, O] fp32, overwritten.
 * Errors: COLI_EINVAL, COLI_ESHAPE, COLI_EALIGN, COLI_ERANGE (gs or I out of
 * range), COLI_EDEVICE. */
int coli_qgemv_grouped(const void *W, const float *scale, int gs, const float *x, float *y,
                       int S, int I, int O, void *stream);

/* Router: sigmoid scores and noaux_tc top-K with one group
 * [glm.c@98759bf -- moe, phase A; metal@93cde63 -- r_router, r_top8,
 *  r_top8_par].  For each token s:
 *     logit[e] = sum_d Wr[e, d] * x[s, d]      (accumulated in fp64)
 *     sig[s,e] = fp32(1 / (1 + exp(-logit[e])))  (fp64, rounded once)
 *     choice[e] = sig[s,e] + bias[e]           (fp32 add)
 *     K picks: the largest choice among experts not yet taken; equal
 *              choices go to the lower expert index.
 *     w[kk] = sig[s, idx[kk]]  (the score, not the choice)
 *     topp in (0,1): reorder the picks by descending weight (stable) and keep
 *              the shortest prefix whose running fp32 sum reaches
 *              topp * (1e-20 + total); keff[s] = its length; else keff[s] = K.
 *     norm_topk != 0: w[kk] /= (sum_{kk<keff} w + 1e-20), in fp32.
 *     w[kk] *= routed_scale.
 *   Wr    [E, D] fp32.   bias [E] fp32.   x [S, D] fp32.
 *   idx   [S, K] int32 out; slots kk >= keff[s] hold -1.
 *   w     [S, K] fp32 out; slots kk >= keff[s] hold 0.
 *   keff  [S] int32 out, or NULL.
 *   sig   [S, E] fp32 out (the sigmoid scores); required.
 *   ws    device scratch of ws_bytes >= coli_router_workspace_bytes(S, E, D)
 *         bytes, 8-byte aligned (partial fp64 logits).
 *   1 <= K <= min(E, 64), 1 <= E <= 1024, D >= 1, S >= 0.
 * Errors: COLI_EINVAL, COLI_ESHAPE, COLI_ERANGE, COLI_EALIGN, COLI_EWORKSPACE,
 * COLI_EDEVICE. */
int coli_router(const float *Wr, const float *bias, const float *x, int S,
                int E, int D, int K, int norm_topk, float routed_scale,
                float topp, int32_t *idx, float *w, int32_t *keff, float *sig,
                void *ws, size_t ws_bytes, void *stream);

/* Scratch bytes coli_router needs for S tokens, E experts, width D (0 for
 * invalid arguments).  Host only. */
size_t coli_router_workspace_bytes(int S, int E, int D);

/* Weight layouts of the MoE tensors.
 *   COLI_LAYOUT_ROWS  : the pages' row-major packed rows, [O, coli_row_bytes]
 *                       per matrix.
 *   COLI_LAYOUT_TILED : the same bytes regrouped by coli_pack_tiled() so that
 *                       the matrix cores read each weight chunk with one
 *                       contiguous 1 KB load per wave (see there).
 *   COLI_LAYOUT_TILED_GROUPED : grouped-scale int4 (gs > 0) only: the tiled
 *                       layout with each segment's 16 words transposed
 *                       (coli_pack_tiled_grouped), and the scales packed by
 *                       coli_pack_scales_grouped. */
enum coli_layout { COLI_LAYOUT_ROWS = 0, COLI_LAYOUT_TILED = 1, COLI_LAYOUT_TILED_GROUPED = 2 };

/* Bytes of the tiled copy of `count` stacked [O, I] matrices of format fmt
 * (COLI_I8 / I4 / I2), or -1 for invalid arguments.  It is count * ceil(O /
 * 16) * ceil(coli_row_bytes(fmt, I) / 64) * 1024, equal to the row-major size
 * when O is a multiple of 16 and a row a multiple of 64 bytes.  Host only. */
int64_t coli_tiled_bytes(int fmt, int64_t count, int O, int I);

/* Writes the tiled layout of `count` stacked row-major matrices W [count, O,
 * coli_row_bytes(fmt, I)] into dst [coli_tiled_bytes(fmt, count, O, I)] --
 * caller memory, 16-byte aligned, not overlapping W; nothing is allocated.
 * The values are the pages' row formats unchanged [glm.c@98759bf -- typedef
 * QT, pack_int4, pack_int2]; only their order in memory changes.  A matrix is
 * cut into units of 16 rows x 64 bytes (1 KB): unit (m, g) holds rows 16m ..
 * 16m+15, bytes 64g .. 64g+63 of each, and inside it bytes 16L .. 16L+15,
 * L = 16q + c (q < 4, c < 16), are row 16m+c's bytes 64g+16q .. +15 -- the
 * order in which a 64-lane wave feeds 16 rows to the bf16 matrix-core
 * operand.  Units are ordered by groups of 8 row tiles (128 rows; the last
 * group may hold fewer), inside a group by segment g, then by row tile:
 * offset (1024 *) (8 T NS + g n_T + m mod 8), T = m / 8, NS = ceil(rb / 64),
 * n_T = min(8, ceil(O/16) - 8 T).  Bytes past a row's end and rows past O
 * are zero.  Each matrix's tiled bytes follow the previous one's.
 * W needs whole 16-byte row segments (coli_row_bytes(fmt, I) % 16 == 0) and
 * 16-byte alignment.  Asynchronous on `stream`.
 * Errors: COLI_EFMT, COLI_EINVAL (NULL), COLI_ESHAPE, COLI_EALIGN,
 * COLI_EDEVICE. */
int coli_pack_tiled(int fmt, const void *W, int64_t count, int O, int I, void *dst, void *stream);

/* The grouped tiled layout of int4 matrices with one scale per gs elements
 * (the pages' int4-grouped format [docs-quickstart -- qt_resolve_fmt]): the
 * coli_pack_tiled layout of COLI_I4 rows (same size, coli_tiled_bytes) with
 * the 16 four-byte words of each row's 64-byte segment transposed -- word 4q
 * + s of the unit row comes from word 4s + q of the segment -- so that the
 * matrix cores' step s (the s-th word of every lane chunk) covers 32
 * consecutive elements 32 s .. 32 s + 31, one group of 32 or a part of a
 * larger group.  Arguments and errors as coli_pack_tiled (fmt COLI_I4). */
int coli_pack_tiled_grouped(const void *W, int64_t count, int O, int I, void *dst, void *stream);

/* Bytes of the packed group scales of `count` stacked [O, I] matrices with
 * one scale per gs elements: count * ceil(O / 16) * (kpad / gs) * 64, kpad =
 * I rounded up to 1024; -1 for invalid arguments (gs not one of 32, 64, 128,
 * 256, 512, 1024).  Host only. */
int64_t coli_grouped_scale_bytes(int64_t count, int O, int I, int gs);

/* Packs scales S [count, O, ceil(I / gs)] fp32 (row o's groups consecutive)
 * into dst [coli_grouped_scale_bytes(count, O, I, gs) bytes]: per matrix,
 * per 16-row tile t and group g, the 16 rows' scales of g (64 bytes) at
 * float offset (t * (kpad / gs) + g) * 16 -- zero for rows past O and groups
 * past ceil(I / gs).  Caller memory, 16-byte aligned; nothing is allocated.
 * Asynchronous on `stream`.  Errors: COLI_EINVAL (NULL), COLI_ESHAPE,
 * COLI_ERANGE (gs), COLI_EALIGN, COLI_EDEVICE. */
int coli_pack_scales_grouped(const float *S, int64_t count, int O, int I, int gs, float *dst, void *stream);

/* Routed experts stacked in one allocation per tensor
 * [glm.c@98759bf -- typedef ESlot; metal@93cde63 -- moe_submit]:
 *   w_gate, w_up  [E, F, coli_row_bytes(fmt, D)] bytes,
 *   w_down        [E, D, coli_row_bytes(fmt, F)] bytes,
 *   s_gate, s_up  [E, F] fp32,   s_down [E, D] fp32.
 * fmt is one of COLI_I8 / I4 / I2 (all three tensors share it).
 * layout COLI_LAYOUT_ROWS (0), or COLI_LAYOUT_TILED: then each weight tensor
 * is the coli_pack_tiled() copy of the stack above (w_gate of E matrices
 * [F, D], w_down of E matrices [D, F]), 16-byte aligned, with whole 16-byte
 * row segments (rows of D and of F).
 * gs: 0 (one scale per row), or grouped-scale int4 [docs-quickstart --
 * qt_resolve_fmt]: fmt COLI_I4, one scale per gs (32, 64, .., 1024)
 * consecutive elements along the row, layout COLI_LAYOUT_TILED_GROUPED --
 * the weights packed by coli_pack_tiled_grouped, s_gate / s_up the
 * coli_pack_scales_grouped copies of [E, F, ceil(D/gs)] and s_down of
 * [E, D, ceil(F/gs)] (16-byte aligned):
 *     y[o] = sum_g s[o, g] * sum_{i in group g} v(o, i) x_i.
 * Grouped experts run at COLI_PREC_FP32 or COLI_PREC_BF16 (COLI_PREC_IDOT:
 * COLI_EFMT). */
typedef struct {
    int fmt;
    int E, D, F;
    const void *w_gate, *w_up, *w_down;
    const float *s_gate, *s_up, *s_down;
    int layout;
    int gs;
} coli_experts;

/* One SwiGLU MLP applied with weight 1 to every token: the shared expert
 * [glm.c@98759bf -- moe, phase E; dense_mlp]:  down(silu(gate x) * up x).
 *   w_gate, w_up [F, coli_row_bytes(fmt, D)], w_down [D, coli_row_bytes(fmt, F)],
 *   s_gate, s_up [F], s_down [D].  D is the experts' D.
 *   layout and gs as coli_experts (one matrix each); a tiled shared expert
 *   needs tiled routed experts of the same fmt, F, layout and gs. */
typedef struct {
    int fmt;
    int F;
    const void *w_gate, *w_up, *w_down;
    const float *s_gate, *s_up, *s_down;
    int layout;
    int gs;
} coli_mlp;

/* Router parameters for coli_moe_layer (see coli_router).  E and D are the
 * experts'. */
typedef struct {
    const float *w;     /* [E, D] fp32 */
    const float *bias;  /* [E] fp32 (e_score_correction_bias) */
    int K;
    int norm_topk;
    float routed_scale;
    float topp;         /* <= 0 or >= 1: off */
} coli_router_params;

/* Device workspace size (bytes) needed by coli_moe_gemv / coli_moe_layer for
 * S tokens, K slots per token, E experts of width D x F, a shared expert of
 * width F_shared (0 = none), at precision prec.  Returns 0 for invalid
 * arguments.  Host only.  The workspace needs 256-byte alignment. */
size_t coli_moe_workspace_bytes(int S, int K, int E, int D, int F,
                                int F_shared, int prec);

/* Byte offsets of the documented regions inside the workspace, for callers
 * that want the intermediates (all relative to the workspace base; a region
 * absent for the given arguments has offset -1):
 *   flags      uint32: bit 0 = an expert id outside [-1, E) was skipped,
 *                      bit 1 = a token listed one expert twice.
 *   sig        [S, E] fp32 router scores (coli_moe_layer running the router).
 *   idx, w     [S, K] routing used (copy of the inputs or the router's).
 *   offsets    [E + 1] int32: rows of expert e are offsets[e]..offsets[e+1]-1
 *              in the grouped order.
 *   row_pair   [S*K] int32: grouped row r holds pair p = s*K + kk.
 *   pair_row   [S*K] int32: inverse map (-1 for a skipped slot).
 *   counts     [E] int32: rows per expert.
 *   h          [S*K + S, Fmax] fp32: SwiGLU output per grouped row; the
 *              shared expert's row for token s is S*K + s (COLI_PREC_BF16
 *              keeps the SwiGLU output only as the bf16 row table hf).
 *   y          [S*K + S, D] fp32: expert output per grouped row (same
 *              numbering), before the routing weight; COLI_PREC_BF16: rounded
 *              to bf16 (uint16 elements, row stride D), unless a shared
 *              expert of another format or width runs on the vector ALUs.
 *   router_part  fp64 partial router logits (scratch).
 *   xf, xsum, hf, hsum, work, n_work   matrix-core scratch and the
 *              device-built list of passes.  xf holds one row per token and
 *              hf one row per grouped row: the row's activations (x, resp.
 *              the SwiGLU output) in the kernels' fragment order,
 *              xf_stride / hf_stride bf16 per row -- COLI_PREC_FP32: bf16
 *              hi/lo pairs, xsum and hsum empty; COLI_PREC_BF16: bf16 values,
 *              xsum = [S] per-token sums of the stored x, then per grouped
 *              row its xf row (int32) and activation sum; hsum = per grouped
 *              row KpF/32 (grouped-scale experts: KpF/16) partial sums of the
 *              stored h (KpF = F rounded up to 1024), then their totals; COLI_PREC_IDOT: int8 values (KpD,
 *              resp. KpF, bytes a row), xsum = per token its scale and four
 *              partial sums of its int8 values, then per grouped row its xf
 *              row, scale and sum; hsum = per grouped row the scale and four
 *              partial sums of h's int8 row, then its scale and sum.
 *   xn         [S, D] fp32: the RMSNorm rows coli_moe_layer_tail feeds the
 *              block.
 *   gpart      grouping of more than 1024 slots (S K > 1024): per chunk of
 *              1024 slots E int32 counts, turned into the chunk's first
 *              position per expert, then one flags word per chunk. */
typedef struct {
    int64_t flags, sig, idx, w, offsets, counts, row_pair, pair_row, h, y, router_part;
    int64_t xf, xsum, hf, hsum, work, n_work;
    int64_t xn;                    /* coli_moe_layer_tail: [S, D] fp32 RMSNorm rows */
    int64_t gpart;                 /* grouping of more than 1024 slots: per 1024-slot
                                      chunk, E counts / first positions and a flags word */
    int64_t n_pass_max;            /* passes the scratch is sized for */
    int64_t xf_stride, hf_stride;  /* bf16 elements per row */
    int64_t h_ld;   /* row stride of h in floats (max of F and F_shared) */
    int64_t total;  /* == coli_moe_workspace_bytes(...) */
} coli_ws_layout;

int coli_moe_workspace_layout(int S, int K, int E, int D, int F, int F_shared,
                              int prec, coli_ws_layout *out /* host */);

/* Routed experts for S tokens with given routing (the batch-union MoE, phases
 * B and D) [glm.c@98759bf -- moe, phases B and D; metal@93cde63 -- moe_gemv,
 * moe_silu, moe_finish; glm.c@97c756a -- matmul_i4_pair, expert_gate_up]:
 *     out[s] = sum_{kk : idx[s,kk] >= 0} w[s,kk] * down_e(silu(gate_e x_s) * up_e x_s),
 *     e = idx[s,kk].
 * Slots are grouped by expert on the device (stable in s*K + kk order) so each
 * active expert's weights stream from memory once per call; gate and up are
 * computed in one pass over x and SwiGLU is applied before h is stored; the
 * weighted sum runs in slot order kk = 0..K-1, so results are deterministic.
 *   ex     routed experts (device pointers inside; the struct itself is host).
 *   x      [S, D] fp32.   idx [S, K] int32: an expert id, or -1 = empty slot.
 *   w      [S, K] fp32.   out [S, D] fp32, overwritten.
 *   prec   COLI_PREC_FP32, COLI_PREC_BF16 or COLI_PREC_IDOT.
 *   ws     device workspace of ws_bytes >= coli_moe_workspace_bytes(S,K,E,D,F,0,prec).
 * An id < -1 or >= E is skipped and a listed-twice expert is computed twice;
 * both set a flag that coli_check_device_flags() reports.
 * 1 <= K <= 64, 1 <= E <= 1024, S >= 0, D, F >= 1.
 * Size limit (COLI_ERANGE otherwise): every expert matrix (F * row_bytes(D)
 * and D * row_bytes(F), routed and shared) and every activation table --
 * S rows, and S*K (+ S with a shared expert) rows, of 4 (COLI_PREC_FP32),
 * 2 (COLI_PREC_BF16) or 1 (COLI_PREC_IDOT) bytes per element of D resp. max(F, F_shared) rounded
 * up to 1024 -- stays below 2^32 - 4096 bytes.  At D = 6144, F = 2048, K = 8
 * with a shared expert that is S <= 58254 tokens per call (fp32 precision).
 * Errors: COLI_EINVAL, COLI_EFMT, COLI_ESHAPE, COLI_ERANGE, COLI_EALIGN,
 * COLI_EWORKSPACE, COLI_EDEVICE. */
int coli_moe_gemv(const coli_experts *ex, const float *x, int S, int K,
                  const int32_t *idx, const float *w, float *out, int prec,
                  void *ws, size_t ws_bytes, void *stream);

/* Full MoE block for S tokens (ragged decode rows or a prefill batch):
 * router (unless routing is given), routed experts, shared expert, combine
 * [glm.c@98759bf -- moe, phases A, B, D, E; metal@93cde63 --
 *  coli_metal_layer_decode, coli_metal_moe_block]:
 *     out[s] = sum_kk w[s,kk] * expert_{idx[s,kk]}(x_s)  +  shared(x_s).
 *   r          router parameters; used when pre_idx == NULL.
 *   ex         routed experts.   shared: the shared expert, or NULL.
 *   x          [S, D] fp32.
 *   pre_idx, pre_w  [S, K] given routing (both or neither), the analogue of
 *              routing computed elsewhere and handed to moe(); when given the
 *              router does not run.
 *   out        [S, D] fp32, overwritten.
 *   idx_out, w_out  [S, K] routing actually used, or NULL.
 *   ws, ws_bytes    as coli_moe_gemv, sized with F_shared = shared ? shared->F : 0.
 * Errors: as coli_moe_gemv. */
int coli_moe_layer(const coli_router_params *r, const coli_experts *ex,
                   const coli_mlp *shared, const float *x, int S,
                   const int32_t *pre_idx, const float *pre_w, float *out,
                   int32_t *idx_out, float *w_out, int prec, void *ws,
                   size_t ws_bytes, void *stream);

/* The layer tail around the MoE block: the post-attention RMSNorm of the
 * residual stream, the block on the normalised rows, and the residual add
 * [glm.c@98759bf -- rmsnorm; the layer forward's post-attention half]:
 *     n_s   = rmsnorm(x_s) = (x_s * r_s) * norm_w,
 *     r_s   = 1 / sqrtf((float)(sum_i x_si^2 / D) + eps)   (sum in fp64),
 *     out_s = x_s + moe_layer(n_s)                          (fp32 add).
 *   norm_w     [D] fp32 RMSNorm weight.   eps: >= 0 (the pages' default 1e-5).
 *   x, out     [S, D] fp32; out may be x itself (in place).
 *   other arguments as coli_moe_layer; the routing written to idx_out /
 *   w_out is the one taken on the normalised rows, and the workspace region
 *   xn receives them.
 * Errors: as coli_moe_layer, and COLI_EINVAL for a NULL norm_w or a negative
 * or NaN eps, COLI_EALIGN for a norm_w not 4-byte aligned. */
int coli_moe_layer_tail(const coli_router_params *r, const coli_experts *ex,
                        const coli_mlp *shared, const float *x, const float *norm_w,
                        float eps, int S, const int32_t *pre_idx, const float *pre_w,
                        float *out, int32_t *idx_out, float *w_out, int prec, void *ws,
                        size_t ws_bytes, void *stream);

/* coli_moe_layer for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same computation and arguments without ws / ws_bytes.  The scratch is
 * a static device array of COLI_NOALLOC_SCRATCH_BYTES (64 MiB) that each GPU
 * the library runs on holds until the process ends; the call allocates
 * nothing (no hipMalloc / hipFree, no allocating library routine).  Sizes
 * whose coli_moe_workspace_bytes() exceeds it are refused with COLI_ERANGE
 * before any device work (128 decode tokens of 256 experts of 6144 x 2048,
 * K = 8, with a shared expert, need 55 MiB at COLI_PREC_FP32).  All calls on
 * one GPU share that GPU's array, which keeps the last call's contents; every
 * region a call reads is written earlier in the same call, so nothing needs
 * clearing between calls.  Calls that overlap on one GPU -- on different
 * streams, or from host threads without ordering -- race and give wrong
 * results: the caller orders them (one stream, or events).  Bad routing ids
 * are skipped as in coli_moe_layer, but their flags are not reported (no
 * workspace to pass to coli_check_device_flags).
 * Errors: as coli_moe_layer, COLI_ERANGE for a too-large size. */
#define COLI_NOALLOC_SCRATCH_BYTES (64u << 20)
int coli_moe_layer_noalloc(const coli_router_params *r, const coli_experts *ex,
                           const coli_mlp *shared, const float *x, int S,
                           const int32_t *pre_idx, const float *pre_w, float *out,
                           int32_t *idx_out, float *w_out, int prec, void *stream);

/* Waits for `stream`, then reads the workspace flags the last MoE call on it
 * left.  *flags_out (host, may be NULL) receives the raw bits.  Returns
 * COLI_OK when none is set, COLI_EIDX when a routing id was skipped or
 * duplicated, COLI_EDEVICE on a runtime error. */
int coli_check_device_flags(const void *ws, void *stream, uint32_t *flags_out);

/* Stage timing, for benchmarks and profiling.  Off by default; while on,
 * every call records a hipEvent pair on its stream around each stage it runs
 * (the only state the library keeps between calls).  coli_stage_times waits
 * for the recorded events and writes, per stage, the total milliseconds and
 * the number of timed launches since the last reset (host arrays of
 * COLI_NSTAGES entries; either may be NULL).  Stages: 0 router, 1 grouping,
 * 2 gate/up + SwiGLU, 3 down, 4 combine, 5 qgemv, 6 matrix-core preparation
 * (activation fragments and per-row sums ahead of gate/up, where the grouping
 * launch does not already write them: fp32 precision up to 1024 slots, the
 * grouping stage covers them), 7 RMSNorm of the layer tail.  The pages time the same
 * phases of their MoE block [metal@93cde63 -- moe_finish timers;
 * glm.c@98759bf -- profile counters]. */
#define COLI_NSTAGES 8
int coli_stage_timing(int enable);
int coli_stage_times(double *ms, int64_t *calls, int reset);
const char *coli_stage_name(int stage);

/* Static text for a status code. */
const char *coli_strerror(int status);

/* Library version: major * 10000 + minor * 100 + patch. */
int coli_version(void);

#ifdef __cplusplus
}
#endif

#endif /* COLI_H */
