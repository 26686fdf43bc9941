/*
 * coli_validate.c -- host-side argument checks, size queries and workspace
 * layout of libcoli.  Plain C, no HIP: it is linked into libcoli.so and also
 * built alone so the checks can be exercised on a machine without a GPU.
 *
 * The refusal of mismatched sizes follows the pages' hardening of weight
 * format resolution: a byte count that fits no known layout is an error,
 * never a guess [docs-quickstart -- qt_resolve_fmt].
 */
#include <stdint.h>
#include <stddef.h>

#include "coli.h"
#include "coli_internal.h"

#define ALIGN_WS 256

int64_t coli_row_bytes(int fmt, int64_t I)
{
    if (I < 0) return -1;
    switch (fmt) {
    case COLI_F32: return I > INT64_MAX / 4 ? -1 : 4 * I;
    case COLI_I8:  return I;
    case COLI_I4:  return (I + 1) / 2;
    case COLI_I2:  return (I + 3) / 4;
    default:       return -1;
    }
}

const char *coli_strerror(int status)
{
    switch (status) {
    case COLI_OK:         return "ok";
    case COLI_EINVAL:     return "invalid argument (NULL pointer or flag out of range)";
    case COLI_ESHAPE:     return "invalid size (negative, or byte count overflow)";
    case COLI_EFMT:       return "unsupported weight format";
    case COLI_EALIGN:     return "misaligned pointer";
    case COLI_ERANGE:     return "count out of supported range (K, E)";
    case COLI_EWORKSPACE: return "workspace missing or too small";
    case COLI_EDEVICE:    return "HIP runtime error";
    case COLI_EIDX:       return "routing ids out of range or duplicated (device flag)";
    default:              return "unknown status";
    }
}

int coli_version(void) { return 1 * 10000 + 0 * 100 + 0; }

/* a*b with overflow check into *out; returns 0 on overflow */
static int mul_ok(int64_t a, int64_t b, int64_t *out)
{
    if (a < 0 || b < 0) return 0;
    if (a != 0 && b > INT64_MAX / a) return 0;
    *out = a * b;
    return 1;
}

static int aligned(const void *p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

int coli__check_qgemv(int fmt, const void *W, const float *scale,
                      const float *x, const float *y, int S, int I, int O)
{
    if (fmt < COLI_F32 || fmt > COLI_I2) return COLI_EFMT;
    if (S < 0 || I < 0 || O < 0) return COLI_ESHAPE;
    int64_t rb = coli_row_bytes(fmt, I), t;
    if (rb < 0 || !mul_ok(rb, O, &t) || !mul_ok((int64_t)S, I, &t) ||
        !mul_ok((int64_t)S, O, &t) || !mul_ok(t, 4, &t))
        return COLI_ESHAPE;
    if (S == 0 || O == 0) return COLI_OK;
    if (!y) return COLI_EINVAL;
    if (I > 0 && (!W || !x)) return COLI_EINVAL;
    if (!scale && fmt != COLI_F32) return COLI_EINVAL;
    if ((W && !aligned(W, 4)) || (x && !aligned(x, 4)) || !aligned(y, 4) ||
        (scale && !aligned(scale, 4)))
        return COLI_EALIGN;
    return COLI_OK;
}

int coli__check_router(const float *Wr, const float *bias, const float *x,
                       int S, int E, int D, int K, int norm_topk,
                       const int32_t *idx, const float *w, const float *sig,
                       const void *ws, size_t ws_bytes)
{
    if (S < 0 || E < 0 || D < 0 || K < 0) return COLI_ESHAPE;
    if (E < 1 || E > COLI_MAX_E || K < 1 || K > COLI_MAX_K || K > E) return COLI_ERANGE;
    if (D < 1) return COLI_ESHAPE;
    if (norm_topk != 0 && norm_topk != 1) return COLI_EINVAL;
    int64_t t;
    if (!mul_ok((int64_t)S, D, &t) || !mul_ok((int64_t)E, D, &t) ||
        !mul_ok((int64_t)S, E, &t) || !mul_ok(t, 8, &t))
        return COLI_ESHAPE;
    if (S == 0) return COLI_OK;
    if (!Wr || !bias || !x || !idx || !w || !sig) return COLI_EINVAL;
    if (!aligned(Wr, 4) || !aligned(bias, 4) || !aligned(x, 4) || !aligned(idx, 4) ||
        !aligned(w, 4) || !aligned(sig, 4))
        return COLI_EALIGN;
    if (!ws || ws_bytes < (size_t)coli__router_partial_bytes(S, E, D)) return COLI_EWORKSPACE;
    if (!aligned(ws, 8)) return COLI_EALIGN;
    return COLI_OK;
}

static int64_t round_up(int64_t v, int64_t a) { return (v + a - 1) / a * a; }

int coli__router_token_tile(int S)
{
    return S >= 256 ? 64 : 16;   /* 64: each router row fragment feeds 4 token tiles */
}

int coli__router_splits(int S, int E, int D, int *slice)
{
    const int tt = coli__router_token_tile(S);
    int64_t tiles = (int64_t)((S + tt - 1) / tt) * ((E + 63) / 64);
    int64_t want = tiles > 0 ? (512 + tiles - 1) / tiles : 1;
    int64_t maxs = D / 64 > 0 ? D / 64 : 1;
    if (want > maxs) want = maxs;
    if (want < 1) want = 1;
    int64_t sl = round_up((D + want - 1) / want, 16);
    if (sl < 16) sl = 16;
    if (slice) *slice = (int)sl;
    return (int)((D + sl - 1) / sl);
}

int64_t coli__router_partial_bytes(int S, int E, int D)
{
    if (S <= 0 || E <= 0 || D <= 0) return 0;
    int splits = coli__router_splits(S, E, D, 0);
    return (int64_t)splits * S * E * 8;
}

size_t coli_router_workspace_bytes(int S, int E, int D)
{
    if (S < 0 || E < 1 || E > COLI_MAX_E || D < 1) return 0;
    int64_t b = coli__router_partial_bytes(S, E, D);
    return (size_t)(b > 0 ? b : 256);
}

/* Workspace layout: one 256-byte aligned region after the other. */
int coli_moe_workspace_layout(int S, int K, int E, int D, int F, int F_shared,
                              int prec, coli_ws_layout *out)
{
    if (!out) return COLI_EINVAL;
    if (S < 0 || K < 1 || E < 1 || D < 1 || F < 1 || F_shared < 0) return COLI_ESHAPE;
    if (prec != COLI_PREC_FP32 && prec != COLI_PREC_BF16 && prec != COLI_PREC_IDOT) return COLI_EINVAL;
    int64_t P, rows, Fmax = F > F_shared ? F : F_shared, t, off = 0;
    if (!mul_ok((int64_t)S, K, &P)) return COLI_ESHAPE;
    rows = P + (F_shared > 0 ? S : 0);
#define REGION(field, bytes)                                   \
    do {                                                       \
        int64_t b_ = (bytes);                                  \
        if (b_ < 0 || off > INT64_MAX - b_ - ALIGN_WS) return COLI_ESHAPE; \
        out->field = off;                                      \
        off = round_up(off + b_, ALIGN_WS);                    \
    } while (0)
    REGION(flags, 64);
    if (!mul_ok((int64_t)S, E, &t) || !mul_ok(t, 4, &t)) return COLI_ESHAPE;
    REGION(sig, t);
    REGION(idx, P * 4);
    REGION(w, P * 4);
    REGION(offsets, ((int64_t)E + 2) * 4);
    REGION(counts, ((int64_t)E + 2) * 4);
    REGION(row_pair, P * 4);
    REGION(pair_row, P * 4);
    if (!mul_ok(rows, Fmax, &t) || !mul_ok(t, 4, &t)) return COLI_ESHAPE;
    REGION(h, t);
    if (!mul_ok(rows, D, &t) || !mul_ok(t, 4, &t)) return COLI_ESHAPE;
    REGION(y, t);
    REGION(router_part, coli__router_partial_bytes(S, E, D));
    /* matrix-core path: the activations' row tables and sums (below), and
     * the work list of (group, pass) entries; a pass is COLI_MM_TPP_FP32
     * rows (fp32 precision) or COLI_MM_TPP_BF16 rows (bf16 precision). */
    const int bf16 = prec == COLI_PREC_BF16, idot = prec == COLI_PREC_IDOT;
    const int64_t tpp = bf16 || idot ? COLI_MM_TPP_BF16 : COLI_MM_TPP_FP32;
    int64_t ngp = (rows + tpp - 1) / tpp + (int64_t)E + 1;   /* passes */
    int64_t KpD = round_up(D, 1024), KpF = round_up(Fmax, 1024);
    if (idot) {
        /* integer dots: int8 row tables of x (per token) and of the SwiGLU
         * output (per grouped row), KpD / KpF bytes a row; xsum: per token
         * its scale and four partial sums, then per grouped row its table
         * row, scale and sum; hsum: per grouped row the scale and four
         * partial sums of h's row, then its scale and sum again */
        if (!mul_ok((int64_t)S, KpD, &t)) return COLI_ESHAPE;
        REGION(xf, t);
        REGION(xsum, ((int64_t)5 * S + 3 * rows) * 4);
        if (!mul_ok(rows, KpF, &t)) return COLI_ESHAPE;
        REGION(hf, t);
        REGION(hsum, rows * 7 * 4);
    } else if (bf16) {
        /* bf16 precision: bf16 row tables of x (per token) and of the SwiGLU
         * output (per grouped row); xsum: per-token sums of the stored x,
         * then per grouped row its table row (int32) and activation sum;
         * hsum: per grouped row KpF/16 partial sums of the stored h (KpF/32
         * with one scale per row, KpF/16 with grouped scales, whose items
         * have half the rows), then their totals */
        if (!mul_ok((int64_t)S, 2 * KpD, &t)) return COLI_ESHAPE;
        REGION(xf, t);
        REGION(xsum, ((int64_t)S + 2 * rows) * 4);
        if (!mul_ok(rows, 2 * KpF, &t)) return COLI_ESHAPE;
        REGION(hf, t);
        if (!mul_ok(rows, KpF / 16 + 1, &t) || !mul_ok(t, 4, &t)) return COLI_ESHAPE;
        REGION(hsum, t);
    } else {
        /* fp32 precision: one row table per token (x) and per grouped row
         * (the SwiGLU output), bf16 hi/lo pairs in fragment order */
        if (!mul_ok((int64_t)S, 4 * KpD, &t)) return COLI_ESHAPE;
        REGION(xf, t);
        REGION(xsum, 0);
        if (!mul_ok(rows, 4 * KpF, &t)) return COLI_ESHAPE;
        REGION(hf, t);
        REGION(hsum, 0);
    }
    REGION(work, (ngp + 1) * 4);
    REGION(n_work, 64);
    if (!mul_ok((int64_t)S, D, &t) || !mul_ok(t, 4, &t)) return COLI_ESHAPE;
    REGION(xn, t);
    /* chunked grouping: per chunk of COLI_GROUP_CHUNK slots, E counts (then
     * the chunk's first position per expert) and a flags word */
    {
        const int64_t C = (P + COLI_GROUP_CHUNK - 1) / COLI_GROUP_CHUNK;
        if (!mul_ok(C, (int64_t)E + 1, &t) || !mul_ok(t, 4, &t)) return COLI_ESHAPE;
        REGION(gpart, t);
    }
#undef REGION
    out->n_pass_max = ngp;
    out->xf_stride = idot ? KpD / 2 : bf16 ? KpD : 2 * KpD;
    out->hf_stride = idot ? KpF / 2 : bf16 ? KpF : 2 * KpF;
    out->h_ld = Fmax;
    out->total = off;
    return COLI_OK;
}

size_t coli_moe_workspace_bytes(int S, int K, int E, int D, int F, int F_shared, int prec)
{
    coli_ws_layout L;
    if (coli_moe_workspace_layout(S, K, E, D, F, F_shared, prec, &L) != COLI_OK) return 0;
    return (size_t)L.total;
}

int64_t coli_tiled_bytes(int fmt, int64_t count, int O, int I)
{
    if (fmt != COLI_I8 && fmt != COLI_I4 && fmt != COLI_I2) return -1;
    if (count < 0 || O < 0 || I < 0) return -1;
    const int64_t rb = coli_row_bytes(fmt, I);
    int64_t t;
    if (!mul_ok(((int64_t)O + 15) / 16, (rb + 63) / 64, &t) || !mul_ok(t, 1024, &t) || !mul_ok(t, count, &t))
        return -1;
    return t;
}

/* Bytes of one weight matrix [O, I] in the given layout. */
static int64_t matrix_bytes(int fmt, int layout, int O, int I)
{
    int64_t t;
    if (layout == COLI_LAYOUT_TILED || layout == COLI_LAYOUT_TILED_GROUPED)
        return coli_tiled_bytes(fmt, 1, O, I);
    if (!mul_ok(coli_row_bytes(fmt, I), O, &t)) return -1;
    return t;
}

static int valid_gs(int gs)
{
    return gs == 32 || gs == 64 || gs == 128 || gs == 256 || gs == 512 || gs == 1024;
}

static int check_mlp_tensors(int fmt, int layout, int gs, int D, int F, const void *wg, const void *wu,
                             const void *wd, const float *sg, const float *su,
                             const float *sd, int64_t count)
{
    if (fmt != COLI_I8 && fmt != COLI_I4 && fmt != COLI_I2) return COLI_EFMT;
    if (layout != COLI_LAYOUT_ROWS && layout != COLI_LAYOUT_TILED && layout != COLI_LAYOUT_TILED_GROUPED)
        return COLI_EINVAL;
    /* grouped scales: int4 in the grouped tiled layout, and only there */
    if (gs != 0 && !valid_gs(gs)) return COLI_ERANGE;
    if ((gs != 0) != (layout == COLI_LAYOUT_TILED_GROUPED)) return COLI_EINVAL;
    if (gs != 0 && fmt != COLI_I4) return COLI_EFMT;
    if (gs != 0 && (!aligned(sg, 16) || !aligned(su, 16) || !aligned(sd, 16))) return COLI_EALIGN;
    if (F < 1 || D < 1) return COLI_ESHAPE;
    int64_t a = matrix_bytes(fmt, layout, F, D), b = matrix_bytes(fmt, layout, D, F);
    if (a < 0 || b < 0 || !mul_ok(a, count, &a) || !mul_ok(b, count, &b)) return COLI_ESHAPE;
    if (!wg || !wu || !wd || !sg || !su || !sd) return COLI_EINVAL;
    if (!aligned(wg, 4) || !aligned(wu, 4) || !aligned(wd, 4) || !aligned(sg, 4) ||
        !aligned(su, 4) || !aligned(sd, 4))
        return COLI_EALIGN;
    /* the tiled layouts are read by the matrix-core kernels only */
    if (layout != COLI_LAYOUT_ROWS &&
        (coli_row_bytes(fmt, D) % 16 || coli_row_bytes(fmt, F) % 16 || !aligned(wg, 16) ||
         !aligned(wu, 16) || !aligned(wd, 16)))
        return COLI_EALIGN;
    return COLI_OK;
}

int coli__check_pack(int fmt, const void *W, int64_t count, int O, int I, const void *dst)
{
    if (fmt != COLI_I8 && fmt != COLI_I4 && fmt != COLI_I2) return COLI_EFMT;
    if (count < 0 || O < 0 || I < 0 || coli_tiled_bytes(fmt, count, O, I) < 0) return COLI_ESHAPE;
    int64_t t;
    if (!mul_ok(coli_row_bytes(fmt, I), O, &t) || !mul_ok(t, count, &t)) return COLI_ESHAPE;
    if (count == 0 || O == 0 || I == 0) return COLI_OK;
    if (!W || !dst) return COLI_EINVAL;
    if (coli_row_bytes(fmt, I) % 16 || !aligned(W, 16) || !aligned(dst, 16)) return COLI_EALIGN;
    return COLI_OK;
}

/* The expert kernels address one weight matrix, and one activation row
 * table, with 32-bit byte offsets (cheaper address arithmetic in the inner
 * loop).  Both must stay below 2^32 - 4096 bytes: per matrix F * rb(D) and
 * D * rb(F) (routed and shared), and the row tables of x (S rows) and of the
 * SwiGLU output (S K rows, plus S for a shared expert), 4 (fp32 precision)
 * or 2 (bf16 precision) bytes per element of the width rounded up to 1024. */
static int check_off32(const coli_experts *ex, const coli_mlp *sh, int S, int K, int prec)
{
    const int64_t lim = ((int64_t)1 << 32) - 4096;
    const int64_t Fmax = sh && sh->F > ex->F ? sh->F : ex->F;
    const int64_t eb = prec == COLI_PREC_IDOT ? 1 : prec == COLI_PREC_BF16 ? 2 : 4;
    const int64_t rows = (int64_t)S * K + (sh ? S : 0);
    int64_t t;
    t = matrix_bytes(ex->fmt, ex->layout, ex->F, ex->D);
    if (t < 0 || t >= lim) return COLI_ERANGE;
    t = matrix_bytes(ex->fmt, ex->layout, ex->D, ex->F);
    if (t < 0 || t >= lim) return COLI_ERANGE;
    if (sh) {
        t = matrix_bytes(sh->fmt, sh->layout, sh->F, ex->D);
        if (t < 0 || t >= lim) return COLI_ERANGE;
        t = matrix_bytes(sh->fmt, sh->layout, ex->D, sh->F);
        if (t < 0 || t >= lim) return COLI_ERANGE;
    }
    if (!mul_ok((int64_t)S, eb * coli__kpad(ex->D), &t) || t >= lim) return COLI_ERANGE;
    if (!mul_ok(rows, eb * coli__kpad(Fmax), &t) || t >= lim) return COLI_ERANGE;
    return COLI_OK;
}

int coli__check_moe(const coli_experts *ex, const coli_mlp *sh, const float *x,
                    int S, int K, const int32_t *idx, const float *w,
                    const float *out, int prec, const void *ws, size_t ws_bytes,
                    int need_routing)
{
    if (!ex) return COLI_EINVAL;
    if (prec != COLI_PREC_FP32 && prec != COLI_PREC_BF16 && prec != COLI_PREC_IDOT) return COLI_EINVAL;
    if (S < 0 || K < 0 || ex->E < 0 || ex->D < 0 || ex->F < 0) return COLI_ESHAPE;
    if (ex->E < 1 || ex->E > COLI_MAX_E || K < 1 || K > COLI_MAX_K) return COLI_ERANGE;
    int rc = check_mlp_tensors(ex->fmt, ex->layout, ex->gs, ex->D, ex->F, ex->w_gate, ex->w_up, ex->w_down,
                               ex->s_gate, ex->s_up, ex->s_down, ex->E);
    if (rc) return rc;
    if (sh) {
        if (sh->F < 1) return COLI_ESHAPE;
        rc = check_mlp_tensors(sh->fmt, sh->layout, sh->gs, ex->D, sh->F, sh->w_gate, sh->w_up, sh->w_down,
                               sh->s_gate, sh->s_up, sh->s_down, 1);
        if (rc) return rc;
        /* a tiled shared expert runs as one more group of the routed kernels */
        if (sh->layout != COLI_LAYOUT_ROWS &&
            (ex->layout != sh->layout || sh->fmt != ex->fmt || sh->F != ex->F || sh->gs != ex->gs))
            return COLI_EINVAL;
    }
    if (ex->gs != 0 && prec == COLI_PREC_IDOT) return COLI_EFMT;   /* no integer dots with grouped scales */
    if (prec == COLI_PREC_IDOT) {
        /* the integer-dot kernels: int8 / int4, tiled, rows of whole 16-byte
         * segments, widths within the quantiser's 16384 */
        if (ex->fmt != COLI_I8 && ex->fmt != COLI_I4) return COLI_EFMT;
        if (ex->layout != COLI_LAYOUT_TILED) return COLI_EINVAL;
        if (coli_row_bytes(ex->fmt, ex->D) % 16 || coli_row_bytes(ex->fmt, ex->F) % 16) return COLI_ESHAPE;
        if (ex->D > 16384 || ex->F > 16384) return COLI_ERANGE;
        if (sh && (sh->layout != COLI_LAYOUT_TILED || sh->fmt != ex->fmt || sh->F != ex->F)) return COLI_EINVAL;
    }
    int64_t t;
    if (!mul_ok((int64_t)S, ex->D, &t) || !mul_ok(t, 4, &t)) return COLI_ESHAPE;
    size_t need = coli_moe_workspace_bytes(S, K, ex->E, ex->D, ex->F, sh ? sh->F : 0, prec);
    if (need == 0) return COLI_ESHAPE;
    rc = check_off32(ex, sh, S, K, prec);
    if (rc) return rc;
    if (S == 0) return COLI_OK;
    if (!x || !out) return COLI_EINVAL;
    if (need_routing && (!idx || !w)) return COLI_EINVAL;
    if (!aligned(x, 4) || !aligned(out, 4) || (idx && !aligned(idx, 4)) || (w && !aligned(w, 4)))
        return COLI_EALIGN;
    if (!ws || ws_bytes < need) return COLI_EWORKSPACE;
    if (!aligned(ws, ALIGN_WS)) return COLI_EALIGN;
    return COLI_OK;
}

int64_t coli_grouped_scale_bytes(int64_t count, int O, int I, int gs)
{
    if (count < 0 || O < 0 || I < 0 || !valid_gs(gs)) return -1;
    int64_t t;
    const int64_t ngp = coli__kpad(I) / gs;
    if (!mul_ok(count, (O + 15) / 16, &t) || !mul_ok(t, ngp, &t) || !mul_ok(t, 64, &t)) return -1;
    return t;
}

int coli__check_pack_scales(const float *S, int64_t count, int O, int I, int gs, const float *dst)
{
    if (!valid_gs(gs)) return COLI_ERANGE;
    if (count < 0 || O < 0 || I < 0 || coli_grouped_scale_bytes(count, O, I, gs) < 0) return COLI_ESHAPE;
    if (count == 0 || O == 0 || I == 0) return COLI_OK;
    if (!S || !dst) return COLI_EINVAL;
    if (!aligned(S, 4) || !aligned(dst, 16)) return COLI_EALIGN;
    return COLI_OK;
}
