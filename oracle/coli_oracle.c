/*
 * coli_oracle.c -- plain, slow CPU reference of the dequant-on-use qgemv and
 * its batched MoE form.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file; only the tests, the smoke check and the benchmark's CPU
 * baseline leg do.  It shares no code, header, table or constant with the HIP
 * library: every step below is written out from the pages' definitions.
 *
 * Arithmetic: every sum and product is carried in fp64; results are handed
 * back in fp64 (the caller rounds where it compares).  The one place the
 * pages fix a narrower precision -- the router's selection key, sigmoid value
 * plus bias taken in fp32 -- is done in fp32 on purpose (see cor_router).
 * OpenMP is used only to split independent output rows / tokens across
 * threads; it never changes the order of any sum.
 *
 * Sources (page title -- section):
 *   [glm.c@98759bf]   colibri-strix c/glm.c, commit 98759bf
 *   [glm.c@97c756a]   colibri-strix c/glm.c, commit 97c756a
 *   [metal@93cde63]   colibri c/backend_metal.mm, commit 93cde63
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Format codes: the QT tensor's fmt field [glm.c@98759bf -- typedef QT]:
 * 0 f32, 1 int8, 2 int4 two per byte, 3 int2 four per byte. */
enum { OR_F32 = 0, OR_I8 = 1, OR_I4 = 2, OR_I2 = 3 };

int cor_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Host threads for the parallel loops that follow (n >= 1). Work is split
 * over output rows or tokens, each result summed by one thread in a fixed
 * order, so the thread count changes timing only, never a value. Returns
 * the previous count. */
int cor_set_threads(int n)
{
    const int prev = cor_num_threads();
#ifdef _OPENMP
    if (n >= 1) omp_set_num_threads(n);
#else
    (void)n;
#endif
    return prev;
}

/* Bytes of one packed row of I elements [glm.c@98759bf -- qt_bytes]. */
int64_t cor_row_bytes(int fmt, int64_t I)
{
    switch (fmt) {
    case OR_F32: return 4 * I;
    case OR_I8:  return I;
    case OR_I4:  return (I + 1) / 2;
    case OR_I2:  return (I + 3) / 4;
    default:     return -1;
    }
}

/* Value of element i of one packed row, as an exact integer (or the f32
 * weight itself).
 *   int8: the byte read as a signed char            [glm.c@98759bf -- matmul_q]
 *   int4: element i sits in byte i/2; even i takes the low nibble, odd i the
 *         high nibble; value = nibble - 8           [glm.c@98759bf -- matmul_i4]
 *   int2: element i sits in byte i/4 at bits 2*(i%4)..2*(i%4)+1;
 *         value = crumb - 2                         [glm.c@98759bf -- matmul_i2]
 */
double cor_unpack(int fmt, const uint8_t *row, int64_t i)
{
    switch (fmt) {
    case OR_F32: {
        float f;
        memcpy(&f, row + 4 * i, sizeof f);
        return (double)f;
    }
    case OR_I8:
        return (double)(int8_t)row[i];
    case OR_I4: {
        unsigned b = row[i / 2];
        unsigned nib = (i % 2 == 0) ? (b & 0xFu) : (b >> 4);
        return (double)((int)nib - 8);
    }
    case OR_I2: {
        unsigned b = row[i / 4];
        unsigned crumb = (b >> (2 * (i % 4))) & 0x3u;
        return (double)((int)crumb - 2);
    }
    default:
        return NAN;
    }
}

/* One output of the quantized matrix-vector product
 *   y = scale[o] * sum_i v(o,i) * x[i]
 * with the scale applied after the sum [glm.c@98759bf -- matmul_q, matmul_i4,
 * matmul_i2; metal@93cde63 -- mm_gemv].  `mag` receives
 *   |scale[o]| * sum_i |v(o,i) * x[i]|,
 * the magnitude the float tolerance is measured against.  scale == NULL means
 * 1 (only meaningful for f32 rows, whose glm.c path carries no scale). */
static double qdot(int fmt, const uint8_t *row, const double *x, int64_t I,
                   double scale, double *mag)
{
    double acc = 0.0, am = 0.0;
    for (int64_t i = 0; i < I; ++i) {
        double t = cor_unpack(fmt, row, i) * x[i];
        acc += t;
        am += fabs(t);
    }
    if (mag) *mag = fabs(scale) * am;
    return scale * acc;
}

/* The grouped-scale form of qdot [docs-quickstart -- qt_resolve_fmt, the
 * int4-grouped format]: sum_g sc[g] * sum_{i in group g} v(i) x[i], groups
 * of gs consecutive elements (the last one shorter), in fp64; mag =
 * sum_g |sc[g]| sum_{i in g} |v x|. */
static double qdot_grouped(int fmt, const uint8_t *row, const double *x, int64_t I, int gs,
                           const float *sc, double *mag)
{
    double acc = 0.0, am = 0.0;
    int64_t ng = (I + gs - 1) / gs;
    for (int64_t g = 0; g < ng; ++g) {
        double part = 0.0, pm = 0.0;
        int64_t lo = g * gs, hi = lo + gs < I ? lo + gs : I;
        for (int64_t i = lo; i < hi; ++i) {
            double t = cor_unpack(fmt, row, i) * x[i];
            part += t;
            pm += fabs(t);
        }
        acc += (double)sc[g] * part;
        am += fabs((double)sc[g]) * pm;
    }
    if (mag) *mag = am;
    return acc;
}

/* y[s,o] = scale[o] * sum_i v(o,i) x[s,i] over x given in fp64.
 * W is [O, row_bytes(I)] row-major; y and mag are [S,O] (mag may be NULL). */
int cor_qgemv_d(int fmt, const void *W, const float *scale, const double *x,
                int S, int I, int O, double *y, double *mag)
{
    int64_t rb = cor_row_bytes(fmt, I);
    if (rb < 0 || S < 0 || I < 0 || O < 0) return -1;
    const uint8_t *Wb = (const uint8_t *)W;
#pragma omp parallel for schedule(static)
    for (int o = 0; o < O; ++o) {
        const uint8_t *row = Wb + (int64_t)o * rb;
        double sc = scale ? (double)scale[o] : 1.0;
        for (int s = 0; s < S; ++s) {
            double m;
            double v = qdot(fmt, row, x + (int64_t)s * I, I, sc, &m);
            y[(int64_t)s * O + o] = v;
            if (mag) mag[(int64_t)s * O + o] = m;
        }
    }
    return 0;
}

/* Same product over fp32 x (widened exactly to fp64 first). */
int cor_qgemv(int fmt, const void *W, const float *scale, const float *x,
              int S, int I, int O, double *y, double *mag)
{
    int64_t n = (int64_t)S * I;
    double *xd = (double *)malloc((size_t)(n > 0 ? n : 1) * sizeof(double));
    if (!xd) return -2;
    for (int64_t k = 0; k < n; ++k) xd[k] = (double)x[k];
    int rc = cor_qgemv_d(fmt, W, scale, xd, S, I, O, y, mag);
    free(xd);
    return rc;
}

/* ------------------------------------------------------------------------
 * Router: sigmoid scores, noaux_tc selection with one group, top-K weights
 * [glm.c@98759bf -- moe, phase A; metal@93cde63 -- r_router, r_top8].
 *
 * Per token s:
 *   logit[e] = sum_d Wr[e,d] * x[s,d]                       (fp64)
 *   sig[e]   = fp32( 1 / (1 + exp(-logit[e])) )             (fp64, rounded once)
 *   c[e]     = sig[e] + bias[e]                             (an fp32 add)
 *   K times: take the not-yet-taken expert with the largest c, scanning e
 *            upward and replacing only on a strictly larger value, so the
 *            lowest index wins a tie;  w[kk] = sig[best]    (the score, not c)
 *   if norm_topk: w[kk] /= (sum_kk w + 1e-20)
 *   w[kk] *= routed_scale
 * The selection key is an fp32 value on both the pages' CPU and GPU paths, so
 * it is kept in fp32 here too; the logit itself is taken in fp64 and the
 * sigmoid rounded once, a precision the GPU side can reproduce exactly.
 *
 * topp in (0,1) enables the adaptive truncation the pages offer as an option
 * [glm.c@98759bf -- moe, phase A, TOPP]: the K picks are reordered by
 * descending weight (stable: ties keep selection order), and keff is the
 * shortest prefix whose running fp32 sum reaches topp * (1e-20 + total); the
 * normalisation and scaling then use that prefix only.  topp outside (0,1)
 * keeps all K (keff = K).
 *
 * Outputs: idx[S,K] int32, w[S,K] fp64 (entries past keff are 0 / -1),
 * keff[S] (may be NULL), sig[S,E] fp32 (may be NULL), logit[S,E] fp64
 * (may be NULL).
 * ------------------------------------------------------------------------ */
int cor_router(const float *Wr, const float *bias, const float *x, int S,
               int E, int D, int K, int norm_topk, double routed_scale,
               double topp, int32_t *idx, double *w, int32_t *keff,
               float *sig_out, double *logit_out)
{
    if (S < 0 || E <= 0 || D <= 0 || K <= 0 || K > E) return -1;
    int rc = 0;
#pragma omp parallel
    {
        float *sig = (float *)malloc((size_t)E * sizeof(float));
        float *c = (float *)malloc((size_t)E * sizeof(float));
        unsigned char *taken = (unsigned char *)malloc((size_t)E);
        int *pick = (int *)malloc((size_t)K * sizeof(int));
        float *pw = (float *)malloc((size_t)K * sizeof(float));
        int ok = sig && c && taken && pick && pw;
        if (!ok) {
#pragma omp atomic write
            rc = -2;
        }
        /* every thread reaches the work-sharing loop, even one whose
         * scratch allocation failed (it then skips its share) */
        {
#pragma omp for schedule(static)
            for (int s = 0; s < S; ++s) {
                if (!ok) continue;
                const float *xs = x + (int64_t)s * D;
                for (int e = 0; e < E; ++e) {
                    const float *we = Wr + (int64_t)e * D;
                    double l = 0.0;
                    for (int d = 0; d < D; ++d) l += (double)we[d] * (double)xs[d];
                    double sg = 1.0 / (1.0 + exp(-l));
                    sig[e] = (float)sg;
                    c[e] = sig[e] + bias[e];
                    if (logit_out) logit_out[(int64_t)s * E + e] = l;
                    if (sig_out) sig_out[(int64_t)s * E + e] = sig[e];
                }
                memset(taken, 0, (size_t)E);
                for (int kk = 0; kk < K; ++kk) {
                    int best = -1;
                    for (int e = 0; e < E; ++e) {
                        if (taken[e]) continue;
                        if (best < 0 || c[e] > c[best]) best = e;
                    }
                    taken[best] = 1;
                    pick[kk] = best;
                    pw[kk] = sig[best];
                }
                int ke = K;
                if (topp > 0.0 && topp < 1.0) {
                    /* stable reorder by descending weight */
                    for (int a = 1; a < K; ++a) {
                        int ii = pick[a];
                        float wv = pw[a];
                        int b = a - 1;
                        while (b >= 0 && pw[b] < wv) {
                            pw[b + 1] = pw[b];
                            pick[b + 1] = pick[b];
                            --b;
                        }
                        pw[b + 1] = wv;
                        pick[b + 1] = ii;
                    }
                    /* keff is an integer decided by float compares: it is
                     * taken in the pages' fp32, in their order */
                    float tot = 1e-20f, cum = 0.f, tp = (float)topp;
                    for (int kk = 0; kk < K; ++kk) tot += pw[kk];
                    for (int kk = 0; kk < K; ++kk) {
                        cum += pw[kk];
                        if (cum >= tp * tot) { ke = kk + 1; break; }
                    }
                }
                double sum = 0.0;
                for (int kk = 0; kk < ke; ++kk) sum += pw[kk];
                double den = norm_topk ? sum + 1e-20 : 1.0;
                for (int kk = 0; kk < K; ++kk) {
                    idx[(int64_t)s * K + kk] = kk < ke ? pick[kk] : -1;
                    w[(int64_t)s * K + kk] =
                        kk < ke ? ((double)pw[kk] / den) * routed_scale : 0.0;
                }
                if (keff) keff[s] = ke;
            }
        }
        free(sig); free(c); free(taken); free(pick); free(pw);
    }
    return rc;
}

/* ------------------------------------------------------------------------
 * Expert MLP and MoE combine.
 *
 * One expert on one token row [glm.c@98759bf -- moe, phase D; dense_mlp]:
 *   g = gate(x), u = up(x)           (two qgemv's over the same x)
 *   h[j] = silu(g[j]) * u[j],  silu(z) = z / (1 + exp(-z))
 *   y = down(h)
 * all in fp64 with no intermediate rounding.
 * MoE output for token s [glm.c@98759bf -- moe, phases D and E]:
 *   out[s] = sum_{kk < keff} w[s,kk] * y_{idx[s,kk]}(x_s)  +  y_shared(x_s)
 * The shared expert (if any) is the same MLP with weight 1 on every token.
 *
 * Magnitude returned for the float tolerance (`mag`, per output element):
 *   sum_kk |w[s,kk]| * |sd[o]| * sum_j |vd(o,j) * h_j|   (+ the shared
 *   expert's |sd[o]| * sum_j |vd(o,j) * h_j|),
 * i.e. the per-product magnitude of the final contraction, weighted as it is
 * combined.
 * ------------------------------------------------------------------------ */
typedef struct {
    int fmt, E, D, F;
    const void *wg, *wu, *wd;   /* [E,F,rb(D)], [E,F,rb(D)], [E,D,rb(F)] */
    const float *sg, *su, *sd;  /* [E,F], [E,F], [E,D]; grouped: [E,F,ceil(D/gs)], .., [E,D,ceil(F/gs)] */
    int gs;                     /* 0: one scale per row; else int4 with one scale per gs elements */
} cor_experts;

typedef struct {
    int fmt, F;
    const void *wg, *wu, *wd;   /* [F,rb(D)], [F,rb(D)], [D,rb(F)] */
    const float *sg, *su, *sd;  /* [F], [F], [D]; grouped as for cor_experts */
    int gs;
} cor_mlp;

static double silu_d(double z) { return z / (1.0 + exp(-z)); }

/* One SwiGLU MLP on one fp64 row.  Buffers: g,u,h [F]; y, ymag [D].
 * Optional gmag/umag [F] receive the two projections' magnitudes. */
static void mlp_row(int fmt, int gs, int D, int F, const uint8_t *wg, const uint8_t *wu,
                    const uint8_t *wd, const float *sg, const float *su,
                    const float *sd, const double *x, double *g, double *u,
                    double *h, double *gmag, double *umag, double *y,
                    double *ymag)
{
    int64_t rbD = cor_row_bytes(fmt, D), rbF = cor_row_bytes(fmt, F);
    int64_t ngD = gs > 0 ? (D + gs - 1) / gs : 1, ngF = gs > 0 ? (F + gs - 1) / gs : 1;
    for (int j = 0; j < F; ++j) {
        double mg, mu;
        if (gs > 0) {
            g[j] = qdot_grouped(fmt, wg + (int64_t)j * rbD, x, D, gs, sg + j * ngD, &mg);
            u[j] = qdot_grouped(fmt, wu + (int64_t)j * rbD, x, D, gs, su + j * ngD, &mu);
        } else {
            g[j] = qdot(fmt, wg + (int64_t)j * rbD, x, D, sg ? sg[j] : 1.0, &mg);
            u[j] = qdot(fmt, wu + (int64_t)j * rbD, x, D, su ? su[j] : 1.0, &mu);
        }
        if (gmag) gmag[j] = mg;
        if (umag) umag[j] = mu;
        h[j] = silu_d(g[j]) * u[j];
    }
    for (int o = 0; o < D; ++o)
        y[o] = gs > 0 ? qdot_grouped(fmt, wd + (int64_t)o * rbF, h, F, gs, sd + o * ngF, &ymag[o])
                      : qdot(fmt, wd + (int64_t)o * rbF, h, F, sd ? sd[o] : 1.0, &ymag[o]);
}

/* Full MoE combine for S tokens.
 *   idx[S,K], w[S,K]: routing (w in fp64; pass the fp32 values the device
 *     used, widened, when comparing against a device run); entries with
 *     idx < 0 are skipped (a truncated keff).
 *   out, mag: [S,D].
 *   Optional per-pair intermediates (pair p = s*K + kk), any may be NULL:
 *     h_out [S*K, F]   SwiGLU output,
 *     g_out, u_out, gmag_out, umag_out [S*K, F]  gate/up values and magnitudes,
 *     y_out [S*K, D]   expert output before weighting.
 *   Shared-expert intermediates use row p = S*K + s of the same arrays when
 *   those arrays hold S*K + S rows (pair_rows == S*K + S), else are skipped.
 * Returns 0, or -1 on an out-of-range expert id. */
int cor_moe(const cor_experts *ex, const cor_mlp *sh, const float *x, int S,
            int K, const int32_t *idx, const double *w, double *out,
            double *mag, int64_t pair_rows, double *h_out, double *g_out,
            double *u_out, double *gmag_out, double *umag_out, double *y_out)
{
    int E = ex->E, D = ex->D, F = ex->F, fmt = ex->fmt;
    int Fs = sh ? sh->F : 0;
    int64_t rbD = cor_row_bytes(fmt, D), rbF = cor_row_bytes(fmt, F);
    /* scales per row: one, or one per group of gs elements */
    int64_t ngD = ex->gs > 0 ? (D + ex->gs - 1) / ex->gs : 1;
    int64_t ngF = ex->gs > 0 ? (F + ex->gs - 1) / ex->gs : 1;
    if (ex->gs < 0 || (ex->gs > 0 && fmt != OR_I4)) return -1;
    if (sh && (sh->gs < 0 || (sh->gs > 0 && sh->fmt != OR_I4))) return -1;
    int64_t rbDs = sh ? cor_row_bytes(sh->fmt, D) : 0;
    int64_t rbFs = sh ? cor_row_bytes(sh->fmt, Fs) : 0;
    int Fmax = F > Fs ? F : Fs;
    int rc = 0;
    for (int64_t p = 0; p < (int64_t)S * K; ++p)
        if (idx[p] >= E) return -1;
#pragma omp parallel
    {
        double *xd = (double *)malloc((size_t)D * sizeof(double));
        double *g = (double *)malloc((size_t)Fmax * sizeof(double));
        double *u = (double *)malloc((size_t)Fmax * sizeof(double));
        double *h = (double *)malloc((size_t)Fmax * sizeof(double));
        double *gm = (double *)malloc((size_t)Fmax * sizeof(double));
        double *um = (double *)malloc((size_t)Fmax * sizeof(double));
        double *y = (double *)malloc((size_t)D * sizeof(double));
        double *ym = (double *)malloc((size_t)D * sizeof(double));
        int ok = xd && g && u && h && gm && um && y && ym;
        if (!ok) {
#pragma omp atomic write
            rc = -2;
        }
        {
#pragma omp for schedule(dynamic, 1)
            for (int s = 0; s < S; ++s) {
                if (!ok) continue;
                double *os = out + (int64_t)s * D, *ms = mag + (int64_t)s * D;
                for (int d = 0; d < D; ++d) {
                    xd[d] = (double)x[(int64_t)s * D + d];
                    os[d] = 0.0;
                    ms[d] = 0.0;
                }
                for (int kk = 0; kk < K; ++kk) {
                    int64_t p = (int64_t)s * K + kk;
                    int e = idx[p];
                    if (e < 0) continue;
                    mlp_row(fmt, ex->gs, D, F,
                            (const uint8_t *)ex->wg + (int64_t)e * F * rbD,
                            (const uint8_t *)ex->wu + (int64_t)e * F * rbD,
                            (const uint8_t *)ex->wd + (int64_t)e * D * rbF,
                            ex->sg ? ex->sg + (int64_t)e * F * ngD : NULL,
                            ex->su ? ex->su + (int64_t)e * F * ngD : NULL,
                            ex->sd ? ex->sd + (int64_t)e * D * ngF : NULL,
                            xd, g, u, h, gm, um, y, ym);
                    double wk = w[p];
                    for (int d = 0; d < D; ++d) {
                        os[d] += wk * y[d];
                        ms[d] += fabs(wk) * ym[d];
                    }
                    if (h_out) memcpy(h_out + p * F, h, (size_t)F * sizeof(double));
                    if (g_out) memcpy(g_out + p * F, g, (size_t)F * sizeof(double));
                    if (u_out) memcpy(u_out + p * F, u, (size_t)F * sizeof(double));
                    if (gmag_out) memcpy(gmag_out + p * F, gm, (size_t)F * sizeof(double));
                    if (umag_out) memcpy(umag_out + p * F, um, (size_t)F * sizeof(double));
                    if (y_out) memcpy(y_out + p * D, y, (size_t)D * sizeof(double));
                }
                if (sh) {
                    mlp_row(sh->fmt, sh->gs, D, Fs, (const uint8_t *)sh->wg,
                            (const uint8_t *)sh->wu, (const uint8_t *)sh->wd,
                            sh->sg, sh->su, sh->sd, xd, g, u, h, gm, um, y, ym);
                    for (int d = 0; d < D; ++d) {
                        os[d] += y[d];
                        ms[d] += ym[d];
                    }
                    int64_t p = (int64_t)S * K + s;
                    if (pair_rows == (int64_t)S * K + S) {
                        /* shared rows share the F stride only when Fs == F */
                        if (Fs == F) {
                            if (h_out) memcpy(h_out + p * F, h, (size_t)F * sizeof(double));
                            if (g_out) memcpy(g_out + p * F, g, (size_t)F * sizeof(double));
                            if (u_out) memcpy(u_out + p * F, u, (size_t)F * sizeof(double));
                            if (gmag_out) memcpy(gmag_out + p * F, gm, (size_t)F * sizeof(double));
                            if (umag_out) memcpy(umag_out + p * F, um, (size_t)F * sizeof(double));
                        }
                        if (y_out) memcpy(y_out + p * D, y, (size_t)D * sizeof(double));
                    }
                }
            }
        }
        free(xd); free(g); free(u); free(h); free(gm); free(um); free(y); free(ym);
    }
    (void)rbDs; (void)rbFs;
    return rc;
}

/* ------------------------------------------------------------------------
 * Grouped-scale int4 (the pages' fmt 4, "int4-grouped") [docs-quickstart --
 * qt_resolve_fmt; glm.c@98759bf -- qt_from_disk]: the int4 row layout, with
 * one fp32 scale per group of gs consecutive elements along I instead of one
 * per row; scale is [O, ng], ng = ceil(I / gs), the last group shorter when
 * gs does not divide I:
 *   y[s,o] = sum_g scale[o, g] * sum_{i in group g} v(o,i) x[s,i],
 * in fp64; mag = sum_g |scale[o, g]| sum_{i in g} |v x|.
 * ------------------------------------------------------------------------ */
int cor_qgemv_grouped(const void *W, const float *scale, int gs, const float *x,
                      int S, int I, int O, double *y, double *mag)
{
    if (gs < 1 || S < 0 || I < 0 || O < 0) return -1;
    int64_t rb = cor_row_bytes(OR_I4, I);
    int ng = (I + gs - 1) / gs;
#pragma omp parallel for schedule(static)
    for (int o = 0; o < O; ++o) {
        const uint8_t *row = (const uint8_t *)W + (int64_t)o * rb;
        for (int s = 0; s < S; ++s) {
            const float *xs = x + (int64_t)s * I;
            double acc = 0.0, am = 0.0;
            for (int g = 0; g < ng; ++g) {
                double part = 0.0, pm = 0.0;
                int lo = g * gs, hi = lo + gs < I ? lo + gs : I;
                for (int i = lo; i < hi; ++i) {
                    double t = cor_unpack(OR_I4, row, i) * (double)xs[i];
                    part += t;
                    pm += fabs(t);
                }
                double sg = (double)scale[(int64_t)o * ng + g];
                acc += sg * part;
                am += fabs(sg) * pm;
            }
            y[(int64_t)s * O + o] = acc;
            if (mag) mag[(int64_t)s * O + o] = am;
        }
    }
    return 0;
}

/* ------------------------------------------------------------------------
 * Integer-dot qgemv (IDOT) [glm.c@98759bf -- qrow_i8, dot_i8i8, dot_i4i8,
 * matmul_q_idot, matmul_i4_idot]: each activation row is quantised to int8
 * by its absolute maximum, the dot product with the int8 / int4 weight
 * values is taken in exact integer arithmetic, and the result is scaled back
 * in fp32.  A lossy variant by design; the pages fix every step in fp32:
 *   amax = max_i |x_i|;  s = amax / 127 (at least 1e-12);  inv = 1 / s;
 *   q_i = round-half-even(x_i * inv) as int8;
 *   y[s,o] = ((float)dot(v(o,.), q) * scale[o]) * s,
 * rounded in fp32 after each operation, which the oracle reproduces
 * (volatile forces the roundings).  The dot itself is exact (int64 here).
 * ------------------------------------------------------------------------ */
float cor_qrow_i8(const float *x, int I, int8_t *q)
{
    float amax = 0.f;
    for (int i = 0; i < I; ++i) {
        float a = fabsf(x[i]);
        if (a > amax) amax = a;
    }
    volatile float s = amax / 127.f;
    if (s < 1e-12f) s = 1e-12f;
    volatile float inv = 1.f / s;
    for (int i = 0; i < I; ++i) {
        volatile float t = x[i] * inv;
        q[i] = (int8_t)lrintf(t);   /* round half to even (default mode) */
    }
    return s;
}

/* y [S,O] fp32; fmt int8 or int4 only (the pages' IDOT formats); also
 * returns the exact integer dots in dot_out [S,O] (may be NULL). */
int cor_qgemv_idot(int fmt, const void *W, const float *scale, const float *x,
                   int S, int I, int O, float *y, int64_t *dot_out)
{
    if (fmt != OR_I8 && fmt != OR_I4) return -1;
    int64_t rb = cor_row_bytes(fmt, I);
    int8_t *xq = (int8_t *)malloc((size_t)S * I + 1);
    float *sx = (float *)malloc((size_t)S * sizeof(float) + 4);
    if (!xq || !sx) { free(xq); free(sx); return -2; }
    for (int s = 0; s < S; ++s) sx[s] = cor_qrow_i8(x + (int64_t)s * I, I, xq + (int64_t)s * I);
#pragma omp parallel for schedule(static)
    for (int o = 0; o < O; ++o) {
        const uint8_t *row = (const uint8_t *)W + (int64_t)o * rb;
        for (int s = 0; s < S; ++s) {
            const int8_t *qs = xq + (int64_t)s * I;
            int64_t dot = 0;
            for (int i = 0; i < I; ++i) dot += (int64_t)cor_unpack(fmt, row, i) * qs[i];
            if (dot_out) dot_out[(int64_t)s * O + o] = dot;
            volatile float d = (float)dot;
            volatile float t = d * scale[o];
            y[(int64_t)s * O + o] = t * sx[s];
        }
    }
    free(xq);
    free(sx);
    return 0;
}

/* ------------------------------------------------------------------------
 * The MoE block on the integer-dot path [glm.c@98759bf -- moe, phase D, with
 * the expert matmuls taking the IDOT branch of matmul_qt (matmul_q_idot /
 * matmul_i4_idot)]: each product quantises its input row as cor_qrow_i8 does
 * and takes the exact integer dot, scaled back in fp32 in the pages' order:
 *   token row:  qx, sx = qrow_i8(x[s])        (once; every expert of the
 *                                              token and the shared expert)
 *   g[o] = ((float)dot(vg(o,.), qx) * sg[o]) * sx,   u[o] alike
 *   h[o] = silu(g[o]) * u[o],  silu(z) = z / (1 + expf(-z)), each step fp32
 *   qh, sh = qrow_i8(h)
 *   y[o] = ((float)dot(vd(o,.), qh) * sd[o]) * sh
 *   out[s] = sum_kk w[s,kk] y_kk + y_shared     (fp64 of the fp32 y)
 * h_in (may be NULL): [pair_rows, F] fp32; when given, the down product of
 * pair row p quantises h_in's row p instead of the h computed here (so a
 * caller can check another implementation's down products on its own h).
 * Outputs (each may be NULL): h_out [pair_rows, F], g_out [pair_rows, F] (the
 * gate product) and y_out [pair_rows, D] fp32, pair row p = s K + kk, the
 * shared expert's at S K + s (when pair_rows == S K + S).  Returns 0, -1 on an expert id >= E or an int16 /
 * int2 format, -2 on allocation failure.
 * ------------------------------------------------------------------------ */
static void idot_rows(int fmt, const uint8_t *W, int64_t rb, const float *sc, int O, int I,
                      const int8_t *q, float sq, float *out)
{
    for (int o = 0; o < O; ++o) {
        const uint8_t *row = W + (int64_t)o * rb;
        int64_t dot = 0;
        for (int i = 0; i < I; ++i) dot += (int64_t)cor_unpack(fmt, row, i) * q[i];
        volatile float d = (float)dot;
        volatile float t = d * sc[o];
        out[o] = t * sq;
    }
}

static void idot_mlp(int fmt, int D, int F, const uint8_t *wg, const uint8_t *wu, const uint8_t *wd,
                     const float *sg, const float *su, const float *sd, const int8_t *qx, float sx,
                     const float *h_in, float *g, float *u, float *h, int8_t *qh, float *y)
{
    int64_t rbD = cor_row_bytes(fmt, D), rbF = cor_row_bytes(fmt, F);
    idot_rows(fmt, wg, rbD, sg, F, D, qx, sx, g);
    idot_rows(fmt, wu, rbD, su, F, D, qx, sx, u);
    for (int o = 0; o < F; ++o) {
        volatile float e = expf(-g[o]);
        volatile float den = 1.0f + e;
        volatile float sl = g[o] / den;
        h[o] = sl * u[o];
    }
    float sh = cor_qrow_i8(h_in ? h_in : h, F, qh);
    idot_rows(fmt, wd, rbF, sd, D, F, qh, sh, y);
}

int cor_moe_idot(const cor_experts *ex, const cor_mlp *sh, const float *x, int S, int K,
                 const int32_t *idx, const double *w, const float *h_in, int64_t pair_rows,
                 double *out, float *h_out, float *y_out, float *g_out)
{
    int E = ex->E, D = ex->D, F = ex->F, fmt = ex->fmt;
    if (fmt != OR_I8 && fmt != OR_I4) return -1;
    if (ex->gs != 0 || (sh && (sh->fmt != fmt || sh->F != F || sh->gs != 0))) return -1;
    int64_t rbD = cor_row_bytes(fmt, D), rbF = cor_row_bytes(fmt, F);
    for (int64_t p = 0; p < (int64_t)S * K; ++p)
        if (idx[p] >= E) return -1;
    int rc = 0;
#pragma omp parallel
    {
        int8_t *qx = (int8_t *)malloc((size_t)D + 1), *qh = (int8_t *)malloc((size_t)F + 1);
        float *g = (float *)malloc((size_t)F * sizeof(float)), *u = (float *)malloc((size_t)F * sizeof(float));
        float *h = (float *)malloc((size_t)F * sizeof(float)), *y = (float *)malloc((size_t)D * sizeof(float));
        int ok = qx && qh && g && u && h && y;
        if (!ok) {
#pragma omp atomic write
            rc = -2;
        }
#pragma omp for schedule(dynamic, 1)
        for (int s = 0; s < S; ++s) {
            if (!ok) continue;
            double *os = out + (int64_t)s * D;
            for (int d = 0; d < D; ++d) os[d] = 0.0;
            float sx = cor_qrow_i8(x + (int64_t)s * D, D, qx);
            for (int kk = 0; kk <= K; ++kk) {
                int64_t p;
                const uint8_t *wg, *wu, *wd;
                const float *sg, *su, *sd;
                double wk;
                if (kk < K) {
                    p = (int64_t)s * K + kk;
                    int e = idx[p];
                    if (e < 0) continue;
                    wg = (const uint8_t *)ex->wg + (int64_t)e * F * rbD;
                    wu = (const uint8_t *)ex->wu + (int64_t)e * F * rbD;
                    wd = (const uint8_t *)ex->wd + (int64_t)e * D * rbF;
                    sg = ex->sg + (int64_t)e * F;
                    su = ex->su + (int64_t)e * F;
                    sd = ex->sd + (int64_t)e * D;
                    wk = w[p];
                } else {
                    if (!sh) break;
                    p = (int64_t)S * K + s;
                    wg = (const uint8_t *)sh->wg;
                    wu = (const uint8_t *)sh->wu;
                    wd = (const uint8_t *)sh->wd;
                    sg = sh->sg;
                    su = sh->su;
                    sd = sh->sd;
                    wk = 1.0;
                }
                const int have = p < pair_rows;
                idot_mlp(fmt, D, F, wg, wu, wd, sg, su, sd, qx, sx,
                         h_in && have ? h_in + p * F : NULL, g, u, h, qh, y);
                for (int d = 0; d < D; ++d) os[d] += wk * (double)y[d];
                if (h_out && have) memcpy(h_out + p * F, h, (size_t)F * sizeof(float));
                if (y_out && have) memcpy(y_out + p * D, y, (size_t)D * sizeof(float));
                if (g_out && have) memcpy(g_out + p * F, g, (size_t)F * sizeof(float));
            }
        }
        free(qx);
        free(qh);
        free(g);
        free(u);
        free(h);
        free(y);
    }
    return rc;
}

/* ------------------------------------------------------------------------
 * Layer tail around the MoE block [glm.c@98759bf -- rmsnorm; the layer
 * forward's post-attention half]: the residual stream x is normalised with
 * the post-attention RMSNorm, the MoE block runs on the normalised rows, and
 * its output is added back onto x.
 *
 * RMSNorm, in the precision the pages fix: the mean square is accumulated in
 * fp64 (each square exact in fp64), converted once to fp32, eps added in
 * fp32, r = 1 / sqrtf(.) in fp32, and each output is (x * r) * w rounded in
 * fp32 after each product.  This is a function the pages define with fp32
 * intermediates, so the oracle reproduces those roundings instead of
 * carrying fp64 through.
 * ------------------------------------------------------------------------ */
void cor_rmsnorm(const float *x, const float *w, int S, int D, float eps, float *out)
{
#pragma omp parallel for schedule(static)
    for (int s = 0; s < S; ++s) {
        const float *xs = x + (int64_t)s * D;
        float *os = out + (int64_t)s * D;
        double ms = 0.0;
        for (int i = 0; i < D; ++i) ms += (double)xs[i] * (double)xs[i];
        volatile float mean = (float)(ms / D);   /* one fp32 rounding, as on the pages */
        volatile float den = sqrtf(mean + eps);
        const float r = 1.0f / den;
        for (int i = 0; i < D; ++i) {
            volatile float xr = xs[i] * r;
            os[i] = xr * w[i];
        }
    }
}

/* ------------------------------------------------------------------------
 * Weight preparation helpers the pages define for filling QT tensors from
 * f32 weights; used by the tests to produce packed rows from known values,
 * never by the products above.
 *
 * Symmetric per-row quantisation [glm.c@98759bf -- quantize_rows]:
 *   qmax = 2^(bits-1) - 1; s = max(amax/qmax, 1e-8); q = lrint(w/s) clamped
 *   to [-qmax-1, qmax].
 * int4 packing [glm.c@98759bf -- pack_int4]: values clamped to [-8, qmax],
 *   stored as v+8, element 2k in the low nibble of byte k, 2k+1 in the high
 *   nibble; a missing last element of an odd row is stored as 8 (value 0).
 * int2 packing [glm.c@98759bf -- pack_int2]: values clamped to [-2, qmax],
 *   stored as v+2 at bits 2*(i%4) of byte i/4; missing elements leave 0 bits.
 * The arithmetic mirrors the pages' fp32 code (amax, division and rounding in
 * fp32), since these functions define stored bytes, not a float result.
 * ------------------------------------------------------------------------ */
static float row_scale(const float *wr, int I, int qmax)
{
    float amax = 0.f;
    for (int i = 0; i < I; ++i) {
        float a = fabsf(wr[i]);
        if (a > amax) amax = a;
    }
    float s = amax / (float)qmax;
    if (s < 1e-8f) s = 1e-8f;
    return s;
}

static int qclamp(float v, float s, int lo, int hi)
{
    int q = (int)lrintf(v / s);
    if (q > hi) q = hi;
    if (q < lo) q = lo;
    return q;
}

void cor_quantize_rows(const float *w, int8_t *q, float *scale, int O, int I, int bits)
{
    int qmax = (1 << (bits - 1)) - 1;
    for (int o = 0; o < O; ++o) {
        const float *wr = w + (int64_t)o * I;
        float s = row_scale(wr, I, qmax);
        scale[o] = s;
        for (int i = 0; i < I; ++i)
            q[(int64_t)o * I + i] = (int8_t)qclamp(wr[i], s, -qmax - 1, qmax);
    }
}

void cor_pack_int4(const float *w, uint8_t *q4, float *scale, int O, int I, int bits)
{
    int qmax = (1 << (bits - 1)) - 1;
    int64_t rb = (I + 1) / 2;
    for (int o = 0; o < O; ++o) {
        const float *wr = w + (int64_t)o * I;
        float s = row_scale(wr, I, qmax);
        scale[o] = s;
        for (int i = 0; i < I; i += 2) {
            int v0 = qclamp(wr[i], s, -8, qmax);
            int v1 = (i + 1 < I) ? qclamp(wr[i + 1], s, -8, qmax) : 0;
            q4[(int64_t)o * rb + i / 2] = (uint8_t)((v0 + 8) | ((v1 + 8) << 4));
        }
    }
}

void cor_pack_int2(const float *w, uint8_t *q2, float *scale, int O, int I, int bits)
{
    int qmax = (1 << (bits - 1)) - 1;
    int64_t rb = (I + 3) / 4;
    for (int o = 0; o < O; ++o) {
        const float *wr = w + (int64_t)o * I;
        float s = row_scale(wr, I, qmax);
        scale[o] = s;
        for (int i = 0; i < I; i += 4) {
            unsigned byte = 0;
            for (int k = 0; k < 4 && i + k < I; ++k)
                byte |= (unsigned)(qclamp(wr[i + k], s, -2, qmax) + 2) << (2 * k);
            q2[(int64_t)o * rb + i / 4] = (uint8_t)byte;
        }
    }
}
