/*
 * Multi-Token Attention forward: CPU ORACLE (test infrastructure only).
 *
 * This file is the plain, slow, literal float64 statement of what the MTA
 * attention forward computes.  It exists so that the GPU path can be checked
 * against it.  Only the tests, the smoke check and the benchmark's CPU-baseline
 * leg may load it; the product library never links or calls it, and it shares
 * no code, header or table with the GPU path.
 *
 * Source of every step: the web page "Multi-Token Attention — Paper Graph"
 * (a structured summary of arXiv 2504.00927), section 3.4 "Detailed,
 * Sentence-Based Technical Breakdown", subsections
 *   - "Standard Multi-Head Attention"       (logits, causal softmax, A·V)
 *   - "Key-Query Convolution"               (Conv2d_theta, Eq. 4, two-pass
 *                                             masking, post-softmax variant,
 *                                             Eq. 4's exact causal indicator)
 *   - "Head Mixing Convolution"             (Eq. 7 and its pre-softmax form)
 *   - "Putting Everything Together"         (composition order)
 *   - "Group Normalization with Sigmoid Gating" (GroupNorm per head; the
 *     alternative "layer-dependent depth scaling" is the scale used here)
 * and the companion overview page "Article Overview: Multi-Token Attention",
 * item 2 ("Group Normalization with Depth Scaling").
 *
 * Readings taken where the pages are silent (each is listed in the design
 * notes of the repository):
 *   - padding outside [0,T) in the key-query convolution is zero;
 *   - j' runs over [-floor(c_k/2), ceil(c_k/2)-1] as printed; the kernel
 *     column index is jj = j' + floor(c_k/2);
 *   - heads are grouped contiguously, w[g][a][b] maps source head b to output
 *     head a of group g, no bias;
 *   - when both convolutions sit on the same side of the softmax the
 *     key-query convolution runs first;
 *   - the post-softmax key-query convolution is not renormalised;
 *   - GroupNorm uses the biased variance over the d channels of one head at
 *     one token, epsilon from the caller, per-channel affine [H][d];
 *   - the depth scale is a scalar supplied by the caller, applied after the
 *     affine step.
 *
 * Parity status of every function here: pinned by the CPU test-suite
 * (library-routine special cases, closed forms, invariants, hand-computed
 * fixtures, brute force at tiny sizes).  No function is "parity unpinned".
 *
 * Build: gcc -O2 -fopenmp -shared -fPIC mta_oracle.c -o libmta_oracle.so -lm
 */
#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_PRE 0
#define ORACLE_POST 1
#define ORACLE_PRE_EXACT 2   /* before the softmax, Eq. 4 with its indicator */

/* Optional planted mistakes, used only by the oracle's own mutation test to
 * show that the pins catch them.  The default build has ORACLE_MUTANT == 0. */
#ifndef ORACLE_MUTANT
#define ORACLE_MUTANT 0
#endif

/* ------------------------------------------------------------------------ */
/* Step 1.  Logits  Ahat = Q K^T / sqrt(d)
 * ("Standard Multi-Head Attention": the attention logits are the scaled dot
 * products of each query with each key).  Rows [a0, a1) of the explicit
 * T x T matrix, all T columns (the future included; masking is a later,
 * separate step).  S is (a1-a0) x T. */
static void step_logits(const double *q, const double *k, int T, int d,
                        int a0, int a1, double *S)
{
    const double inv_sqrt_d = 1.0 / sqrt((double)d);
    for (int a = a0; a < a1; ++a)
        for (int j = 0; j < T; ++j) {
            double dot = 0.0;
            for (int c = 0; c < d; ++c) dot += q[(size_t)a * d + c] * k[(size_t)j * d + c];
#if ORACLE_MUTANT == 1 /* planted: forgot the 1/sqrt(d) scale */
            S[(size_t)(a - a0) * T + j] = dot;
#else
            S[(size_t)(a - a0) * T + j] = dot * inv_sqrt_d;
#endif
        }
}

/* Step 2.  Mask_0: future positions (j > i) are replaced by 0
 * ("Key-Query Convolution", two-pass masking: the first mask uses 0 so that
 * future logits do not contribute to the convolution; also the final Mask_0 of
 * the post-softmax variant).  In place on rows [a0,a1). */
static void step_mask_zero(double *X, int T, int a0, int a1)
{
    for (int a = a0; a < a1; ++a)
        for (int j = 0; j < T; ++j)
#if ORACLE_MUTANT == 2 /* planted: mask keeps the diagonal off */
            if (j >= a) X[(size_t)(a - a0) * T + j] = 0.0;
#else
            if (j > a) X[(size_t)(a - a0) * T + j] = 0.0;
#endif
}

/* Step 3.  Conv2d_theta over the (query, key) plane of one head
 * ("Key-Query Convolution", the expanded form Eq. 4):
 *   Y[i][j] = sum_{i'=0}^{c_q-1} sum_{j'=-floor(c_k/2)}^{ceil(c_k/2)-1}
 *                 [indicator] theta[i'][j' + floor(c_k/2)] * X[i-i'][j-j']
 * with X = 0 outside [0,T) x [0,T).
 *   indicator == 0: no indicator; the two-pass scheme applies it to the map
 *                   already masked by Mask_0 (and the post-softmax variant to
 *                   probabilities, which are 0 in the future);
 *   indicator == 1: Eq. 4's causal indicator 1{i >= j - j'}: a tap counts only
 *                   if its key is not in the future of the OUTPUT query i; X is
 *                   then the unmasked logit map.
 * X holds rows [x0, x0+nx); the caller passes every row in [0,T) the sum can
 * reach from output rows [i0,i1) (a row it does not hold yields NaN rather
 * than a silent zero). */
static void step_kq_conv(const double *X, int T, int x0, int nx,
                         const double *theta, int c_q, int c_k, int indicator,
                         int i0, int i1, double *Y)
{
    const int jlo = -(c_k / 2);            /* -floor(c_k/2)      */
    const int jhi = (c_k + 1) / 2 - 1;     /* ceil(c_k/2) - 1    */
    for (int i = i0; i < i1; ++i)
        for (int j = 0; j < T; ++j) {
            double acc = 0.0;
            for (int ip = 0; ip < c_q; ++ip) {
#if ORACLE_MUTANT == 3 /* planted: looks at later queries instead of earlier */
                const int r = i + ip;
#else
                const int r = i - ip;
#endif
                if (r < 0 || r >= T) continue;          /* zero padding */
                if (r < x0 || r >= x0 + nx) {           /* not held: caller error */
                    acc = NAN;
                    break;
                }
                for (int jp = jlo; jp <= jhi; ++jp) {
#if ORACLE_MUTANT == 4 /* planted: key offset sign flipped */
                    const int cidx = j + jp;
#else
                    const int cidx = j - jp;
#endif
                    if (cidx < 0 || cidx >= T) continue;  /* zero padding */
#if ORACLE_MUTANT == 9 /* planted: indicator taken against the input row */
                    if (indicator && cidx > r) continue;
#else
                    if (indicator && cidx > i) continue;  /* 1{i >= j - j'} */
#endif
#if ORACLE_MUTANT == 5 /* planted: kernel read transposed in its key axis */
                    const double th = theta[ip * c_k + (c_k - 1 - (jp - jlo))];
#else
                    const double th = theta[ip * c_k + (jp - jlo)];
#endif
                    acc += th * X[(size_t)(r - x0) * T + cidx];
                }
            }
            Y[(size_t)(i - i0) * T + j] = acc;
        }
}

/* Step 4.  Head mixing within a group of c_h heads
 * ("Head Mixing Convolution", Eq. 7 for probabilities and its pre-softmax
 * counterpart for logits):  Y^a = sum_b w[a][b] X^b, elementwise.
 * X and Y are arrays of c_h pointers to n-element maps. */
static void step_head_mix(double *const *X, const double *w, int c_h,
                          size_t n, double *const *Y)
{
    for (int a = 0; a < c_h; ++a)
        for (size_t e = 0; e < n; ++e) {
            double acc = 0.0;
            for (int b = 0; b < c_h; ++b)
#if ORACLE_MUTANT == 6 /* planted: mixing matrix transposed */
                acc += w[b * c_h + a] * X[b][e];
#else
                acc += w[a * c_h + b] * X[b][e];
#endif
            Y[a][e] = acc;
        }
}

/* Step 5.  Mask_{-inf} then softmax over keys
 * ("Standard Multi-Head Attention": positions j > i are set to -infinity and
 * each row is normalised over the key axis into a probability distribution).
 * Row a of X (absolute row index a) becomes a distribution over j <= a.  The
 * maximum is subtracted only for numerical range; exp(-inf) is exactly 0. */
static void step_causal_softmax(const double *X, int T, int a0, int a1, double *P)
{
    for (int a = a0; a < a1; ++a) {
        const double *x = X + (size_t)(a - a0) * T;
        double *p = P + (size_t)(a - a0) * T;
        double mx = -INFINITY;
        for (int j = 0; j < T; ++j) {
            const double l = (j > a) ? -INFINITY : x[j];
            if (l > mx) mx = l;
        }
        double sum = 0.0;
        for (int j = 0; j < T; ++j) {
            const double l = (j > a) ? -INFINITY : x[j];
            p[j] = exp(l - mx);
            sum += p[j];
        }
#if ORACLE_MUTANT == 7 /* planted: rows left unnormalised */
        (void)sum;
#else
        for (int j = 0; j < T; ++j) p[j] /= sum;
#endif
    }
}

/* Step 6.  Output per head  O = A V  ("Standard Multi-Head Attention"; after
 * post-softmax head mixing the mixed map of head a multiplies head a's own
 * values, "Head Mixing Convolution", the Appendix B identity). */
static void step_pv(const double *A, const double *v, int T, int d, int i0, int i1, double *O)
{
    for (int i = i0; i < i1; ++i)
        for (int c = 0; c < d; ++c) {
            double acc = 0.0;
            for (int j = 0; j < T; ++j) acc += A[(size_t)(i - i0) * T + j] * v[(size_t)j * d + c];
            O[(size_t)(i - i0) * d + c] = acc;
        }
}

/* Step 7.  GroupNorm with each head's d channels as one group, per-channel
 * affine, then the head's output scale ("Group Normalization with Sigmoid
 * Gating": heads are the normalisation groups, and each head's normalised
 * output is multiplied by sigma(g_h) for a learned per-head gate g; the
 * overview page names the alternative "Group Normalization with Depth
 * Scaling").  Biased variance.  `depth_scale` is the head's total factor. */
static void step_groupnorm_scale(const double *O, const double *gw, const double *gb,
                                 int d, int i0, int i1, double eps, double depth_scale,
                                 double *Y)
{
    for (int i = i0; i < i1; ++i) {
        const double *o = O + (size_t)(i - i0) * d;
        double mu = 0.0;
        for (int c = 0; c < d; ++c) mu += o[c];
        mu /= d;
        double var = 0.0;
        for (int c = 0; c < d; ++c) var += (o[c] - mu) * (o[c] - mu);
        var /= d;
        const double rstd = 1.0 / sqrt(var + eps);
        for (int c = 0; c < d; ++c)
            Y[(size_t)(i - i0) * d + c] = ((o[c] - mu) * rstd * gw[c] + gb[c]) * depth_scale;
    }
}

/* ------------------------------------------------------------------------ */
/* Composition for one (batch b, head group g) unit and output rows [r0, r1)
 * ("Putting Everything Together"): logits -> [kq conv pre: Mask_0, Conv2d,
 * then Mask_-inf; or, exact form, Conv2d with Eq. 4's indicator on the
 * unmasked logits, then Mask_-inf] -> [head mix pre] -> softmax -> [kq conv
 * post: Conv2d then Mask_0] -> [head mix post] -> A V -> GroupNorm x scale.
 *
 * Every stage is an explicit matrix over the extended rows [e0, r1) (the
 * key-query convolution looks c_q-1 query rows back) and all T key columns.
 * If `stages` is non-NULL the intermediate maps are copied out (tests).     */

typedef struct {
    int B, H, T, d, c_q, c_k, c_h, kq_place, head_place;
    double eps, depth_scale;
    const double *gate;  /* [H] per-head gate logits, or NULL (no gate) */
} oracle_cfg;

/* The sigmoid of the gate ("Group Normalization with Sigmoid Gating"). */
static double head_scale(const oracle_cfg *cf, int h)
{
    if (!cf->gate) return cf->depth_scale;
#if ORACLE_MUTANT == 8 /* planted: gate used without its sigmoid */
    return cf->depth_scale * cf->gate[h];
#else
    return cf->depth_scale / (1.0 + exp(-cf->gate[h]));
#endif
}

/* Stage dump layout for one unit, full rows [0,T) only:
 *   S, C, Cmix, P, P2, P3 : [c_h][T][T] each
 *   O, Y                  : [c_h][T][d] each (Y is after GroupNorm x scale) */
typedef struct {
    double *S, *C, *Cmix, *P, *P2, *P3, *O, *Y;
} oracle_stages;

static int unit_rows(const oracle_cfg *cf, const double *q, const double *k, const double *v,
                     const double *theta_kq, const double *theta_head,
                     const double *gn_w, const double *gn_b,
                     int b, int g, int r0, int r1, double *out, const oracle_stages *st)
{
    const int T = cf->T, d = cf->d, c_h = cf->c_h, H = cf->H;
    /* e0: first row the key-query convolution can reach from row r0 */
    const int e0 = (r0 - (cf->c_q - 1)) > 0 ? (r0 - (cf->c_q - 1)) : 0;
    const int ne = r1 - e0;           /* extended rows [e0, r1)   */
    const int nr = r1 - r0;           /* output rows   [r0, r1)   */
    const size_t ext = (size_t)ne * T;
    const size_t off = (size_t)(r0 - e0) * T;   /* offset of row r0 in an extended buffer */
    /* v0: first row on which the map entering the softmax is defined.  With the
     * key-query convolution before the softmax only the output rows are (the
     * convolution of a halo row would need rows further back); with it after
     * the softmax, the softmax must cover the halo rows too. */
    const int v0 = (cf->kq_place == ORACLE_POST) ? e0 : r0;
    const size_t voff = (size_t)(v0 - e0) * T;
    const size_t nv = (size_t)(r1 - v0) * T;
    int rc = 0;

    double **S = calloc(c_h, sizeof(double *));
    double **A1 = calloc(c_h, sizeof(double *));
    double **A2 = calloc(c_h, sizeof(double *));
    double **A3 = calloc(c_h, sizeof(double *));
    double **O = calloc(c_h, sizeof(double *));
    double **X = calloc(c_h, sizeof(double *));
    double **Y = calloc(c_h, sizeof(double *));
    if (!S || !A1 || !A2 || !A3 || !O || !X || !Y) { rc = -1; goto done; }
    for (int a = 0; a < c_h; ++a) {
        S[a] = malloc(ext * sizeof(double));
        A1[a] = malloc(ext * sizeof(double));
        A2[a] = malloc(ext * sizeof(double));
        A3[a] = malloc(ext * sizeof(double));
        O[a] = malloc((size_t)nr * d * sizeof(double));
        if (!S[a] || !A1[a] || !A2[a] || !A3[a] || !O[a]) { rc = -1; goto done; }
        /* rows a stage does not define stay NaN, so a stray read would show */
        for (size_t e = 0; e < ext; ++e) A1[a][e] = A2[a][e] = A3[a][e] = NAN;
    }

    /* Logits on the extended rows. */
    for (int a = 0; a < c_h; ++a) {
        const int h = g * c_h + a;
        const size_t base = ((size_t)b * H + h) * (size_t)T * d;
        step_logits(q + base, k + base, T, d, e0, r1, S[a]);
    }

    /* A1 <- the map that enters the softmax.
     *   kq PRE      : Conv2d(Mask_0(S)) on rows [r0, r1)
     *   kq PRE_EXACT: Conv2d with the indicator, on S itself, rows [r0, r1)
     *   kq POST     : S itself on rows [e0, r1) */
    for (int a = 0; a < c_h; ++a) {
        const int h = g * c_h + a;
        if (cf->kq_place == ORACLE_PRE) {
            memcpy(A2[a], S[a], ext * sizeof(double));
            step_mask_zero(A2[a], T, e0, r1);
            step_kq_conv(A2[a], T, e0, ne, theta_kq + (size_t)h * cf->c_q * cf->c_k,
                         cf->c_q, cf->c_k, 0, r0, r1, A1[a] + off);
        } else if (cf->kq_place == ORACLE_PRE_EXACT) {
            step_kq_conv(S[a], T, e0, ne, theta_kq + (size_t)h * cf->c_q * cf->c_k,
                         cf->c_q, cf->c_k, 1, r0, r1, A1[a] + off);
        } else {
            memcpy(A1[a], S[a], ext * sizeof(double));
        }
    }
    if (st)
        for (int a = 0; a < c_h; ++a) {
            memcpy(st->S + (size_t)a * T * T, S[a], ext * sizeof(double));
            memcpy(st->C + (size_t)a * T * T, A1[a], ext * sizeof(double));
        }

    /* Head mix before the softmax (the pre-softmax form of Eq. 7), rows [v0,r1). */
    if (cf->head_place == ORACLE_PRE) {
        for (int a = 0; a < c_h; ++a) { X[a] = A1[a] + voff; Y[a] = A2[a] + voff; }
        step_head_mix(X, theta_head + (size_t)g * c_h * c_h, c_h, nv, Y);
        for (int a = 0; a < c_h; ++a) memcpy(A1[a] + voff, A2[a] + voff, nv * sizeof(double));
    }
    if (st)
        for (int a = 0; a < c_h; ++a) memcpy(st->Cmix + (size_t)a * T * T, A1[a], ext * sizeof(double));

    /* Mask_-inf and softmax, rows [v0, r1). */
    for (int a = 0; a < c_h; ++a) step_causal_softmax(A1[a] + voff, T, v0, r1, A2[a] + voff);
    if (st)
        for (int a = 0; a < c_h; ++a) memcpy(st->P + (size_t)a * T * T, A2[a], ext * sizeof(double));

    /* kq conv after the softmax: Conv2d on the probabilities of rows [e0,r1),
     * output rows [r0, r1), then Mask_0. */
    if (cf->kq_place == ORACLE_POST) {
        for (int a = 0; a < c_h; ++a) {
            const int h = g * c_h + a;
            step_kq_conv(A2[a], T, e0, ne, theta_kq + (size_t)h * cf->c_q * cf->c_k,
                         cf->c_q, cf->c_k, 0, r0, r1, A3[a] + off);
            step_mask_zero(A3[a] + off, T, r0, r1);
            memcpy(A2[a] + off, A3[a] + off, (size_t)nr * T * sizeof(double));
        }
    }
    if (st)
        for (int a = 0; a < c_h; ++a) memcpy(st->P2 + (size_t)a * T * T, A2[a], ext * sizeof(double));

    /* Head mix after the softmax (Eq. 7), rows [r0, r1). */
    for (int a = 0; a < c_h; ++a) { X[a] = A2[a] + off; Y[a] = A3[a] + off; }
    if (cf->head_place == ORACLE_POST) {
        step_head_mix(X, theta_head + (size_t)g * c_h * c_h, c_h, (size_t)nr * T, Y);
    } else {
        for (int a = 0; a < c_h; ++a) memcpy(Y[a], X[a], (size_t)nr * T * sizeof(double));
    }
    if (st)
        for (int a = 0; a < c_h; ++a) memcpy(st->P3 + (size_t)a * T * T, A3[a], ext * sizeof(double));

    /* A V per head, then GroupNorm x depth scale, rows [r0, r1). */
    for (int a = 0; a < c_h; ++a) {
        const int h = g * c_h + a;
        const size_t base = ((size_t)b * H + h) * (size_t)T * d;
        step_pv(A3[a] + off, v + base, T, d, r0, r1, O[a]);
        step_groupnorm_scale(O[a], gn_w + (size_t)h * d, gn_b + (size_t)h * d, d, r0, r1,
                             cf->eps, head_scale(cf, h), out + base + (size_t)r0 * d);
        if (st) {
            memcpy(st->O + (size_t)a * T * d, O[a], (size_t)nr * d * sizeof(double));
            memcpy(st->Y + (size_t)a * T * d, out + base + (size_t)r0 * d,
                   (size_t)nr * d * sizeof(double));
        }
    }

done:
    for (int a = 0; a < c_h; ++a) {
        if (S) free(S[a]);
        if (A1) free(A1[a]);
        if (A2) free(A2[a]);
        if (A3) free(A3[a]);
        if (O) free(O[a]);
    }
    free(S); free(A1); free(A2); free(A3); free(O); free(X); free(Y);
    return rc;
}

static int check_cfg(const oracle_cfg *c)
{
    if (c->B < 0 || c->H <= 0 || c->T < 0 || c->d <= 0) return -2;
    if (c->c_q < 1 || c->c_k < 1 || c->c_h < 1 || c->H % c->c_h) return -2;
    if (c->kq_place < 0 || c->kq_place > 2 || (c->head_place != 0 && c->head_place != 1)) return -3;
    return 0;
}

/* Public entry 1: the forward over a set of (b, g) units and output rows
 * [row_begin, row_end) of each, split into row chunks of `chunk` rows that
 * run on `n_threads` threads (the arithmetic of an output row does not depend
 * on the chunking).  units == NULL means every unit b*G+g.  Arrays are
 * float64, [B][H][T][d] for q, k, v, out; theta_kq [H][c_q][c_k];
 * theta_head [H/c_h][c_h][c_h]; gn_w, gn_b [H][d]; gate [H] or NULL (each
 * head's output is scaled by depth_scale * sigmoid(gate[h]), or by
 * depth_scale alone without a gate).  Only the requested rows of
 * the requested units of `out` are written.  Returns 0, or a negative code. */
int mta_oracle_forward(const double *q, const double *k, const double *v,
                       const double *theta_kq, const double *theta_head,
                       const double *gn_w, const double *gn_b, const double *gate,
                       int B, int H, int T, int d, int c_q, int c_k, int c_h,
                       int kq_place, int head_place, double eps, double depth_scale,
                       int row_begin, int row_end, const int *units, int n_units,
                       int chunk, int n_threads, double *out)
{
    oracle_cfg cf = {B, H, T, d, c_q, c_k, c_h, kq_place, head_place, eps, depth_scale, gate};
    int rc = check_cfg(&cf);
    if (rc) return rc;
    if (row_begin < 0 || row_end > T || row_begin > row_end) return -2;
    const int G = H / c_h;
    const int nu = units ? n_units : B * G;
    if (chunk <= 0) chunk = row_end - row_begin;
    if (chunk <= 0) return 0;
    const int nchunks = (row_end - row_begin + chunk - 1) / chunk;
    const long ntasks = (long)nu * nchunks;
    int err = 0;
#ifdef _OPENMP
    if (n_threads < 1) n_threads = 1;
#pragma omp parallel for schedule(dynamic, 1) num_threads(n_threads) reduction(| : err)
#endif
    for (long t = 0; t < ntasks; ++t) {
        const int u = units ? units[t / nchunks] : (int)(t / nchunks);
        const int ck = (int)(t % nchunks);
        const int b = u / G, g = u % G;
        if (b < 0 || b >= B) { err |= 1; continue; }
        const int r0 = row_begin + ck * chunk;
        const int r1 = (r0 + chunk < row_end) ? r0 + chunk : row_end;
        if (unit_rows(&cf, q, k, v, theta_kq, theta_head, gn_w, gn_b, b, g, r0, r1, out, NULL))
            err |= 1;
    }
    return err ? -1 : 0;
}

/* Public entry 2: every stage of one unit (b, g) over all T rows (tests).
 * S, C, Cmix, P, P2, P3: [c_h][T][T]; O, Y: [c_h][T][d].  `out` receives the
 * unit's heads of the final result in [B][H][T][d] layout. */
int mta_oracle_stages(const double *q, const double *k, const double *v,
                      const double *theta_kq, const double *theta_head,
                      const double *gn_w, const double *gn_b, const double *gate,
                      int B, int H, int T, int d, int c_q, int c_k, int c_h,
                      int kq_place, int head_place, double eps, double depth_scale,
                      int b, int g, double *S, double *C, double *Cmix, double *P,
                      double *P2, double *P3, double *O, double *Y, double *out)
{
    oracle_cfg cf = {B, H, T, d, c_q, c_k, c_h, kq_place, head_place, eps, depth_scale, gate};
    int rc = check_cfg(&cf);
    if (rc) return rc;
    if (b < 0 || b >= B || g < 0 || g >= H / c_h) return -2;
    oracle_stages st = {S, C, Cmix, P, P2, P3, O, Y};
    return unit_rows(&cf, q, k, v, theta_kq, theta_head, gn_w, gn_b, b, g, 0, T, out, &st);
}

/* ======================================================================== */
/* The general MTA layer ("Putting Everything Together": the key-query and the
 * head convolution on either side of the softmax, the both-pre-softmax "3D
 * convolution view", and the repeated MTA convolution after the softmax of
 * the overall flow).  Every stage is optional:
 *
 *   L   = S,  or  Conv2d_theta1(Mask_0(S))  (two-pass; or Eq. 4's indicator on
 *         S when `exact`),  or the 3D convolution  sum_b Conv2d_theta3[a][b](.)
 *   L   = head mix w_pre (L)                       (not with the 3D kernel)
 *   P   = softmax(Mask_-inf(L))
 *   P   = head mix w_post (P)                      (Eq. 7)
 *   P   = Mask_0(Conv2d_theta2(P))                  (kq conv after the softmax)
 *   P   = head mix w_post2 (P)                     (the repeated head conv)
 *   O   = P V,  GroupNorm x scale.
 * ------------------------------------------------------------------------ */

typedef struct {
    const double *kq_pre;     /* [H][c_q][c_k] or NULL                                 */
    const double *head_pre;   /* [G][c_h][c_h] or NULL                                 */
    const double *conv3d;     /* [G][c_h][c_h][c_q][c_k] or NULL (instead of the two)  */
    const double *head_post;  /* [G][c_h][c_h] or NULL                                 */
    const double *kq_post;    /* [H][c_q2][c_k2] or NULL                               */
    const double *head_post2; /* [G][c_h][c_h] or NULL                                 */
    int exact;                /* pre-softmax convolution with Eq. 4's indicator        */
    int c_q2, c_k2;
} layer_w;

/* Step 3b.  The 3D convolution over (query, key, head) of one group
 * ("Putting Everything Together", both pre-softmax): output head a sums the
 * key-query convolutions of every source head b of the group, each with its
 * own c_q x c_k kernel theta3[a][b]:
 *   Y^a[i][j] = sum_b sum_{i',j'} theta3[a][b][i'][j'] X^b[i-i'][j-j'].
 * Each (a, b) term is step 3 (with the same indicator choice). */
static void step_conv3d(double *const *X, int T, int x0, int nx, const double *th3, int c_h,
                        int c_q, int c_k, int indicator, int i0, int i1, double *const *Y,
                        double *tmp)
{
    const size_t n = (size_t)(i1 - i0) * T;
    for (int a = 0; a < c_h; ++a) {
        for (size_t e = 0; e < n; ++e) Y[a][e] = 0.0;
        for (int b = 0; b < c_h; ++b) {
#if ORACLE_MUTANT == 10 /* planted: output and source head swapped in the 3D kernel */
            const double *th = th3 + ((size_t)b * c_h + a) * c_q * c_k;
#else
            const double *th = th3 + ((size_t)a * c_h + b) * c_q * c_k;
#endif
            step_kq_conv(X[b], T, x0, nx, th, c_q, c_k, indicator, i0, i1, tmp);
            for (size_t e = 0; e < n; ++e) Y[a][e] += tmp[e];
        }
    }
}

/* Stage dump layout of the layer for one unit, full rows [0,T) only:
 *   S, Lc, L, P, Pa, P2, P3 : [c_h][T][T]   (Lc: after the pre-softmax
 *     convolution, L: entering the softmax, Pa: after w_post, P2: after the
 *     post-softmax key-query convolution and Mask_0, P3: after w_post2)
 *   O, Y                    : [c_h][T][d]                                     */
typedef struct {
    double *S, *Lc, *L, *P, *Pa, *P2, *P3, *O, *Y;
} layer_stages;

static int layer_rows(const oracle_cfg *cf, const layer_w *lw, const double *q, const double *k,
                      const double *v, const double *gn_w, const double *gn_b, int b, int g,
                      int r0, int r1, double *out, const layer_stages *st)
{
    const int T = cf->T, d = cf->d, c_h = cf->c_h, H = cf->H;
    const int has_pre = lw->kq_pre || lw->conv3d;
    /* rows of the probabilities the post-softmax convolution reads, and rows of
     * the logits the pre-softmax convolution reads from those */
    const int e2 = lw->kq_post ? ((r0 - (lw->c_q2 - 1)) > 0 ? r0 - (lw->c_q2 - 1) : 0) : r0;
    const int e1 = has_pre ? ((e2 - (cf->c_q - 1)) > 0 ? e2 - (cf->c_q - 1) : 0) : e2;
    const int ne = r1 - e1, nr = r1 - r0;
    const size_t ext = (size_t)ne * T;
    const size_t off2 = (size_t)(e2 - e1) * T;   /* row e2 in an extended buffer */
    const size_t off = (size_t)(r0 - e1) * T;    /* row r0 */
    const size_t n2 = (size_t)(r1 - e2) * T;
    const int G = H / c_h;
    int rc = 0;
    (void)G;

    double **S = calloc(c_h, sizeof(double *)), **A = calloc(c_h, sizeof(double *));
    double **B2 = calloc(c_h, sizeof(double *)), **O = calloc(c_h, sizeof(double *));
    double **X = calloc(c_h, sizeof(double *)), **Y = calloc(c_h, sizeof(double *));
    double *tmp = malloc(ext * sizeof(double));
    if (!S || !A || !B2 || !O || !X || !Y || !tmp) { rc = -1; goto done; }
    for (int a = 0; a < c_h; ++a) {
        S[a] = malloc(ext * sizeof(double));
        A[a] = malloc(ext * sizeof(double));
        B2[a] = malloc(ext * sizeof(double));
        O[a] = malloc((size_t)nr * d * sizeof(double));
        if (!S[a] || !A[a] || !B2[a] || !O[a]) { rc = -1; goto done; }
        for (size_t e = 0; e < ext; ++e) A[a][e] = B2[a][e] = NAN;
    }
#define DUMP(field, buf)                                                               \
    if (st && st->field)                                                               \
        for (int a_ = 0; a_ < c_h; ++a_)                                               \
            memcpy(st->field + (size_t)a_ * T * T, (buf)[a_], ext * sizeof(double));

    for (int a = 0; a < c_h; ++a) {
        const size_t base = ((size_t)b * H + g * c_h + a) * (size_t)T * d;
        step_logits(q + base, k + base, T, d, e1, r1, S[a]);
    }
    DUMP(S, S)

    /* A <- the pre-softmax convolution on rows [e2, r1) */
    if (has_pre) {
        for (int a = 0; a < c_h; ++a) {
            memcpy(B2[a], S[a], ext * sizeof(double));
            if (!lw->exact) step_mask_zero(B2[a], T, e1, r1);
        }
        if (lw->conv3d) {
            for (int a = 0; a < c_h; ++a) Y[a] = A[a] + off2;
            step_conv3d(B2, T, e1, ne, lw->conv3d + (size_t)g * c_h * c_h * cf->c_q * cf->c_k, c_h,
                        cf->c_q, cf->c_k, lw->exact, e2, r1, Y, tmp);
        } else {
            for (int a = 0; a < c_h; ++a)
                step_kq_conv(B2[a], T, e1, ne, lw->kq_pre + (size_t)(g * c_h + a) * cf->c_q * cf->c_k,
                             cf->c_q, cf->c_k, lw->exact, e2, r1, A[a] + off2);
        }
    } else {
        for (int a = 0; a < c_h; ++a) memcpy(A[a] + off2, S[a] + off2, n2 * sizeof(double));
    }
    DUMP(Lc, A)
    if (lw->head_pre && !lw->conv3d) {
        for (int a = 0; a < c_h; ++a) { X[a] = A[a] + off2; Y[a] = B2[a] + off2; }
        step_head_mix(X, lw->head_pre + (size_t)g * c_h * c_h, c_h, n2, Y);
        for (int a = 0; a < c_h; ++a) memcpy(A[a] + off2, B2[a] + off2, n2 * sizeof(double));
    }
    DUMP(L, A)

    /* softmax on rows [e2, r1) */
    for (int a = 0; a < c_h; ++a) {
        step_causal_softmax(A[a] + off2, T, e2, r1, B2[a] + off2);
        memcpy(A[a] + off2, B2[a] + off2, n2 * sizeof(double));
    }
    DUMP(P, A)
    if (lw->head_post) {
        for (int a = 0; a < c_h; ++a) { X[a] = A[a] + off2; Y[a] = B2[a] + off2; }
        step_head_mix(X, lw->head_post + (size_t)g * c_h * c_h, c_h, n2, Y);
        for (int a = 0; a < c_h; ++a) memcpy(A[a] + off2, B2[a] + off2, n2 * sizeof(double));
    }
    DUMP(Pa, A)
    if (lw->kq_post) {
        for (int a = 0; a < c_h; ++a) {
            step_kq_conv(A[a] + off2, T, e2, r1 - e2,
                         lw->kq_post + (size_t)(g * c_h + a) * lw->c_q2 * lw->c_k2, lw->c_q2, lw->c_k2, 0,
                         r0, r1, B2[a] + off);
#if ORACLE_MUTANT != 11 /* planted (11): the Mask_0 after the post-softmax convolution dropped */
            step_mask_zero(B2[a] + off, T, r0, r1);
#endif
        }
        for (int a = 0; a < c_h; ++a) memcpy(A[a] + off, B2[a] + off, (size_t)nr * T * sizeof(double));
    }
    DUMP(P2, A)
    if (lw->head_post2) {
        for (int a = 0; a < c_h; ++a) { X[a] = A[a] + off; Y[a] = B2[a] + off; }
        step_head_mix(X, lw->head_post2 + (size_t)g * c_h * c_h, c_h, (size_t)nr * T, Y);
        for (int a = 0; a < c_h; ++a) memcpy(A[a] + off, B2[a] + off, (size_t)nr * T * sizeof(double));
    }
    DUMP(P3, A)
#undef DUMP

    for (int a = 0; a < c_h; ++a) {
        const int h = g * c_h + a;
        const size_t base = ((size_t)b * H + h) * (size_t)T * d;
        step_pv(A[a] + off, v + base, T, d, r0, r1, O[a]);
        step_groupnorm_scale(O[a], gn_w + (size_t)h * d, gn_b + (size_t)h * d, d, r0, r1, cf->eps,
                             head_scale(cf, h), out + base + (size_t)r0 * d);
        if (st) {
            if (st->O) memcpy(st->O + (size_t)a * T * d, O[a], (size_t)nr * d * sizeof(double));
            if (st->Y)
                memcpy(st->Y + (size_t)a * T * d, out + base + (size_t)r0 * d, (size_t)nr * d * sizeof(double));
        }
    }

done:
    for (int a = 0; a < c_h; ++a) {
        if (S) free(S[a]);
        if (A) free(A[a]);
        if (B2) free(B2[a]);
        if (O) free(O[a]);
    }
    free(S); free(A); free(B2); free(O); free(X); free(Y); free(tmp);
    return rc;
}

static int check_layer(const oracle_cfg *c, const layer_w *lw)
{
    if (c->B < 0 || c->H <= 0 || c->T < 0 || c->d <= 0) return -2;
    if (c->c_q < 1 || c->c_k < 1 || c->c_h < 1 || c->H % c->c_h) return -2;
    if (lw->conv3d && (lw->kq_pre || lw->head_pre)) return -3;
    if (lw->kq_post && (lw->c_q2 < 1 || lw->c_k2 < 1)) return -2;
    return 0;
}

/* Public entry 3: the general layer over a set of (b, g) units and output rows
 * [row_begin, row_end), as mta_oracle_forward.  Every kernel pointer may be
 * NULL (stage absent); conv3d excludes kq_pre and head_pre.  Shapes:
 * kq_pre [H][c_q][c_k]; head_pre, head_post, head_post2 [H/c_h][c_h][c_h];
 * conv3d [H/c_h][c_h][c_h][c_q][c_k]; kq_post [H][c_q2][c_k2]. */
int mta_oracle_layer(const double *q, const double *k, const double *v, const double *kq_pre,
                     const double *head_pre, const double *conv3d, const double *head_post,
                     const double *kq_post, const double *head_post2, const double *gn_w,
                     const double *gn_b, const double *gate, int B, int H, int T, int d, int c_q,
                     int c_k, int c_q2, int c_k2, int c_h, int exact, double eps, double depth_scale,
                     int row_begin, int row_end, const int *units, int n_units, int chunk,
                     int n_threads, double *out)
{
    oracle_cfg cf = {B, H, T, d, c_q, c_k, c_h, 0, 1, eps, depth_scale, gate};
    layer_w lw = {kq_pre, head_pre, conv3d, head_post, kq_post, head_post2, exact, c_q2, c_k2};
    int rc = check_layer(&cf, &lw);
    if (rc) return rc;
    if (row_begin < 0 || row_end > T || row_begin > row_end) return -2;
    const int G = H / c_h;
    const int nu = units ? n_units : B * G;
    if (chunk <= 0) chunk = row_end - row_begin;
    if (chunk <= 0) return 0;
    const int nchunks = (row_end - row_begin + chunk - 1) / chunk;
    const long ntasks = (long)nu * nchunks;
    int err = 0;
#ifdef _OPENMP
    if (n_threads < 1) n_threads = 1;
#pragma omp parallel for schedule(dynamic, 1) num_threads(n_threads) reduction(| : err)
#endif
    for (long t = 0; t < ntasks; ++t) {
        const int u = units ? units[t / nchunks] : (int)(t / nchunks);
        const int ck = (int)(t % nchunks);
        const int b = u / G, g = u % G;
        if (b < 0 || b >= B) { err |= 1; continue; }
        const int r0 = row_begin + ck * chunk;
        const int r1 = (r0 + chunk < row_end) ? r0 + chunk : row_end;
        if (layer_rows(&cf, &lw, q, k, v, gn_w, gn_b, b, g, r0, r1, out, NULL)) err |= 1;
    }
    return err ? -1 : 0;
}

/* Public entry 4: every stage of the layer for one unit (b, g), all T rows
 * (tests); any dump pointer may be NULL. */
int mta_oracle_layer_stages(const double *q, const double *k, const double *v, const double *kq_pre,
                            const double *head_pre, const double *conv3d, const double *head_post,
                            const double *kq_post, const double *head_post2, const double *gn_w,
                            const double *gn_b, const double *gate, int B, int H, int T, int d,
                            int c_q, int c_k, int c_q2, int c_k2, int c_h, int exact, double eps,
                            double depth_scale, int b, int g, double *S, double *Lc, double *L,
                            double *P, double *Pa, double *P2, double *P3, double *O, double *Y,
                            double *out)
{
    oracle_cfg cf = {B, H, T, d, c_q, c_k, c_h, 0, 1, eps, depth_scale, gate};
    layer_w lw = {kq_pre, head_pre, conv3d, head_post, kq_post, head_post2, exact, c_q2, c_k2};
    int rc = check_layer(&cf, &lw);
    if (rc) return rc;
    if (b < 0 || b >= B || g < 0 || g >= H / c_h) return -2;
    layer_stages st = {S, Lc, L, P, Pa, P2, P3, O, Y};
    return layer_rows(&cf, &lw, q, k, v, gn_w, gn_b, b, g, 0, T, out, &st);
}

int mta_oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
