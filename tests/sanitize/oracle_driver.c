/* Drives the float64 oracle through every placement, the general layer and the
 * stage dumps on small inputs, for an AddressSanitizer / UBSan build of
 * oracle/mta_oracle.c (tests/test_sanitize.py).  Exit status 0 when every call
 * returns 0 and every output is finite. */
#include <math.h>
#include <stdio.h>
#include <stdlib.h>

int mta_oracle_forward(const double *, const double *, const double *, const double *, const double *,
                       const double *, const double *, const double *, int, int, int, int, int, int, int, int,
                       int, double, double, int, int, const int *, int, int, int, double *);
int mta_oracle_stages(const double *, const double *, const double *, const double *, const double *,
                      const double *, const double *, const double *, int, int, int, int, int, int, int, int,
                      int, double, double, int, int, double *, double *, double *, double *, double *,
                      double *, double *, double *, double *);
int mta_oracle_layer(const double *, const double *, const double *, const double *, const double *,
                     const double *, const double *, const double *, const double *, const double *,
                     const double *, const double *, int, int, int, int, int, int, int, int, int, int, double,
                     double, int, int, const int *, int, int, int, double *);

static double *rnd(size_t n, unsigned *s)
{
    double *x = malloc(n * sizeof(double));
    for (size_t i = 0; i < n; ++i) {
        *s = *s * 1664525u + 1013904223u;
        x[i] = ((double)(*s >> 8) / 16777216.0 - 0.5) * 2.0;
    }
    return x;
}

static int finite_all(const double *x, size_t n)
{
    for (size_t i = 0; i < n; ++i)
        if (!isfinite(x[i])) return 0;
    return 1;
}

int main(void)
{
    unsigned s = 12345u;
    const int B = 2, H = 4, T = 19, d = 8;
    const size_t n = (size_t)B * H * T * d;
    double *q = rnd(n, &s), *k = rnd(n, &s), *v = rnd(n, &s), *out = calloc(n, sizeof(double));
    double *gw = rnd((size_t)H * d, &s), *gb = rnd((size_t)H * d, &s), *gate = rnd(H, &s);
    int bad = 0;
    const int sizes[][2] = {{3, 5}, {2, 4}, {1, 1}, {5, 7}};
    for (int sz = 0; sz < 4; ++sz) {
        const int cq = sizes[sz][0], ck = sizes[sz][1];
        double *th = rnd((size_t)H * cq * ck, &s);
        for (int ch = 1; ch <= 4; ch *= 2) {
            double *w = rnd((size_t)H * ch, &s);
            for (int kq = 0; kq <= 2; ++kq)
                for (int hp = 0; hp <= 1; ++hp) {
                    if (kq == 2 && hp == 1 && ch == 4) continue;
                    const int rc = mta_oracle_forward(q, k, v, th, w, gw, gb, (sz & 1) ? gate : NULL, B, H, T, d,
                                                      cq, ck, ch, kq, hp, 1e-5, 0.5, 0, T, NULL, 0, 7, 2, out);
                    if (rc != 0 || !finite_all(out, n)) {
                        fprintf(stderr, "forward cq%d ck%d ch%d kq%d hp%d rc %d\n", cq, ck, ch, kq, hp, rc);
                        bad = 1;
                    }
                }
            const size_t tt = (size_t)ch * T * T, td = (size_t)ch * T * d;
            double *S = malloc(tt * 8), *C = malloc(tt * 8), *Cm = malloc(tt * 8), *P = malloc(tt * 8);
            double *P2 = malloc(tt * 8), *P3 = malloc(tt * 8), *O = malloc(td * 8), *Y = malloc(td * 8);
            if (mta_oracle_stages(q, k, v, th, w, gw, gb, NULL, B, H, T, d, cq, ck, ch, 1, 1, 1e-5, 1.0, 1,
                                  H / ch - 1, S, C, Cm, P, P2, P3, O, Y, out) != 0) {
                fprintf(stderr, "stages cq%d ck%d ch%d\n", cq, ck, ch);
                bad = 1;
            }
            double *th3 = rnd((size_t)H * ch * cq * ck, &s), *w2 = rnd((size_t)H * ch, &s);
            double *th2 = rnd((size_t)H * 2 * 3, &s);
            if (mta_oracle_layer(q, k, v, NULL, NULL, th3, w, th2, w2, gw, gb, gate, B, H, T, d, cq, ck, 2, 3, ch,
                                 sz & 1, 1e-5, 0.7, 0, T, NULL, 0, 5, 2, out) != 0 ||
                !finite_all(out, n)) {
                fprintf(stderr, "layer cq%d ck%d ch%d\n", cq, ck, ch);
                bad = 1;
            }
            free(S); free(C); free(Cm); free(P); free(P2); free(P3); free(O); free(Y);
            free(th3); free(w2); free(th2); free(w);
        }
        free(th);
    }
    free(q); free(k); free(v); free(out); free(gw); free(gb); free(gate);
    if (!bad) printf("oracle driver: ok\n");
    return bad;
}
