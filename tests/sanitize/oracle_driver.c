/* Drives every oracle function on small inputs (empty and one-token
 * sequences, NULL and given states and windows, one and several threads)
 * so that an AddressSanitizer / UndefinedBehaviorSanitizer build of the
 * oracle can check its memory accesses and arithmetic.  Values are pinned
 * elsewhere; here only the absence of sanitizer reports and finite outputs
 * are checked.  Exit status 0 on success. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

void gdn_oracle_conv1d_f64(int n_seq, const int32_t *cu, int C, int W, const double *x, const double *w,
                           const double *bias, const double *win_in, int silu, double *y, double *win_out);
void gdn_oracle_conv1d_f32(int n_seq, const int32_t *cu, int C, int W, const float *x, const float *w,
                           const float *bias, const float *win_in, int silu, float *y, int out_bf16,
                           uint16_t *y_bits);
float gdn_oracle_exp_f32(float x);
int gdn_oracle_scan(int n_seq, const int32_t *cu, int Hk, int Hv, int dk, int dv, double scale, unsigned flags,
                    const double *q, const double *k, const double *v, const double *g, const double *beta,
                    const double *state_in, double *o, double *state_out, int n_threads);
void gdn_oracle_gated_rmsnorm(long rows, int d, const double *o, const double *z, const double *w, double eps,
                              double *y);
void gdn_oracle_gating(long n_tok, int H, const double *a, const double *b, const double *A_log,
                       const double *dt_bias, double *g, double *beta);
int gdn_oracle_available_cores(void);

static uint64_t st = 0x9e3779b97f4a7c15ull;
static double rnd(void) {  /* splitmix64 -> [-1, 1) */
    uint64_t z = (st += 0x9e3779b97f4a7c15ull);
    z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
    z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
    z ^= z >> 31;
    return (double)(z >> 11) / 4503599627370496.0 - 1.0;
}
static double *arr(long n) {
    double *p = malloc(sizeof(double) * (n ? n : 1));
    for (long i = 0; i < n; i++) p[i] = rnd();
    return p;
}
static int finite_all(const double *p, long n) {
    for (long i = 0; i < n; i++)
        if (!isfinite(p[i])) return 0;
    return 1;
}

int main(void) {
    int bad = 0;
    /* ragged varlen: empty, one token, partial windows */
    const int32_t cu[] = {0, 0, 1, 4, 4, 11};
    const int n_seq = 5, T = 11, C = 16, W = 4;
    double *x = arr((long)T * C), *w = arr((long)C * W), *b = arr(C), *win = arr((long)n_seq * (W - 1) * C);
    double *y = malloc(sizeof(double) * T * C), *wo = malloc(sizeof(double) * n_seq * (W - 1) * C);
    gdn_oracle_conv1d_f64(n_seq, cu, C, W, x, w, NULL, NULL, 1, y, wo);
    gdn_oracle_conv1d_f64(n_seq, cu, C, W, x, w, b, win, 0, y, wo);
    bad |= !finite_all(y, (long)T * C) || !finite_all(wo, (long)n_seq * (W - 1) * C);
    float *xf = malloc(sizeof(float) * T * C), *wf = malloc(sizeof(float) * C * W), *bf = malloc(sizeof(float) * C);
    float *winf = malloc(sizeof(float) * n_seq * (W - 1) * C), *yf = malloc(sizeof(float) * T * C);
    uint16_t *yb = malloc(sizeof(uint16_t) * T * C);
    for (long i = 0; i < (long)T * C; i++) xf[i] = (float)x[i];
    for (long i = 0; i < (long)C * W; i++) wf[i] = (float)w[i];
    for (long i = 0; i < C; i++) bf[i] = (float)b[i];
    for (long i = 0; i < (long)n_seq * (W - 1) * C; i++) winf[i] = (float)win[i];
    gdn_oracle_conv1d_f32(n_seq, cu, C, W, xf, wf, bf, winf, 1, yf, 0, NULL);
    gdn_oracle_conv1d_f32(n_seq, cu, C, W, xf, wf, NULL, NULL, 1, NULL, 1, yb);
    const float specials[] = {0.0f, -0.0f, 1e-40f, -1e-40f, 88.4f, 88.6f, -85.9f, -86.1f, INFINITY, -INFINITY, NAN};
    for (unsigned i = 0; i < sizeof(specials) / sizeof(specials[0]); i++) (void)gdn_oracle_exp_f32(specials[i]);
    /* scan: grouped heads, d_k != d_v, NULL and given states, 1 and 3 threads */
    const int Hk = 2, Hv = 4, dk = 8, dv = 4;
    double *q = arr((long)T * Hk * dk), *k = arr((long)T * Hk * dk), *v = arr((long)T * Hv * dv);
    double *g = malloc(sizeof(double) * T * Hv), *beta = malloc(sizeof(double) * T * Hv);
    for (long i = 0; i < (long)T * Hv; i++) {
        g[i] = -0.5 * fabs(rnd());
        beta[i] = 0.5 + 0.5 * rnd();
    }
    double *s0 = arr((long)n_seq * Hv * dk * dv);
    double *o = malloc(sizeof(double) * T * Hv * dv), *s1 = malloc(sizeof(double) * n_seq * Hv * dk * dv);
    for (unsigned flags = 0; flags < 4; flags++)
        for (int nt = 1; nt <= 3; nt += 2) {
            if (gdn_oracle_scan(n_seq, cu, Hk, Hv, dk, dv, 0.5, flags, q, k, v, g, beta, flags & 1 ? s0 : NULL,
                                o, s1, nt) < 0)
                bad = 1;
            bad |= !finite_all(o, (long)T * Hv * dv) || !finite_all(s1, (long)n_seq * Hv * dk * dv);
        }
    /* in place: state_out = state_in */
    if (gdn_oracle_scan(n_seq, cu, Hk, Hv, dk, dv, 1.0, 1u, q, k, v, g, beta, s0, o, s0, 2) < 0) bad = 1;
    if (gdn_oracle_scan(n_seq, cu, 3, Hv, dk, dv, 1.0, 0u, q, k, v, g, beta, NULL, o, s1, 1) != -1) bad = 1;
    /* gated norm (with an all-zero row) and gating */
    double *z = arr(6 * dv), *wn = arr(dv), *yn = malloc(sizeof(double) * 6 * dv), *o6 = arr(6 * dv);
    for (int j = 0; j < dv; j++) o6[j] = 0.0;
    gdn_oracle_gated_rmsnorm(6, dv, o6, z, wn, 1e-6, yn);
    gdn_oracle_gated_rmsnorm(0, dv, o6, z, wn, 1e-6, yn);
    bad |= !finite_all(yn, 6 * dv);
    double *ga = arr(T * Hv), *gb = arr(T * Hv), *al = arr(Hv), *db = arr(Hv);
    ga[0] = 80.0;
    ga[1] = -80.0;
    gdn_oracle_gating(T, Hv, ga, gb, al, db, g, beta);
    bad |= !finite_all(g, (long)T * Hv) || !finite_all(beta, (long)T * Hv);
    bad |= gdn_oracle_available_cores() < 1;
    free(x); free(w); free(b); free(win); free(y); free(wo); free(xf); free(wf); free(bf); free(winf); free(yf);
    free(yb); free(q); free(k); free(v); free(g); free(beta); free(s0); free(o); free(s1); free(z); free(wn);
    free(yn); free(o6); free(ga); free(gb); free(al); free(db);
    printf(bad ? "oracle driver: FAILED\n" : "oracle driver: ok\n");
    return bad;
}
