/*
 * gdn_oracle.c -- plain CPU checker for the Gated DeltaNet layer core.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file: only the tests, the smoke check and the CPU-baseline leg
 * of the benchmark use it.  It shares no code with the GPU library.
 *
 * What it computes (every function in fp64 unless its name says f32):
 *
 *  - gdn_oracle_conv1d_f64: the short causal depthwise convolution that
 *    feeds the layer, optionally followed by SiLU (Vallmo.jl README, "What's
 *    here": causal conv1d is one of the hybrid layer's kernels; oxydllm
 *    0.0.0-alpha.12.2 release notes, "New Features": per-sequence state is a
 *    causal-conv window plus the recurrent memory).  Tap W-1 multiplies the
 *    current token; taps 0..W-2 reach back in time; left context comes from
 *    the per-sequence conv window, or zeros.
 *
 *  - gdn_oracle_conv1d_f32: the same convolution evaluated in IEEE fp32 in
 *    one fixed order (acc = bias or 0; acc = fma(w_j, x_j, acc) for j =
 *    0..W-1; y = acc / (1 + E(-acc)), with E the exponential below).  The
 *    convolution must come out bit-exact, so its evaluation order is part of
 *    its definition; this function is that definition.  It is pinned to the
 *    fp64 function above by the tests.
 *
 *  - gdn_oracle_exp_f32: E(x), an fp32 exponential written from the
 *    published Cody & Waite method (Cody and Waite, "Software Manual for the
 *    Elementary Functions", 1980): x = n*ln2 + r with n = rint(x/ln2),
 *    r = (x - n*C1) - n*C2 where C1 + C2 = ln2 and C1 has few enough bits
 *    that n*C1 is exact; e^r from its Taylor series through r^7 (Horner,
 *    fused multiply-adds), then scaled by 2^n.  Constants are derived here,
 *    not copied: C1 = ln2 rounded to 16 significant bits, C2 = fp32(ln2 -
 *    C1), Taylor coefficients fp32(1/k!).
 *
 *  - gdn_oracle_scan: the gated delta rule, token by token.  Per sequence
 *    and v-head, with the state S stored [d_k][d_v]:
 *        S <- alpha_t S                     (alpha_t = exp(g_t))
 *        u  = beta_t (v_t - S^T k_t)
 *        S <- S + k_t u^T
 *        o_t = S^T q_t
 *    which is S_t = alpha_t (I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T,
 *    o_t = S_t^T q_t: the delta rule with a scalar forget gate, the layer the
 *    oxydllm notes ("New Features", Gated DeltaNet runtime) run as a chunked
 *    scan for prefill and as an O(1) recurrent step for decode, with a
 *    32x128x128 fp32 memory per sequence.  Optionally q and k are first L2
 *    normalised (x / sqrt(|x|^2 + 1e-6)), and q is multiplied by `scale`.
 *    v-head h reads q/k head h / (H_v/H_k) (grouped, repeat-interleave) or,
 *    with the tiled flag, h % H_k (the GGUF ordering the oxydllm notes
 *    describe under "GGUF qwen35 architecture").
 *
 * The decode step is this scan with one token per sequence.
 *
 *  - gdn_oracle_gated_rmsnorm: the gated RMS norm applied to the layer's
 *    output before the output projection (the oxydllm notes, "Performance":
 *    the Gated DeltaNet's gated norm runs as one fused kernel over the token
 *    batch; "New Features", GGUF qwen35: this norm, unlike the model's other
 *    norms, uses its weight as stored, with no plus-one).  Per (token,
 *    v-head) row of d_v values, with gate z and weight w[d_v] shared by all
 *    heads:
 *        y_j = w_j * o_j / sqrt(mean_i o_i^2 + eps) * silu(z_j),
 *    silu(a) = a / (1 + e^-a): normalise first, then gate.
 *
 *  - gdn_oracle_gating: the per-token gates from the layer's small raw
 *    projections (the oxydllm notes, "Performance": the beta and decay
 *    projections; "New Features", GGUF qwen35: the per-head decay rate is
 *    stored as the negated exponential of A_log).  Per token t and v-head h:
 *        g    = -exp(A_log[h]) * softplus(a[t][h] + dt_bias[h])
 *        beta = 1 / (1 + exp(-b[t][h]))
 *    softplus(x) = log(1 + e^x), evaluated as max(x, 0) + log1p(e^-|x|).
 *
 * Build: gcc -O2 -std=c11 -ffp-contract=off -fPIC -shared -pthread -lm.
 * -ffp-contract=off matters: the fp32 convolution must not gain or lose
 * fused multiply-adds behind the source's back.
 */
#define _GNU_SOURCE
#include <math.h>
#include <pthread.h>
#include <sched.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define GDN_ORACLE_L2NORM 1u
#define GDN_ORACLE_TILED 2u
#define GDN_ORACLE_L2_EPS 1e-6

/* ------------------------------------------------------------------ conv */

static double silu_f64(double a) { return a / (1.0 + exp(-a)); }

/* x: [n_tok][C], w: [C][W], bias: [C] or NULL, win_in: [n_seq][W-1][C] or NULL
 * (zeros), cu: [n_seq+1] token offsets.  y: [n_tok][C].  win_out:
 * [n_seq][W-1][C] or NULL: the last W-1 raw inputs of (window ++ sequence). */
void gdn_oracle_conv1d_f64(int n_seq, const int32_t *cu, int C, int W,
                           const double *x, const double *w, const double *bias,
                           const double *win_in, int silu, double *y, double *win_out)
{
    int Wm1 = W - 1;
    for (int s = 0; s < n_seq; s++) {
        long t0 = cu[s], t1 = cu[s + 1], len = t1 - t0;
        for (long t = 0; t < len; t++) {
            for (int c = 0; c < C; c++) {
                double acc = bias ? bias[c] : 0.0;
                for (int j = 0; j < W; j++) {
                    long src = t - Wm1 + j; /* position in the sequence */
                    double xv;
                    if (src >= 0)
                        xv = x[(t0 + src) * C + c];
                    else /* window slot Wm1 + src holds position src (src = -1 is the newest) */
                        xv = win_in ? win_in[((long)s * Wm1 + (Wm1 + src)) * C + c] : 0.0;
                    acc += w[c * W + j] * xv;
                }
                y[(t0 + t) * C + c] = silu ? silu_f64(acc) : acc;
            }
        }
        if (win_out) {
            for (int i = 0; i < Wm1; i++) {
                long src = len - Wm1 + i;
                for (int c = 0; c < C; c++) {
                    double xv;
                    if (src >= 0)
                        xv = x[(t0 + src) * C + c];
                    else
                        xv = win_in ? win_in[((long)s * Wm1 + (Wm1 + src)) * C + c] : 0.0;
                    win_out[((long)s * Wm1 + i) * C + c] = xv;
                }
            }
        }
    }
}

/* ---- fp32 exponential (Cody & Waite reduction + Taylor polynomial) ---- */

float gdn_oracle_exp_f32(float x)
{
    if (x != x) return x;
    if (x > 88.5f) return INFINITY;
    if (x < -86.0f) return 0.0f; /* keeps every result a normal number */
    const double ln2 = 0.69314718055994530942;
    /* C1: ln2 with its significand cut to 16 bits, so n*C1 is exact for |n| < 256 */
    const float c1 = (float)(ldexp(floor(ldexp(ln2, 16)), -16));
    const float c2 = (float)(ln2 - (double)c1);
    const float inv_ln2 = (float)(1.0 / ln2);
    float n = rintf(x * inv_ln2);
    float r = fmaf(-n, c1, x);
    r = fmaf(-n, c2, r);
    float p = (float)(1.0 / 5040.0);          /* 1/7! */
    p = fmaf(p, r, (float)(1.0 / 720.0));     /* 1/6! */
    p = fmaf(p, r, (float)(1.0 / 120.0));     /* 1/5! */
    p = fmaf(p, r, (float)(1.0 / 24.0));      /* 1/4! */
    p = fmaf(p, r, (float)(1.0 / 6.0));       /* 1/3! */
    p = fmaf(p, r, 0.5f);                     /* 1/2! */
    p = fmaf(p, r, 1.0f);                     /* 1/1! */
    p = fmaf(p, r, 1.0f);                     /* 1/0! */
    return ldexpf(p, (int)n);
}

static float silu_f32(float a) { return a / (1.0f + gdn_oracle_exp_f32(-a)); }

static uint16_t f32_to_bf16_rne(float f)
{
    uint32_t u;
    memcpy(&u, &f, 4);
    if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu)) return 0x7fc0;
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

/* Same arguments as the f64 version, but fp32 values; when out_bf16 != 0
 * the outputs are written as bf16 bit patterns (uint16, round to nearest
 * even) into y_bits instead of y. */
void gdn_oracle_conv1d_f32(int n_seq, const int32_t *cu, int C, int W,
                           const float *x, const float *w, const float *bias,
                           const float *win_in, int silu, float *y,
                           int out_bf16, uint16_t *y_bits)
{
    int Wm1 = W - 1;
    for (int s = 0; s < n_seq; s++) {
        long t0 = cu[s], t1 = cu[s + 1], len = t1 - t0;
        for (long t = 0; t < len; t++) {
            for (int c = 0; c < C; c++) {
                float acc = bias ? bias[c] : 0.0f;
                for (int j = 0; j < W; j++) {
                    long src = t - Wm1 + j;
                    float xv;
                    if (src >= 0)
                        xv = x[(t0 + src) * C + c];
                    else
                        xv = win_in ? win_in[((long)s * Wm1 + (Wm1 + src)) * C + c] : 0.0f;
                    acc = fmaf(w[c * W + j], xv, acc);
                }
                float r = silu ? silu_f32(acc) : acc;
                if (out_bf16)
                    y_bits[(t0 + t) * C + c] = f32_to_bf16_rne(r);
                else
                    y[(t0 + t) * C + c] = r;
            }
        }
    }
}

/* ------------------------------------------------------------------ scan */

typedef struct {
    int n_seq, Hk, Hv, dk, dv;
    const int32_t *cu;
    double scale;
    unsigned flags;
    const double *q, *k, *v, *g, *beta, *state_in;
    double *o, *state_out;
    long next; /* next work item, taken under the lock */
    pthread_mutex_t lock;
} scan_job;

static void l2_normalise(const double *src, int n, double mul, double *dst, int do_norm)
{
    double f = mul;
    if (do_norm) {
        double ss = 0.0;
        for (int i = 0; i < n; i++) ss += src[i] * src[i];
        f = mul / sqrt(ss + GDN_ORACLE_L2_EPS);
    }
    for (int i = 0; i < n; i++) dst[i] = src[i] * f;
}

static void scan_one(const scan_job *J, int s, int h, double *S, double *qh, double *kh, double *u)
{
    const int dk = J->dk, dv = J->dv, Hk = J->Hk, Hv = J->Hv;
    const int hk = (J->flags & GDN_ORACLE_TILED) ? (h % Hk) : (h / (Hv / Hk));
    const int norm = (J->flags & GDN_ORACLE_L2NORM) != 0;
    const long t0 = J->cu[s], t1 = J->cu[s + 1];

    if (J->state_in)
        memcpy(S, J->state_in + ((long)s * Hv + h) * dk * dv, sizeof(double) * dk * dv);
    else
        memset(S, 0, sizeof(double) * dk * dv);

    for (long t = t0; t < t1; t++) {
        const double *qt = J->q + (t * Hk + hk) * dk;
        const double *kt = J->k + (t * Hk + hk) * dk;
        const double *vt = J->v + (t * Hv + h) * dv;
        const double alpha = exp(J->g[t * Hv + h]);
        const double b = J->beta[t * Hv + h];
        l2_normalise(qt, dk, J->scale, qh, norm);
        l2_normalise(kt, dk, 1.0, kh, norm);

        /* decay: S <- alpha S */
        for (int i = 0; i < dk * dv; i++) S[i] *= alpha;
        /* delta: u = beta (v - S^T k) */
        for (int j = 0; j < dv; j++) {
            double acc = 0.0;
            for (int i = 0; i < dk; i++) acc += S[i * dv + j] * kh[i];
            u[j] = b * (vt[j] - acc);
        }
        /* write: S <- S + k u^T */
        for (int i = 0; i < dk; i++)
            for (int j = 0; j < dv; j++) S[i * dv + j] += kh[i] * u[j];
        /* read: o = S^T q */
        double *ot = J->o + (t * Hv + h) * dv;
        for (int j = 0; j < dv; j++) {
            double acc = 0.0;
            for (int i = 0; i < dk; i++) acc += S[i * dv + j] * qh[i];
            ot[j] = acc;
        }
    }
    if (J->state_out)
        memcpy(J->state_out + ((long)s * Hv + h) * dk * dv, S, sizeof(double) * dk * dv);
}

static void *scan_worker(void *arg)
{
    scan_job *J = (scan_job *)arg;
    double *S = malloc(sizeof(double) * J->dk * J->dv);
    double *qh = malloc(sizeof(double) * J->dk);
    double *kh = malloc(sizeof(double) * J->dk);
    double *u = malloc(sizeof(double) * J->dv);
    const long total = (long)J->n_seq * J->Hv;
    for (;;) {
        pthread_mutex_lock(&J->lock);
        long item = J->next++;
        pthread_mutex_unlock(&J->lock);
        if (item >= total) break;
        scan_one(J, (int)(item / J->Hv), (int)(item % J->Hv), S, qh, kh, u);
    }
    free(S); free(qh); free(kh); free(u);
    return NULL;
}

int gdn_oracle_available_cores(void)
{
    cpu_set_t set;
    if (sched_getaffinity(0, sizeof(set), &set) == 0) return CPU_COUNT(&set);
    return 1;
}

/* q,k: [n_tok][Hk][dk]; v: [n_tok][Hv][dv]; g, beta: [n_tok][Hv];
 * state_in: [n_seq][Hv][dk][dv] or NULL (zeros); o: [n_tok][Hv][dv];
 * state_out: [n_seq][Hv][dk][dv] or NULL.  n_threads <= 0: every core in the
 * affinity mask.  Returns the number of threads used, or -1 on bad shapes. */
int gdn_oracle_scan(int n_seq, const int32_t *cu, int Hk, int Hv, int dk, int dv,
                    double scale, unsigned flags,
                    const double *q, const double *k, const double *v,
                    const double *g, const double *beta, const double *state_in,
                    double *o, double *state_out, int n_threads)
{
    if (n_seq < 0 || Hk <= 0 || Hv <= 0 || Hv % Hk != 0 || dk <= 0 || dv <= 0) return -1;
    scan_job J = {n_seq, Hk, Hv, dk, dv, cu, scale, flags, q, k, v, g, beta, state_in,
                  o, state_out, 0, PTHREAD_MUTEX_INITIALIZER};
    long total = (long)n_seq * Hv;
    int nt = n_threads > 0 ? n_threads : gdn_oracle_available_cores();
    if (nt > total) nt = (int)(total > 0 ? total : 1);
    if (nt <= 1) {
        scan_worker(&J);
        return 1;
    }
    pthread_t *th = malloc(sizeof(pthread_t) * nt);
    for (int i = 0; i < nt; i++) pthread_create(&th[i], NULL, scan_worker, &J);
    for (int i = 0; i < nt; i++) pthread_join(th[i], NULL);
    free(th);
    return nt;
}

/* ---------------------------------------------------------- gated norm */

/* o, z, y: [rows][d] (a row is one token's one v-head); w: [d]. */
void gdn_oracle_gated_rmsnorm(long rows, int d, const double *o, const double *z,
                              const double *w, double eps, double *y)
{
    for (long r = 0; r < rows; r++) {
        const double *orow = o + r * d, *zrow = z + r * d;
        double ss = 0.0;
        for (int j = 0; j < d; j++) ss += orow[j] * orow[j];
        const double inv_rms = 1.0 / sqrt(ss / d + eps);
        for (int j = 0; j < d; j++) y[r * d + j] = w[j] * orow[j] * inv_rms * silu_f64(zrow[j]);
    }
}

/* --------------------------------------------------------------- gating */

static double softplus_f64(double x) { return (x > 0.0 ? x : 0.0) + log1p(exp(-fabs(x))); }

/* a, b, g, beta: [n_tok][H]; A_log, dt_bias: [H]. */
void gdn_oracle_gating(long n_tok, int H, const double *a, const double *b, const double *A_log,
                       const double *dt_bias, double *g, double *beta)
{
    for (long t = 0; t < n_tok; t++)
        for (int h = 0; h < H; h++) {
            const long i = t * H + h;
            g[i] = -exp(A_log[h]) * softplus_f64(a[i] + dt_bias[h]);
            beta[i] = 1.0 / (1.0 + exp(-b[i]));
        }
}
