/*
 * kda_oracle.c -- plain, slow, sequential fp64 reference of the Kimi Delta
 * Attention (KDA) layer core: short-conv(4) + SiLU + L2 prologue, the gated
 * delta-rule recurrence, and the sigma(g) * RMSNorm epilogue.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, includes
 * or calls this file; only the test suite, the smoke check and the CPU
 * baseline of the benchmark load it.  It shares no code, header or constant
 * with the HIP kernels.
 *
 * Sources (web pages on Kimi K3; cited by title and section):
 *  [Atlas]  "Kimi K3 - KDA layer" (OpenModelAtlas), the per-step equation
 *           list of the KDA block: conv + SiLU, L2 normalisation, the gates,
 *           S <- Diag(alpha) S, S <- S + beta k (v - S^T k)^T,
 *           o~ = S^T q / sqrt(128), o^g = sigma(g) * RMSNorm(o~).
 *  [Baena]  "Inside Kimi K3: How KDA, AttnRes, and 896 Experts Work",
 *           section "KDA writes corrections into a recurrent matrix" (the
 *           five-step order: decay, predict, error, write, read) and section
 *           "Short convolutions give KDA local order before recurrence"
 *           (kernel size four; Swish; L2 on q and k only).
 *  [SGLang] "Kimi K3: Architecture and SGLang Day-0 Support", section
 *           "Math details: how KDA gates and rewrites the same S" (alpha
 *           scales row j of S, i.e. the key channel; gate first, then the
 *           delta rewrite against the decayed state).
 *
 * Arithmetic is IEEE double throughout, in the order the pages state the
 * steps.  No blocking, chunking, reassociation or fused forms: one token at
 * a time, one (sequence, head) pair at a time.  Threads only split the
 * independent (sequence, head) pairs.
 *
 * Readings taken where the pages are silent (all passed in by the caller):
 *  - the read scale 1/sqrt(dk) is a parameter (`scale`);
 *  - the L2 normalisation is x / sqrt(sum x^2 + l2_eps);
 *  - RMSNorm is per head over dv channels, x / sqrt(mean x^2 + rms_eps) * w,
 *    with one gain vector w[dv] shared by all heads and no bias;
 *  - the causal depthwise conv has no bias, tap j multiplies x_{t-j}, and
 *    the history before a sequence is the given conv cache or zeros;
 *  - the conv cache holds the three most recent pre-conv inputs, oldest first.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define CONV_HIST 3 /* kernel size 4 minus the current token */

typedef struct {
    int n_seqs, n_heads, dk, dv;
    const int64_t *cu; /* [n_seqs + 1] token offsets */
    const double *q, *k, *v; /* [T][H][dk], [T][H][dk], [T][H][dv] */
    const double *g;         /* [T][H][dv] or NULL when the epilogue is off */
    const double *log_alpha; /* [T][H][dk] */
    const double *beta;      /* [T][H] */
    const double *wq, *wk, *wv; /* [H*dk][4], [H*dk][4], [H*dv][4] */
    const double *cq_in, *ck_in, *cv_in; /* [N][3][H*dk|dv] or NULL (zeros) */
    const double *rms_w;     /* [dv] or NULL (ones) */
    const double *s_in;      /* [N][H][dk][dv] or NULL (zeros) */
    double scale, l2_eps, rms_eps;
    int prologue, epilogue;
    double *o;               /* [T][H][dv] */
    double *s_out;           /* [N][H][dk][dv] or NULL */
    double *cq_out, *ck_out, *cv_out; /* [N][3][H*dk|dv] or NULL */
    int next_item;           /* work counter shared by the threads */
} job_t;

static double sigmoid(double x) { return 1.0 / (1.0 + exp(-x)); }

/* The two low-rank gates.  Both read u = z_down W_up + b_alpha for output channel
 * c = h * d + i, with W_up passed output-major (w[c][j] = W_up[j][c]), b_alpha one value
 * per output channel and A one scalar per head (the per-head A_h of [Jawad],
 * "Channel-wise decay, and the floor K3 puts under it"); these are readings where the
 * pages are silent.  Plain loops in fp64, token by token.
 *   z    [T][r]       the low-rank projection z_down of each token
 *   w    [H*d][r]     W_up, row c = output channel c
 *   b    [H*d]        b_alpha
 *   a    [H]          A_h
 *   out  [T][H][d]    log alpha
 * K3's gate ([Atlas] step list; [Jawad], same section): alpha = exp(-5 sigmoid(e^A u)),
 * so log alpha lies in (-5, 0).
 * Kimi Linear's gate, the unbounded log-decay that [Jawad]'s section contrasts with it:
 * log alpha = -e^A softplus(u), softplus(u) = log(1 + e^u), any value in (-inf, 0).  For
 * u > 0 softplus is evaluated as u + log(1 + e^-u), the same value without overflowing e^u. */
static double softplus(double u) { return u > 0.0 ? u + log1p(exp(-u)) : log1p(exp(u)); }

static int lowrank_gate(int64_t T, int H, int d, int r, const double *z, const double *w,
                        const double *b, const double *a, int unbounded, double *out) {
    if (T < 0 || H <= 0 || d <= 0 || r <= 0 || !z || !w || !b || !a || !out) return 1;
    for (int64_t t = 0; t < T; ++t)
        for (int h = 0; h < H; ++h) {
            const double ea = exp(a[h]);
            for (int i = 0; i < d; ++i) {
                const int64_t c = (int64_t)h * d + i;
                double zc = 0.0;
                for (int j = 0; j < r; ++j) zc += z[t * r + j] * w[c * r + j];
                const double u = zc + b[c];
                out[(t * H + h) * d + i] = unbounded ? -ea * softplus(u) : -5.0 * sigmoid(ea * u);
            }
        }
    return 0;
}

int kda_oracle_lowrank_log_alpha(int64_t T, int H, int d, int r, const double *z, const double *w,
                                 const double *b, const double *a, double *out) {
    return lowrank_gate(T, H, d, r, z, w, b, a, 0, out);
}

int kda_oracle_softplus_log_alpha(int64_t T, int H, int d, int r, const double *z, const double *w,
                                  const double *b, const double *a, double *out) {
    return lowrank_gate(T, H, d, r, z, w, b, a, 1, out);
}

/* The write strength from its pre-activation ([Atlas] step list: w = x W_beta, then
 * beta = sigma(w)), one value per (token, head):  beta = 1 / (1 + e^-w).  For w far below
 * zero e^-w overflows to +inf and beta is 0, the limit. */
int kda_oracle_beta_from_logit(int64_t n, const double *w, double *beta) {
    if (n < 0 || (n > 0 && (!w || !beta))) return 1;
    for (int64_t i = 0; i < n; ++i) beta[i] = 1.0 / (1.0 + exp(-w[i]));
    return 0;
}

/* One stream of the prologue for one token ([Atlas] conv + SiLU step):
 * y_c = sum_{j=0..3} w[c][j] * x_{t-j}[c],  a_c = y_c * sigmoid(y_c).
 * hist[0..2] holds x_{t-3}, x_{t-2}, x_{t-1} and is shifted to take x_t. */
static void conv_silu(int d, const double *x_t, const double *w, double *hist,
                      double *out) {
    for (int c = 0; c < d; ++c) {
        const double *wc = w + (size_t)c * 4;
        double y = wc[0] * x_t[c] + wc[1] * hist[2 * d + c] +
                   wc[2] * hist[1 * d + c] + wc[3] * hist[0 * d + c];
        out[c] = y * sigmoid(y);
        hist[0 * d + c] = hist[1 * d + c];
        hist[1 * d + c] = hist[2 * d + c];
        hist[2 * d + c] = x_t[c];
    }
}

/* x <- x / sqrt(sum x^2 + eps)  ([Atlas] q^ = q^h/||q^h||, k^ likewise). */
static void l2_normalise(int d, double *x, double eps) {
    double ss = 0.0;
    for (int c = 0; c < d; ++c) ss += x[c] * x[c];
    double inv = 1.0 / sqrt(ss + eps);
    for (int c = 0; c < d; ++c) x[c] *= inv;
}

/* 1. decay: S <- Diag(alpha) S.  alpha[i] scales row i of S, the key channel
 *    ([SGLang] "Math details": Diag(alpha_t) scales row j of S by alpha_t[j]). */
static void decay_rows(int dk, int dv, double *S, const double *alpha) {
    for (int i = 0; i < dk; ++i)
        for (int j = 0; j < dv; ++j) S[i * dv + j] *= alpha[i];
}

/* 2. predict what the (decayed) state returns for the key: r = S^T k. */
static void predict(int dk, int dv, const double *S, const double *kh, double *r) {
    for (int j = 0; j < dv; ++j) {
        double acc = 0.0;
        for (int i = 0; i < dk; ++i) acc += S[i * dv + j] * kh[i];
        r[j] = acc;
    }
}

/* 3-4. error v - r, written with strength beta: S <- S + beta k (v - r)^T
 *      ([Atlas] delta-rule step). */
static void write_error(int dk, int dv, double *S, const double *kh, const double *vv,
                        const double *r, double b) {
    for (int i = 0; i < dk; ++i)
        for (int j = 0; j < dv; ++j) S[i * dv + j] += b * kh[i] * (vv[j] - r[j]);
}

/* 5. read the updated state: o~ = scale * S^T q  ([Atlas] read step, scale
 *    1/sqrt(128) at d_k = 128). */
static void read_state(int dk, int dv, const double *S, const double *qh, double scale,
                       double *ot) {
    for (int j = 0; j < dv; ++j) {
        double acc = 0.0;
        for (int i = 0; i < dk; ++i) acc += S[i * dv + j] * qh[i];
        ot[j] = scale * acc;
    }
}

static void load_hist(const job_t *jb, const double *src, int n, int h, int d,
                      double *hist) {
    size_t width = (size_t)jb->n_heads * d;
    for (int j = 0; j < CONV_HIST; ++j)
        for (int c = 0; c < d; ++c)
            hist[j * d + c] =
                src ? src[((size_t)n * CONV_HIST + j) * width + (size_t)h * d + c]
                    : 0.0;
}

static void store_hist(const job_t *jb, double *dst, int n, int h, int d,
                       const double *hist) {
    if (!dst) return;
    size_t width = (size_t)jb->n_heads * d;
    for (int j = 0; j < CONV_HIST; ++j)
        for (int c = 0; c < d; ++c)
            dst[((size_t)n * CONV_HIST + j) * width + (size_t)h * d + c] =
                hist[j * d + c];
}

/* The whole recurrence for one (sequence n, head h) pair. */
static void run_pair(const job_t *jb, int n, int h, double *scratch) {
    const int H = jb->n_heads, dk = jb->dk, dv = jb->dv;
    double *S = scratch;                 /* dk*dv, S[i*dv + j], i = key channel */
    double *qh = S + (size_t)dk * dv;    /* dk */
    double *kh = qh + dk;                /* dk */
    double *vv = kh + dk;                /* dv */
    double *alpha = vv + dv;             /* dk */
    double *r = alpha + dk;              /* dv */
    double *ot = r + dv;                 /* dv */
    double *hq = ot + dv;                /* 3*dk */
    double *hk = hq + CONV_HIST * dk;    /* 3*dk */
    double *hv = hk + CONV_HIST * dk;    /* 3*dv */

    const size_t sdim = (size_t)dk * dv;
    if (jb->s_in)
        memcpy(S, jb->s_in + ((size_t)n * H + h) * sdim, sdim * sizeof(double));
    else
        memset(S, 0, sdim * sizeof(double));
    if (jb->prologue) {
        load_hist(jb, jb->cq_in, n, h, dk, hq);
        load_hist(jb, jb->ck_in, n, h, dk, hk);
        load_hist(jb, jb->cv_in, n, h, dv, hv);
    }

    for (int64_t t = jb->cu[n]; t < jb->cu[n + 1]; ++t) {
        const size_t row_k = ((size_t)t * H + h) * dk;
        const size_t row_v = ((size_t)t * H + h) * dv;

        /* Prologue ([Atlas] conv/SiLU/L2 steps; [Baena] short convolutions). */
        if (jb->prologue) {
            conv_silu(dk, jb->q + row_k, jb->wq + (size_t)h * dk * 4, hq, qh);
            conv_silu(dk, jb->k + row_k, jb->wk + (size_t)h * dk * 4, hk, kh);
            conv_silu(dv, jb->v + row_v, jb->wv + (size_t)h * dv * 4, hv, vv);
            l2_normalise(dk, qh, jb->l2_eps);
            l2_normalise(dk, kh, jb->l2_eps);
        } else {
            memcpy(qh, jb->q + row_k, dk * sizeof(double));
            memcpy(kh, jb->k + row_k, dk * sizeof(double));
            memcpy(vv, jb->v + row_v, dv * sizeof(double));
        }
        for (int i = 0; i < dk; ++i) alpha[i] = exp(jb->log_alpha[row_k + i]);
        const double b = jb->beta[(size_t)t * H + h];

        /* [Baena] order: decay, predict, error + write, read the new state. */
        decay_rows(dk, dv, S, alpha);
        predict(dk, dv, S, kh, r);
        write_error(dk, dv, S, kh, vv, r, b);
        read_state(dk, dv, S, qh, jb->scale, ot);

        /* Epilogue ([Atlas] o^g = sigma(g) * RMSNorm(o~)). */
        double *o = jb->o + row_v;
        if (jb->epilogue) {
            double ms = 0.0;
            for (int j = 0; j < dv; ++j) ms += ot[j] * ot[j];
            ms /= dv;
            double inv = 1.0 / sqrt(ms + jb->rms_eps);
            for (int j = 0; j < dv; ++j) {
                double w = jb->rms_w ? jb->rms_w[j] : 1.0;
                o[j] = sigmoid(jb->g[row_v + j]) * (ot[j] * inv) * w;
            }
        } else {
            for (int j = 0; j < dv; ++j) o[j] = ot[j];
        }
    }

    if (jb->s_out)
        memcpy(jb->s_out + ((size_t)n * H + h) * sdim, S, sdim * sizeof(double));
    if (jb->prologue) {
        store_hist(jb, jb->cq_out, n, h, dk, hq);
        store_hist(jb, jb->ck_out, n, h, dk, hk);
        store_hist(jb, jb->cv_out, n, h, dv, hv);
    }
}

static void *worker(void *arg) {
    job_t *jb = (job_t *)arg;
    const int dk = jb->dk, dv = jb->dv;
    size_t words = (size_t)dk * dv + 3 * (size_t)dk + 4 * (size_t)dv +
                   CONV_HIST * (2 * (size_t)dk + dv);
    double *scratch = (double *)malloc(words * sizeof(double));
    if (!scratch) return (void *)1;
    const int items = jb->n_seqs * jb->n_heads;
    for (;;) {
        int it = __atomic_fetch_add(&jb->next_item, 1, __ATOMIC_RELAXED);
        if (it >= items) break;
        run_pair(jb, it / jb->n_heads, it % jb->n_heads, scratch);
    }
    free(scratch);
    return NULL;
}

/* Entry point used through ctypes.  Returns 0 on success, nonzero when the
 * arguments are inconsistent or memory could not be obtained. */
int kda_oracle_run(int n_seqs, int n_heads, int dk, int dv, const int64_t *cu,
                   const double *q, const double *k, const double *v,
                   const double *g, const double *log_alpha, const double *beta,
                   const double *wq, const double *wk, const double *wv,
                   const double *cq_in, const double *ck_in, const double *cv_in,
                   const double *rms_w, const double *s_in, double scale,
                   double l2_eps, double rms_eps, int prologue, int epilogue,
                   double *o, double *s_out, double *cq_out, double *ck_out,
                   double *cv_out, int n_threads) {
    if (n_seqs < 0 || n_heads <= 0 || dk <= 0 || dv <= 0 || !cu) return 1;
    if (prologue && (!wq || !wk || !wv)) return 1;
    if (epilogue && !g) return 1;
    for (int n = 0; n < n_seqs; ++n)
        if (cu[n + 1] < cu[n]) return 1;
    if (n_seqs == 0) return 0;
    job_t jb = {n_seqs, n_heads, dk, dv, cu, q, k, v, g, log_alpha, beta,
                wq, wk, wv, cq_in, ck_in, cv_in, rms_w, s_in,
                scale, l2_eps, rms_eps, prologue, epilogue,
                o, s_out, cq_out, ck_out, cv_out, 0};
    int items = n_seqs * n_heads;
    if (n_threads < 1) n_threads = 1;
    if (n_threads > items) n_threads = items;
    if (n_threads == 1) return worker(&jb) ? 2 : 0;
    pthread_t *th = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)n_threads);
    if (!th) return 2;
    int rc = 0, started = 0;
    for (; started < n_threads; ++started)
        if (pthread_create(&th[started], NULL, worker, &jb) != 0) break;
    if (started == 0) rc = worker(&jb) ? 2 : 0;
    for (int i = 0; i < started; ++i) {
        void *ret = NULL;
        pthread_join(th[i], &ret);
        if (ret) rc = 2;
    }
    free(th);
    return rc;
}
