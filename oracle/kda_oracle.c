/*
 * kda_oracle.c -- plain fp64 CPU oracle for the KDA token mixer.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header, table or constant with the HIP library, and the HIP library never
 * calls it.
 *
 * What it computes (sources are the pages on Kimi K3; none prints a formula,
 * so each step below is the plainest reading of the words):
 *
 *   Per (batch b, head h) the memory is a fixed-size matrix S (d_k x d_v)
 *   [lotamate.com "Kimi K3 是如何训练出来的", §一.1: history is compressed
 *   into a fixed-size memory-state matrix; devpress.csdn.net K3 article §十六:
 *   KDA keeps a recursive state instead of per-token K/V].
 *
 *   For each token t, in order:
 *     1. retention, per key channel c (the channel-wise forget gate with a
 *        per-step lower bound) [zuoshipin.com/article/18261 §二; devpress
 *        §二 last paragraph]:
 *            lambda_c = max(log_alpha_{t,c}, log_alpha_min)
 *            S[c,:]  <- exp(lambda_c) * S[c,:]
 *     2. q and k are L2-normalised over d_k [zuoshipin §四, FlashKDA
 *        paragraph, lists Query/Key normalisation among the per-chunk steps]:
 *            kh = k_t / max(|k_t|, 1e-6),   qh likewise
 *     3. predict from the retained memory, take the error against the new
 *        value, write the correction with strength beta_t [devpress §二:
 *        predict, compare, correct; "new memory = retained old memory +
 *        correction of its wrong part"]:
 *            p = S^T kh ;  u = beta_t (v_t - p) ;  S <- S + kh u^T
 *     4. read-out after the write, then the full-rank output gate
 *        [zuoshipin §二: the output gate decides which channels reach the
 *        next layer]:
 *            o = S^T qh ;  out_t = o * sigmoid(g_t)
 *
 *   kda_oracle_summary: the per-segment pair of the context-parallel scheme
 *   [zuoshipin §三, "KDA 上下文并行" paragraph: how the segment changes an
 *   existing memory, and what it builds from an empty one]:
 *     S_end = A S_start + Bz, A (d_k x d_k) = product of the per-token maps,
 *     Bz = the run from S_start = 0.  Computed by running the same steps on
 *     the augmented state [Bz | A] from [0 | I] with value columns [v | 0].
 *
 *   kda_oracle_combine: the in-order prefix merge of those pairs (same
 *   paragraph): S_in(0) = S_init, S_in(n+1) = A_n S_in(n) + Bz_n.
 *
 *   kda_oracle_grad: the gradients of L = <d_out, out> + <d_state, S_T> with
 *   respect to q, k, v, log_alpha, beta, g and the initial state -- the
 *   adjoint of the four steps above, taken token by token in reverse (the
 *   backward pass serves training [zuoshipin §四: FlashKDA serves training
 *   throughput]).  The forward pass stores the state entering every token;
 *   each reverse step recomputes that token's intermediates from it.
 *
 * All arrays are fp64, C-contiguous, token-major [B,T,H,d]; states are
 * [B,H,d_k,d_v] with row = key channel.  Work items are (b, h, block of state
 * columns): the columns of S never interact, so a block of them can be
 * advanced alone.  Threads: plain pthreads over the items.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
    int64_t B, T;
    int H, dk, dv;
    const double *q, *k, *v, *log_alpha, *beta, *g;
    double log_alpha_min;
    const double *state_in; /* [B,H,dk,dv] or NULL (zeros) */
    double *out;            /* [B,T,H,dv] or NULL (not written) */
    double *state_out;      /* [B,H,dk,dv] or NULL */
    /* summary mode: advance [Bz | A] (width dv + dk) from [0 | I] */
    int summary;
    double *A;              /* [B,H,dk,dk] */
    double *Bz;             /* [B,H,dk,dv] */
    int ncb;                /* number of column blocks per (b,h) */
    int width;              /* state width: dv, or dv + dk in summary mode */
} job_t;

typedef struct {
    const job_t *job;
    int64_t first, step, count;
    int status;
} worker_t;

/* Advance one block of state columns [c0, c1) of one (b, h) over all tokens. */
static int run_item(const job_t *J, int64_t b, int h, int c0, int c1)
{
    const int dk = J->dk, dv = J->dv, H = J->H, w = c1 - c0;
    double *S = (double *)calloc((size_t)dk * (size_t)w, sizeof(double)); /* S[c][j - c0] */
    double *kh = (double *)malloc((size_t)dk * sizeof(double));
    double *qh = (double *)malloc((size_t)dk * sizeof(double));
    if (!S || !kh || !qh) { free(S); free(kh); free(qh); return 1; }

    /* initial state */
    for (int c = 0; c < dk; ++c)
        for (int j = c0; j < c1; ++j) {
            double s0 = 0.0;
            if (J->summary) {
                if (j >= dv) s0 = (j - dv == c) ? 1.0 : 0.0;   /* A part starts at I */
            } else if (J->state_in) {
                s0 = J->state_in[(((size_t)b * H + h) * dk + c) * dv + j];
            }
            S[(size_t)c * w + (j - c0)] = s0;
        }

    for (int64_t t = 0; t < J->T; ++t) {
        const size_t row = ((size_t)b * (size_t)J->T + (size_t)t) * (size_t)H + (size_t)h;
        const double *kt = J->k + row * dk, *qt = J->q + row * dk;
        const double *lat = J->log_alpha + row * dk;
        const double *vt = J->v + row * dv;
        const double bt = J->beta[row];

        /* 1. retention on key channels, with the per-step lower bound */
        for (int c = 0; c < dk; ++c) {
            double lam = lat[c] > J->log_alpha_min ? lat[c] : J->log_alpha_min;
            double a = exp(lam);
            double *Sc = S + (size_t)c * w;
            for (int j = 0; j < w; ++j) Sc[j] *= a;
        }
        /* 2. L2 normalisation of k and q */
        double nk = 0.0, nq = 0.0;
        for (int c = 0; c < dk; ++c) { nk += kt[c] * kt[c]; nq += qt[c] * qt[c]; }
        nk = sqrt(nk); nq = sqrt(nq);
        if (nk < 1e-6) nk = 1e-6;
        if (nq < 1e-6) nq = 1e-6;
        for (int c = 0; c < dk; ++c) { kh[c] = kt[c] / nk; qh[c] = qt[c] / nq; }

        /* 3. predict, error, corrective write -- column by column */
        for (int j = 0; j < w; ++j) {
            const int col = c0 + j;
            double p = 0.0;
            for (int c = 0; c < dk; ++c) p += S[(size_t)c * w + j] * kh[c];
            const double vj = (col < dv) ? vt[col] : 0.0;   /* A-part columns see v = 0 */
            const double u = bt * (vj - p);
            for (int c = 0; c < dk; ++c) S[(size_t)c * w + j] += kh[c] * u;
        }
        /* 4. read-out after the write, then the output gate */
        if (J->out) {
            const double *gt = J->g + row * dv;
            double *ot = J->out + row * dv;
            for (int j = 0; j < w; ++j) {
                const int col = c0 + j;
                if (col >= dv) continue;
                double o = 0.0;
                for (int c = 0; c < dk; ++c) o += S[(size_t)c * w + j] * qh[c];
                ot[col] = o * (1.0 / (1.0 + exp(-gt[col])));
            }
        }
    }

    /* final state */
    for (int c = 0; c < dk; ++c)
        for (int j = c0; j < c1; ++j) {
            const double s = S[(size_t)c * w + (j - c0)];
            if (J->summary) {
                if (j < dv) J->Bz[(((size_t)b * H + h) * dk + c) * dv + j] = s;
                else        J->A[(((size_t)b * H + h) * dk + c) * dk + (j - dv)] = s;
            } else if (J->state_out) {
                J->state_out[(((size_t)b * H + h) * dk + c) * dv + j] = s;
            }
        }
    free(S); free(kh); free(qh);
    return 0;
}

static void *worker_main(void *arg)
{
    worker_t *W = (worker_t *)arg;
    const job_t *J = W->job;
    for (int64_t n = 0; n < W->count; ++n) {
        const int64_t item = W->first + n * W->step;
        const int64_t bh = item / J->ncb;
        const int cb = (int)(item % J->ncb);
        const int bsz = (J->width + J->ncb - 1) / J->ncb;
        const int c0 = cb * bsz;
        int c1 = c0 + bsz;
        if (c1 > J->width) c1 = J->width;
        if (c0 >= c1) continue;
        if (run_item(J, bh / J->H, (int)(bh % J->H), c0, c1)) { W->status = 1; return NULL; }
    }
    return NULL;
}

static int run_job(job_t *J, int nthreads)
{
    if (J->B < 0 || J->T < 0 || J->H <= 0 || J->dk <= 0 || J->dv <= 0) return 2;
    if (nthreads < 1) nthreads = 1;
    const int64_t nbh = J->B * (int64_t)J->H;
    /* enough column blocks to give every thread work, at least 8 columns each */
    int ncb = 1;
    while (nbh * ncb < nthreads && J->width / (ncb * 2) >= 8) ncb *= 2;
    J->ncb = ncb;
    const int64_t items = nbh * ncb;
    if (items == 0) return 0;
    if (nthreads > items) nthreads = (int)items;

    pthread_t *th = (pthread_t *)calloc((size_t)nthreads, sizeof(pthread_t));
    worker_t *ws = (worker_t *)calloc((size_t)nthreads, sizeof(worker_t));
    if (!th || !ws) { free(th); free(ws); return 1; }
    int started = 0, status = 0;
    for (int i = 0; i < nthreads; ++i) {
        ws[i].job = J;
        ws[i].first = i;
        ws[i].step = nthreads;
        ws[i].count = (items - i + nthreads - 1) / nthreads;
        if (nthreads == 1) { worker_main(&ws[i]); continue; }
        if (pthread_create(&th[i], NULL, worker_main, &ws[i]) != 0) { status = 1; break; }
        ++started;
    }
    for (int i = 0; i < started; ++i) pthread_join(th[i], NULL);
    for (int i = 0; i < nthreads; ++i) status |= ws[i].status;
    free(th); free(ws);
    return status;
}

/* The step recurrence.  Returns 0 on success. */
int kda_oracle_ref(int64_t B, int64_t T, int H, int dk, int dv,
                   const double *q, const double *k, const double *v,
                   const double *log_alpha, const double *beta, const double *g,
                   double log_alpha_min, const double *state_in,
                   double *out, double *state_out, int nthreads)
{
    job_t J;
    memset(&J, 0, sizeof J);
    J.B = B; J.T = T; J.H = H; J.dk = dk; J.dv = dv;
    J.q = q; J.k = k; J.v = v; J.log_alpha = log_alpha; J.beta = beta; J.g = g;
    J.log_alpha_min = log_alpha_min; J.state_in = state_in;
    J.out = out; J.state_out = state_out;
    J.width = dv;
    if (T == 0 && state_out) {   /* nothing to advance: the state passes through */
        for (size_t i = 0; i < (size_t)(B * H) * dk * dv; ++i) state_out[i] = state_in ? state_in[i] : 0.0;
        return 0;
    }
    return run_job(&J, nthreads);
}

/* The segment pair (A, Bz) with S_end = A S_start + Bz.  q and g are unused. */
int kda_oracle_summary(int64_t B, int64_t T, int H, int dk, int dv,
                       const double *k, const double *v,
                       const double *log_alpha, const double *beta,
                       double log_alpha_min, double *A, double *Bz, int nthreads)
{
    job_t J;
    memset(&J, 0, sizeof J);
    J.B = B; J.T = T; J.H = H; J.dk = dk; J.dv = dv;
    J.q = k; J.k = k; J.v = v; J.log_alpha = log_alpha; J.beta = beta;
    J.log_alpha_min = log_alpha_min;
    J.summary = 1; J.A = A; J.Bz = Bz;
    J.width = dv + dk;
    return run_job(&J, nthreads);
}

/* In-order merge of per-segment pairs, one (b, h) chain at a time.
 * A [B,n_seg,H,dk,dk], Bz [B,n_seg,H,dk,dv], state_init [B,H,dk,dv] or NULL,
 * seg_state_in [B,n_seg,H,dk,dv] (the state entering each segment),
 * state_final [B,H,dk,dv] or NULL. */
int kda_oracle_combine(int64_t B, int n_seg, int H, int dk, int dv,
                       const double *A, const double *Bz, const double *state_init,
                       double *seg_state_in, double *state_final)
{
    double *cur = (double *)malloc((size_t)dk * dv * sizeof(double));
    double *nxt = (double *)malloc((size_t)dk * dv * sizeof(double));
    if (!cur || !nxt) { free(cur); free(nxt); return 1; }
    for (int64_t b = 0; b < B; ++b)
        for (int h = 0; h < H; ++h) {
            for (int i = 0; i < dk * dv; ++i)
                cur[i] = state_init ? state_init[((size_t)b * H + h) * dk * dv + i] : 0.0;
            for (int n = 0; n < n_seg; ++n) {
                const size_t sh = ((size_t)b * n_seg + n) * H + h;
                memcpy(seg_state_in + sh * dk * dv, cur, (size_t)dk * dv * sizeof(double));
                const double *An = A + sh * dk * dk, *Bn = Bz + sh * dk * dv;
                for (int i = 0; i < dk; ++i)
                    for (int j = 0; j < dv; ++j) {
                        double s = Bn[(size_t)i * dv + j];
                        for (int c = 0; c < dk; ++c) s += An[(size_t)i * dk + c] * cur[(size_t)c * dv + j];
                        nxt[(size_t)i * dv + j] = s;
                    }
                double *tmp = cur; cur = nxt; nxt = tmp;
            }
            if (state_final) memcpy(state_final + ((size_t)b * H + h) * dk * dv, cur, (size_t)dk * dv * sizeof(double));
        }
    free(cur); free(nxt);
    return 0;
}


/* ------------------------------------------------------------------------ */
/* Gradients (the adjoint of the step recurrence, one (b, h) per work item). */

typedef struct {
    int64_t B, T;
    int H, dk, dv;
    const double *q, *k, *v, *log_alpha, *beta, *g, *state_in, *d_out, *d_state;
    double log_alpha_min;
    double *dq, *dk_, *dv_, *dla, *dbeta, *dg, *d_state_in;
} gjob_t;

typedef struct {
    const gjob_t *job;
    int64_t first, step, count;
    int status;
} gworker_t;

/* x^ = x / max(|x|, 1e-6); returns the divisor */
static double unit(const double *x, double *xh, int n)
{
    double s = 0.0;
    for (int c = 0; c < n; ++c) s += x[c] * x[c];
    s = sqrt(s);
    const double nx = s < 1e-6 ? 1e-6 : s;
    for (int c = 0; c < n; ++c) xh[c] = x[c] / nx;
    return s;
}

/* dx from dx^ for x^ = x / max(|x|, 1e-6): below the floor the divisor is a
 * constant; above it, d(x/|x|) = (I - x^ x^T) / |x|. */
static void unit_back(const double *xh, double norm, const double *dxh, double *dx, int n)
{
    if (norm < 1e-6) {
        for (int c = 0; c < n; ++c) dx[c] = dxh[c] / 1e-6;
        return;
    }
    double dot = 0.0;
    for (int c = 0; c < n; ++c) dot += xh[c] * dxh[c];
    for (int c = 0; c < n; ++c) dx[c] = (dxh[c] - xh[c] * dot) / norm;
}

static int grad_item(const gjob_t *J, int64_t b, int h)
{
    const int dk = J->dk, dv = J->dv, H = J->H;
    const int64_t T = J->T;
    const size_t SZ = (size_t)dk * dv;
    double *hist = (double *)malloc((size_t)(T > 0 ? T : 1) * SZ * sizeof(double)); /* state entering token t */
    double *S = (double *)malloc(SZ * sizeof(double));
    double *Sp = (double *)malloc(SZ * sizeof(double));   /* retained state D S_prev */
    double *dS = (double *)malloc(SZ * sizeof(double));
    double *work = (double *)malloc((size_t)(8 * dk + 8 * dv) * sizeof(double));
    if (!hist || !S || !Sp || !dS || !work) { free(hist); free(S); free(Sp); free(dS); free(work); return 1; }
    double *kh = work, *qh = kh + dk, *D = qh + dk, *dkh = D + dk, *dqh = dkh + dk, *tmpk = dqh + dk;
    double *p = tmpk + 2 * dk, *u = p + dv, *o = u + dv, *du = o + dv, *dp = du + dv, *dov = dp + dv;
    const size_t sb = ((size_t)b * H + h) * SZ;

    for (size_t i = 0; i < SZ; ++i) S[i] = J->state_in ? J->state_in[sb + i] : 0.0;
    /* forward: the same four steps as run_item, keeping the entering states */
    for (int64_t t = 0; t < T; ++t) {
        const size_t row = ((size_t)b * (size_t)T + (size_t)t) * (size_t)H + (size_t)h;
        memcpy(hist + (size_t)t * SZ, S, SZ * sizeof(double));
        for (int c = 0; c < dk; ++c) {
            const double la = J->log_alpha[row * dk + c];
            const double a = exp(la > J->log_alpha_min ? la : J->log_alpha_min);
            for (int j = 0; j < dv; ++j) S[(size_t)c * dv + j] *= a;
        }
        unit(J->k + row * dk, kh, dk);
        for (int j = 0; j < dv; ++j) {
            double pj = 0.0;
            for (int c = 0; c < dk; ++c) pj += S[(size_t)c * dv + j] * kh[c];
            const double uj = J->beta[row] * (J->v[row * dv + j] - pj);
            for (int c = 0; c < dk; ++c) S[(size_t)c * dv + j] += kh[c] * uj;
        }
    }

    /* reverse: dS is the gradient with respect to the state after token t */
    for (size_t i = 0; i < SZ; ++i) dS[i] = J->d_state ? J->d_state[sb + i] : 0.0;
    for (int64_t t = T - 1; t >= 0; --t) {
        const size_t row = ((size_t)b * (size_t)T + (size_t)t) * (size_t)H + (size_t)h;
        const double *Sprev = hist + (size_t)t * SZ;
        const double bt = J->beta[row];
        const double *vt = J->v + row * dv, *gt = J->g + row * dv;
        /* recompute the token's intermediates */
        for (int c = 0; c < dk; ++c) {
            const double la = J->log_alpha[row * dk + c];
            D[c] = exp(la > J->log_alpha_min ? la : J->log_alpha_min);
            for (int j = 0; j < dv; ++j) Sp[(size_t)c * dv + j] = D[c] * Sprev[(size_t)c * dv + j];
        }
        const double nk = unit(J->k + row * dk, kh, dk);
        const double nq = unit(J->q + row * dk, qh, dk);
        for (int j = 0; j < dv; ++j) {
            double pj = 0.0;
            for (int c = 0; c < dk; ++c) pj += Sp[(size_t)c * dv + j] * kh[c];
            p[j] = pj;
            u[j] = bt * (vt[j] - pj);
        }
        for (int c = 0; c < dk; ++c)      /* S = state after the token */
            for (int j = 0; j < dv; ++j) S[(size_t)c * dv + j] = Sp[(size_t)c * dv + j] + kh[c] * u[j];
        for (int j = 0; j < dv; ++j) {
            double oj = 0.0;
            for (int c = 0; c < dk; ++c) oj += S[(size_t)c * dv + j] * qh[c];
            o[j] = oj;
        }
        /* 4. out = o * sigmoid(g), o = S^T qh */
        for (int j = 0; j < dv; ++j) {
            const double dy = J->d_out ? J->d_out[row * dv + j] : 0.0;
            const double sg = 1.0 / (1.0 + exp(-gt[j]));
            dov[j] = dy * sg;
            J->dg[row * dv + j] = dy * o[j] * sg * (1.0 - sg);
        }
        for (int c = 0; c < dk; ++c) {
            double acc = 0.0;
            for (int j = 0; j < dv; ++j) {
                acc += S[(size_t)c * dv + j] * dov[j];
                dS[(size_t)c * dv + j] += qh[c] * dov[j];
            }
            dqh[c] = acc;
        }
        /* 3. S = Sp + kh u^T, u = beta (v - p), p = Sp^T kh */
        for (int j = 0; j < dv; ++j) {
            double acc = 0.0;
            for (int c = 0; c < dk; ++c) acc += dS[(size_t)c * dv + j] * kh[c];
            du[j] = acc;
        }
        double db = 0.0;
        for (int j = 0; j < dv; ++j) {
            db += du[j] * (vt[j] - p[j]);
            J->dv_[row * dv + j] = bt * du[j];
            dp[j] = -bt * du[j];
        }
        J->dbeta[row] = db;
        for (int c = 0; c < dk; ++c) {
            double acc = 0.0;
            for (int j = 0; j < dv; ++j) {
                acc += dS[(size_t)c * dv + j] * u[j] + Sp[(size_t)c * dv + j] * dp[j];
                dS[(size_t)c * dv + j] += kh[c] * dp[j];      /* now the gradient w.r.t. Sp */
            }
            dkh[c] = acc;
        }
        /* 1. Sp = diag(exp(lambda)) S_prev, lambda = max(log_alpha, floor) */
        for (int c = 0; c < dk; ++c) {
            double dl = 0.0;
            for (int j = 0; j < dv; ++j) {
                dl += Sp[(size_t)c * dv + j] * dS[(size_t)c * dv + j];
                dS[(size_t)c * dv + j] *= D[c];                 /* now the gradient w.r.t. S_prev */
            }
            const double la = J->log_alpha[row * dk + c];
            J->dla[row * dk + c] = la > J->log_alpha_min ? dl : 0.0;
        }
        /* 2. normalisations */
        unit_back(kh, nk, dkh, J->dk_ + row * dk, dk);
        unit_back(qh, nq, dqh, J->dq + row * dk, dk);
    }
    if (J->d_state_in) memcpy(J->d_state_in + sb, dS, SZ * sizeof(double));
    free(hist); free(S); free(Sp); free(dS); free(work);
    return 0;
}

static void *gworker_main(void *arg)
{
    gworker_t *W = (gworker_t *)arg;
    const gjob_t *J = W->job;
    for (int64_t n = 0; n < W->count; ++n) {
        const int64_t bh = W->first + n * W->step;
        if (grad_item(J, bh / J->H, (int)(bh % J->H))) { W->status = 1; return NULL; }
    }
    return NULL;
}

/* Gradients of L = <d_out, out> + <d_state, S_T> (either may be NULL = 0).
 * Outputs have the shapes of the inputs; d_state_in may be NULL. */
int kda_oracle_grad(int64_t B, int64_t T, int H, int dk, int dv,
                    const double *q, const double *k, const double *v,
                    const double *log_alpha, const double *beta, const double *g,
                    double log_alpha_min, const double *state_in,
                    const double *d_out, const double *d_state,
                    double *dq, double *dk_, double *dv_, double *dla, double *dbeta, double *dg,
                    double *d_state_in, int nthreads)
{
    if (B < 0 || T < 0 || H <= 0 || dk <= 0 || dv <= 0) return 2;
    gjob_t J;
    memset(&J, 0, sizeof J);
    J.B = B; J.T = T; J.H = H; J.dk = dk; J.dv = dv;
    J.q = q; J.k = k; J.v = v; J.log_alpha = log_alpha; J.beta = beta; J.g = g;
    J.log_alpha_min = log_alpha_min; J.state_in = state_in; J.d_out = d_out; J.d_state = d_state;
    J.dq = dq; J.dk_ = dk_; J.dv_ = dv_; J.dla = dla; J.dbeta = dbeta; J.dg = dg; J.d_state_in = d_state_in;
    const int64_t items = B * (int64_t)H;
    if (items == 0) return 0;
    if (nthreads < 1) nthreads = 1;
    if (nthreads > items) nthreads = (int)items;
    pthread_t *th = (pthread_t *)calloc((size_t)nthreads, sizeof(pthread_t));
    gworker_t *ws = (gworker_t *)calloc((size_t)nthreads, sizeof(gworker_t));
    if (!th || !ws) { free(th); free(ws); return 1; }
    int started = 0, status = 0;
    for (int i = 0; i < nthreads; ++i) {
        ws[i].job = &J;
        ws[i].first = i;
        ws[i].step = nthreads;
        ws[i].count = (items - i + nthreads - 1) / nthreads;
        if (nthreads == 1) { gworker_main(&ws[i]); continue; }
        if (pthread_create(&th[i], NULL, gworker_main, &ws[i]) != 0) { status = 1; break; }
        ++started;
    }
    for (int i = 0; i < started; ++i) pthread_join(th[i], NULL);
    for (int i = 0; i < nthreads; ++i) status |= ws[i].status;
    free(th); free(ws);
    return status;
}
