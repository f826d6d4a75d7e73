/*
 * ttt_oracle.c -- plain, slow, fp64 CPU oracle for the TTT layer inner loop.
 *
 * TEST INFRASTRUCTURE ONLY. Only the test-suite, the smoke check and the CPU
 * baseline leg of the benchmark may load this library. It shares no code,
 * header, table or helper with the GPU path.
 *
 * Citation key (the five source pages):
 *   [D] damodev.csdn.net TTT deep-dive (TTT-Linear, inner-loop excerpt,
 *       initialisation, cache)
 *   [Y] lryc.cn "测试时学习（TTT）" article (LN-residual f, learning-rate gate,
 *       mini-batch b=16, 4x GELU MLP)
 *   [X] xiaohu.ai TTT summary (mini-batch TTT and the dual form)
 *
 * What is computed (per independent sequence (n,h)):
 *   update-then-apply, [D] §3.1 equation:
 *       W_t = W_{t-1} - eta_t * grad_W l(W_{t-1}; x_t),   o_t = f(x_t; W_t)
 *   with the reconstruction loss of [D] §4.2 (target XV - XK, forward
 *   Z = XK W + b, gradient through the fused LN + L2 backward) and the
 *   LN-residual output f(x) = x + LN(f_res(x)) of [Y] §2.1.
 *   Mini-batch TTT ([D] §4.1, [X]): the tokens of one chunk all take their
 *   gradient at the chunk-start state; the updates are then applied in token
 *   order and each token's output uses the state that includes its own update.
 *
 * Readings taken where the pages are silent:
 *   loss per token  l = 1/2 * sum_j (LN(z)_j - tau_j)^2, summed over tokens;
 *   LN uses the biased variance over the d features with eps inside the root;
 *   the same gamma/beta serve the loss and the output; row-vector convention
 *   Z = X W with W[i][j] mapping input i to output j ([D] §4.2 forward line);
 *   chunks are aligned at t = 0 and the last chunk may be partial;
 *   GELU is the exact x * Phi(x);
 *   Modular-TTT options: the inner-product loss scores the prediction
 *   f(xk) = xk + LN(f_res(xk)) against xv as -<f(xk), xv>; weight decay adds
 *   lambda/2 ||W||^2 to each token's loss for every weight matrix (W, or W1
 *   and W2 of the MLP; never a bias), its gradient taken at the chunk-start
 *   state like the rest.
 *
 * Layouts (row-major, contiguous):
 *   XQ, XK, XV, O : [B,H,L,d]         eta : [B,H,L]
 *   W0 : [H,d,d] (w0_batched = 0, shared by every n) or [B,H,d,d]
 *   b0 : [H,d] or [B,H,d]             gamma, beta : [H,d]
 *   W_out : [B,H,d,d]   b_out : [B,H,d]
 *   MLP: W1 [.,d,m], b1 [.,m], W2 [.,m,d], b2 [.,d] with m = 4d.
 *
 * Parity pins: see the oracle tests. All functions here are pinned there
 * against torch autograd / finite differences / closed forms.
 */
#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_OK 0
#define ORACLE_E_ARG (-1)
#define ORACLE_E_SCHEDULE (-2)
#define ORACLE_E_NOMEM (-3)

int oracle_version(void) { return 1; }

/* ------------------------------------------------------------------------ */
/* Layer norm over one row of d features ([Y] §2.1 LN, biased variance).      */
/* ------------------------------------------------------------------------ */
static void ln_row(int d, const double *z, const double *gamma, const double *beta,
                   double eps, double *y)
{
    double mu = 0.0, var = 0.0;
    for (int j = 0; j < d; ++j) mu += z[j];
    mu /= d;
    for (int j = 0; j < d; ++j) var += (z[j] - mu) * (z[j] - mu);
    var /= d;
    double sigma = sqrt(var + eps);
    for (int j = 0; j < d; ++j) y[j] = gamma[j] * ((z[j] - mu) / sigma) + beta[j];
}

/*
 * Gradient of l(z) = 1/2 * || LN_{gamma,beta}(z) - tau ||^2 with respect to z
 * (the "ln_fused_l2_bwd" step of [D] §4.2): layer-norm forward, L2 backward,
 * layer-norm backward.
 *   xh = (z - mu)/sigma,  y = gamma*xh + beta,  g = y - tau,  gh = gamma*g
 *   dl/dz = (gh - mean(gh) - xh * mean(gh*xh)) / sigma
 */
static void ln_l2_grad_row(int d, const double *z, const double *tau,
                           const double *gamma, const double *beta, double eps,
                           double *G)
{
    double mu = 0.0, var = 0.0;
    for (int j = 0; j < d; ++j) mu += z[j];
    mu /= d;
    for (int j = 0; j < d; ++j) var += (z[j] - mu) * (z[j] - mu);
    var /= d;
    double sigma = sqrt(var + eps);
    double m1 = 0.0, m2 = 0.0;
    for (int j = 0; j < d; ++j) {
        double xh = (z[j] - mu) / sigma;
        double y = gamma[j] * xh + beta[j];
        double gh = gamma[j] * (y - tau[j]);
        m1 += gh;
        m2 += gh * xh;
    }
    m1 /= d;
    m2 /= d;
    for (int j = 0; j < d; ++j) {
        double xh = (z[j] - mu) / sigma;
        double y = gamma[j] * xh + beta[j];
        double gh = gamma[j] * (y - tau[j]);
        G[j] = (gh - m1 - xh * m2) / sigma;
    }
}

/*
 * Gradient of the inner-product loss l(z) = -< x + LN_{gamma,beta}(z), v >
 * (the prediction f(x) = x + LN(z) scored against the target v by an inner
 * product instead of a squared distance, the loss alternative named on the
 * Modular-TTT page) with respect to z: the upstream gradient dl/dy is -v, so
 *   gh = -gamma*v,  dl/dz = (gh - mean(gh) - xh * mean(gh*xh)) / sigma.
 * (x does not depend on z; beta drops out.)
 */
static void ln_ip_grad_row(int d, const double *z, const double *v,
                           const double *gamma, double eps, double *G)
{
    double mu = 0.0, var = 0.0;
    for (int j = 0; j < d; ++j) mu += z[j];
    mu /= d;
    for (int j = 0; j < d; ++j) var += (z[j] - mu) * (z[j] - mu);
    var /= d;
    double sigma = sqrt(var + eps);
    double m1 = 0.0, m2 = 0.0;
    for (int j = 0; j < d; ++j) {
        double xh = (z[j] - mu) / sigma;
        double gh = -gamma[j] * v[j];
        m1 += gh;
        m2 += gh * xh;
    }
    m1 /= d;
    m2 /= d;
    for (int j = 0; j < d; ++j) {
        double xh = (z[j] - mu) / sigma;
        double gh = -gamma[j] * v[j];
        G[j] = (gh - m1 - xh * m2) / sigma;
    }
}

void oracle_ln_fwd(int rows, int d, const double *Z, const double *gamma,
                   const double *beta, double eps, double *Y)
{
    for (int r = 0; r < rows; ++r)
        ln_row(d, Z + (size_t)r * d, gamma, beta, eps, Y + (size_t)r * d);
}

/* rows x d gradient; `target` is tau directly (the caller forms XV - XK). */
void oracle_ln_l2_bwd(int rows, int d, const double *Z, const double *target,
                      const double *gamma, const double *beta, double eps, double *G)
{
    for (int r = 0; r < rows; ++r)
        ln_l2_grad_row(d, Z + (size_t)r * d, target + (size_t)r * d, gamma, beta,
                       eps, G + (size_t)r * d);
}

/* ------------------------------------------------------------------------ */
/* GELU (exact, x * Phi(x)) and its derivative ([Y] §2.1 "GELU").             */
/* ------------------------------------------------------------------------ */
static double gelu(double x) { return 0.5 * x * (1.0 + erf(x / sqrt(2.0))); }
static double gelu_prime(double x)
{
    double Phi = 0.5 * (1.0 + erf(x / sqrt(2.0)));
    double phi = exp(-0.5 * x * x) / sqrt(2.0 * M_PI);
    return Phi + x * phi;
}

/* ------------------------------------------------------------------------ */
/* Work distribution over independent (n,h) sequences.                        */
/* ------------------------------------------------------------------------ */
typedef struct {
    int B, H, L, d;
    int nchunks;
    const int *chunk_len;
    int max_chunk;
    double eps;
    const double *XQ, *XK, *XV, *eta;
    const double *W0, *b0, *W2_0, *b2_0; /* Linear: W0,b0. MLP: W1_0,b1_0,W2_0,b2_0 */
    int w0_batched;
    const double *gamma, *beta;
    double *O, *W_out, *b_out, *W2_out, *b2_out;
    int loss;      /* 0 = squared error (the default), 1 = inner product        */
    double wd;     /* weight decay lambda on the weight matrices (0 = none)     */
    int nthreads;
    int tid;
    int status;
} job_t;

typedef void (*seq_fn)(job_t *, int n, int h, double *scratch);

typedef struct {
    job_t *job;
    seq_fn fn;
    size_t scratch_doubles;
} pool_arg_t;

static void *pool_worker(void *p)
{
    pool_arg_t *a = (pool_arg_t *)p;
    job_t *j = a->job;
    double *scratch = (double *)malloc(a->scratch_doubles * sizeof(double));
    if (!scratch) {
        j->status = ORACLE_E_NOMEM;
        return NULL;
    }
    for (int s = j->tid; s < j->B * j->H; s += j->nthreads)
        a->fn(j, s / j->H, s % j->H, scratch);
    free(scratch);
    return NULL;
}

static int run_pool(const job_t *proto, seq_fn fn, size_t scratch_doubles)
{
    int nt = proto->nthreads < 1 ? 1 : proto->nthreads;
    int nseq = proto->B * proto->H;
    if (nt > nseq) nt = nseq;
    if (nseq == 0) return ORACLE_OK;
    job_t *jobs = (job_t *)calloc((size_t)nt, sizeof(job_t));
    pool_arg_t *args = (pool_arg_t *)calloc((size_t)nt, sizeof(pool_arg_t));
    pthread_t *th = (pthread_t *)calloc((size_t)nt, sizeof(pthread_t));
    if (!jobs || !args || !th) {
        free(jobs); free(args); free(th);
        return ORACLE_E_NOMEM;
    }
    for (int t = 0; t < nt; ++t) {
        jobs[t] = *proto;
        jobs[t].nthreads = nt;
        jobs[t].tid = t;
        jobs[t].status = ORACLE_OK;
        args[t].job = &jobs[t];
        args[t].fn = fn;
        args[t].scratch_doubles = scratch_doubles;
    }
    for (int t = 1; t < nt; ++t) pthread_create(&th[t], NULL, pool_worker, &args[t]);
    pool_worker(&args[0]);
    for (int t = 1; t < nt; ++t) pthread_join(th[t], NULL);
    int st = ORACLE_OK;
    for (int t = 0; t < nt; ++t)
        if (jobs[t].status != ORACLE_OK) st = jobs[t].status;
    free(jobs); free(args); free(th);
    return st;
}

static int check_schedule(int L, int nchunks, const int *chunk_len, int *max_chunk)
{
    if (nchunks < 0 || (nchunks > 0 && !chunk_len)) return ORACLE_E_SCHEDULE;
    long long sum = 0;
    int mx = 1;
    for (int c = 0; c < nchunks; ++c) {
        if (chunk_len[c] <= 0) return ORACLE_E_SCHEDULE;
        sum += chunk_len[c];
        if (chunk_len[c] > mx) mx = chunk_len[c];
    }
    if (sum != L) return ORACLE_E_SCHEDULE;
    *max_chunk = mx;
    return ORACLE_OK;
}

/* ------------------------------------------------------------------------ */
/* TTT-Linear, primal mini-batch form.                                        */
/* ------------------------------------------------------------------------ */
static void linear_primal_seq(job_t *j, int n, int h, double *scratch)
{
    const int d = j->d, L = j->L, H = j->H;
    const size_t seq = (size_t)n * H + h;
    const double *xq = j->XQ + seq * L * d, *xk = j->XK + seq * L * d;
    const double *xv = j->XV + seq * L * d, *eta = j->eta + seq * L;
    const double *gamma = j->gamma + (size_t)h * d, *beta = j->beta + (size_t)h * d;
    double *o = j->O + seq * L * d;

    double *W = scratch;                    /* d*d                        */
    double *b = W + (size_t)d * d;          /* d                          */
    double *G = b + d;                      /* max_chunk * d              */
    double *z = G + (size_t)j->max_chunk * d; /* d                        */
    double *tau = z + d;                    /* d                          */
    double *y = tau + d;                    /* d                          */
    double *Wc = y + d;                     /* d*d: chunk-start W (decay)  */

    const size_t w_off = (j->w0_batched ? (size_t)n * H * d * d : 0) + (size_t)h * d * d;
    const size_t b_off = (j->w0_batched ? (size_t)n * H * d : 0) + (size_t)h * d;
    memcpy(W, j->W0 + w_off, sizeof(double) * d * d);
    memcpy(b, j->b0 + b_off, sizeof(double) * d);

    int t0 = 0;
    for (int c = 0; c < j->nchunks; ++c) {
        const int len = j->chunk_len[c];
        /* gradients of every token of the chunk at the chunk-start W, b */
        for (int s = 0; s < len; ++s) {
            const double *k = xk + (size_t)(t0 + s) * d, *v = xv + (size_t)(t0 + s) * d;
            for (int jj = 0; jj < d; ++jj) {
                double acc = b[jj];
                for (int i = 0; i < d; ++i) acc += k[i] * W[(size_t)i * d + jj];
                z[jj] = acc;
                tau[jj] = v[jj] - k[jj];     /* reconstruction target XV - XK */
            }
            if (j->loss == 1)
                ln_ip_grad_row(d, z, v, gamma, j->eps, G + (size_t)s * d);
            else
                ln_l2_grad_row(d, z, tau, gamma, beta, j->eps, G + (size_t)s * d);
        }
        /* weight decay: each token's gradient also carries lambda * W at the
           chunk-start state (the gradient of lambda/2 ||W||^2 there) */
        if (j->wd != 0.0) memcpy(Wc, W, sizeof(double) * d * d);
        /* token order: update with the token's own gradient, then apply */
        for (int s = 0; s < len; ++s) {
            const int t = t0 + s;
            const double *k = xk + (size_t)t * d, *q = xq + (size_t)t * d;
            const double *g = G + (size_t)s * d;
            const double e = eta[t];
            for (int i = 0; i < d; ++i)
                for (int jj = 0; jj < d; ++jj) {
                    double gw = k[i] * g[jj];
                    if (j->wd != 0.0) gw += j->wd * Wc[(size_t)i * d + jj];
                    W[(size_t)i * d + jj] -= e * gw;
                }
            for (int jj = 0; jj < d; ++jj) b[jj] -= e * g[jj];
            for (int jj = 0; jj < d; ++jj) {
                double acc = b[jj];
                for (int i = 0; i < d; ++i) acc += q[i] * W[(size_t)i * d + jj];
                z[jj] = acc;
            }
            ln_row(d, z, gamma, beta, j->eps, y);
            for (int jj = 0; jj < d; ++jj) o[(size_t)t * d + jj] = q[jj] + y[jj];
        }
        t0 += len;
    }
    if (j->W_out) memcpy(j->W_out + seq * d * d, W, sizeof(double) * d * d);
    if (j->b_out) memcpy(j->b_out + seq * d, b, sizeof(double) * d);
}

int oracle_linear_forward(int B, int H, int L, int d, int nchunks, const int *chunk_len,
                          double eps, const double *XQ, const double *XK, const double *XV,
                          const double *eta, const double *W0, const double *b0,
                          int w0_batched, const double *gamma, const double *beta,
                          double *O, double *W_out, double *b_out, int nthreads)
{
    if (B < 0 || H < 0 || L < 0 || d <= 0) return ORACLE_E_ARG;
    job_t j;
    memset(&j, 0, sizeof j);
    int st = check_schedule(L, nchunks, chunk_len, &j.max_chunk);
    if (st) return st;
    j.B = B; j.H = H; j.L = L; j.d = d; j.nchunks = nchunks; j.chunk_len = chunk_len;
    j.eps = eps; j.XQ = XQ; j.XK = XK; j.XV = XV; j.eta = eta; j.W0 = W0; j.b0 = b0;
    j.w0_batched = w0_batched; j.gamma = gamma; j.beta = beta; j.O = O;
    j.W_out = W_out; j.b_out = b_out; j.nthreads = nthreads;
    size_t scratch = 2 * (size_t)d * d + (size_t)d * (4 + j.max_chunk);
    return run_pool(&j, linear_primal_seq, scratch);
}

/*
 * TTT-Linear with the Modular-TTT design choices as options: loss = 0 is the
 * squared reconstruction error above, loss = 1 the inner-product loss
 * -< x + LN(x W + b), v > (ln_ip_grad_row); weight_decay = lambda adds
 * lambda/2 ||W||^2 to every token's loss (W only, the bias is not decayed).
 * Mini-batch rule as before: every gradient, decay term included, is taken at
 * the chunk-start state.
 */
int oracle_linear_forward_opts(int B, int H, int L, int d, int nchunks, const int *chunk_len,
                               double eps, const double *XQ, const double *XK,
                               const double *XV, const double *eta, const double *W0,
                               const double *b0, int w0_batched, const double *gamma,
                               const double *beta, int loss, double weight_decay, double *O,
                               double *W_out, double *b_out, int nthreads)
{
    if (B < 0 || H < 0 || L < 0 || d <= 0 || (loss != 0 && loss != 1)) return ORACLE_E_ARG;
    job_t j;
    memset(&j, 0, sizeof j);
    int st = check_schedule(L, nchunks, chunk_len, &j.max_chunk);
    if (st) return st;
    j.B = B; j.H = H; j.L = L; j.d = d; j.nchunks = nchunks; j.chunk_len = chunk_len;
    j.eps = eps; j.XQ = XQ; j.XK = XK; j.XV = XV; j.eta = eta; j.W0 = W0; j.b0 = b0;
    j.w0_batched = w0_batched; j.gamma = gamma; j.beta = beta; j.O = O;
    j.W_out = W_out; j.b_out = b_out; j.nthreads = nthreads;
    j.loss = loss; j.wd = weight_decay;
    size_t scratch = 2 * (size_t)d * d + (size_t)d * (4 + j.max_chunk);
    return run_pool(&j, linear_primal_seq, scratch);
}

/* ------------------------------------------------------------------------ */
/* TTT-Linear, dual form ([D] §4.2 dual branch; [X] "dual form").             */
/* Same function as the primal form in exact arithmetic; used to pin it.      */
/*   per chunk: Z = XK W + b;  G = lnbwd(Z, XV - XK)                         */
/*   Zbar_t = xq_t W + b - sum_{s<=t} eta_s (xq_t . xk_s + 1) G_s            */
/*   W' = W - (eta * XK)^T G;   b' = b - eta^T G                             */
/* ------------------------------------------------------------------------ */
static void linear_dual_seq(job_t *j, int n, int h, double *scratch)
{
    const int d = j->d, L = j->L, H = j->H;
    const size_t seq = (size_t)n * H + h;
    const double *xq = j->XQ + seq * L * d, *xk = j->XK + seq * L * d;
    const double *xv = j->XV + seq * L * d, *eta = j->eta + seq * L;
    const double *gamma = j->gamma + (size_t)h * d, *beta = j->beta + (size_t)h * d;
    double *o = j->O + seq * L * d;
    const int mc = j->max_chunk;

    double *W = scratch, *b = W + (size_t)d * d, *G = b + d;
    double *Zb = G + (size_t)mc * d, *z = Zb + (size_t)mc * d, *tau = z + d, *y = tau + d;

    const size_t w_off = (j->w0_batched ? (size_t)n * H * d * d : 0) + (size_t)h * d * d;
    const size_t b_off = (j->w0_batched ? (size_t)n * H * d : 0) + (size_t)h * d;
    memcpy(W, j->W0 + w_off, sizeof(double) * d * d);
    memcpy(b, j->b0 + b_off, sizeof(double) * d);

    int t0 = 0;
    for (int c = 0; c < j->nchunks; ++c) {
        const int len = j->chunk_len[c];
        for (int s = 0; s < len; ++s) {
            const double *k = xk + (size_t)(t0 + s) * d, *v = xv + (size_t)(t0 + s) * d;
            for (int jj = 0; jj < d; ++jj) {
                double acc = b[jj];
                for (int i = 0; i < d; ++i) acc += k[i] * W[(size_t)i * d + jj];
                z[jj] = acc;
                tau[jj] = v[jj] - k[jj];
            }
            ln_l2_grad_row(d, z, tau, gamma, beta, j->eps, G + (size_t)s * d);
        }
        for (int t = 0; t < len; ++t) {
            const double *q = xq + (size_t)(t0 + t) * d;
            for (int jj = 0; jj < d; ++jj) {
                double acc = b[jj];
                for (int i = 0; i < d; ++i) acc += q[i] * W[(size_t)i * d + jj];
                Zb[(size_t)t * d + jj] = acc;
            }
            for (int s = 0; s <= t; ++s) {
                const double *k = xk + (size_t)(t0 + s) * d;
                double a = 0.0;
                for (int i = 0; i < d; ++i) a += q[i] * k[i];
                const double m = eta[t0 + s] * (a + 1.0);
                for (int jj = 0; jj < d; ++jj) Zb[(size_t)t * d + jj] -= m * G[(size_t)s * d + jj];
            }
        }
        for (int t = 0; t < len; ++t) {
            ln_row(d, Zb + (size_t)t * d, gamma, beta, j->eps, y);
            const double *q = xq + (size_t)(t0 + t) * d;
            for (int jj = 0; jj < d; ++jj) o[(size_t)(t0 + t) * d + jj] = q[jj] + y[jj];
        }
        for (int i = 0; i < d; ++i)
            for (int jj = 0; jj < d; ++jj) {
                double acc = 0.0;
                for (int s = 0; s < len; ++s)
                    acc += eta[t0 + s] * xk[(size_t)(t0 + s) * d + i] * G[(size_t)s * d + jj];
                W[(size_t)i * d + jj] -= acc;
            }
        for (int jj = 0; jj < d; ++jj) {
            double acc = 0.0;
            for (int s = 0; s < len; ++s) acc += eta[t0 + s] * G[(size_t)s * d + jj];
            b[jj] -= acc;
        }
        t0 += len;
    }
    if (j->W_out) memcpy(j->W_out + seq * d * d, W, sizeof(double) * d * d);
    if (j->b_out) memcpy(j->b_out + seq * d, b, sizeof(double) * d);
}

int oracle_linear_dual(int B, int H, int L, int d, int nchunks, const int *chunk_len,
                       double eps, const double *XQ, const double *XK, const double *XV,
                       const double *eta, const double *W0, const double *b0, int w0_batched,
                       const double *gamma, const double *beta, double *O, double *W_out,
                       double *b_out, int nthreads)
{
    if (B < 0 || H < 0 || L < 0 || d <= 0) return ORACLE_E_ARG;
    job_t j;
    memset(&j, 0, sizeof j);
    int st = check_schedule(L, nchunks, chunk_len, &j.max_chunk);
    if (st) return st;
    j.B = B; j.H = H; j.L = L; j.d = d; j.nchunks = nchunks; j.chunk_len = chunk_len;
    j.eps = eps; j.XQ = XQ; j.XK = XK; j.XV = XV; j.eta = eta; j.W0 = W0; j.b0 = b0;
    j.w0_batched = w0_batched; j.gamma = gamma; j.beta = beta; j.O = O;
    j.W_out = W_out; j.b_out = b_out; j.nthreads = nthreads;
    size_t scratch = (size_t)d * d + (size_t)d * (4 + 2 * (size_t)j.max_chunk);
    return run_pool(&j, linear_dual_seq, scratch);
}

/* ------------------------------------------------------------------------ */
/* TTT-MLP, primal mini-batch form ([Y] §2.1: d -> 4d GELU -> d, LN residual) */
/*   chunk-start forward: z1 = xk W1 + b1, a = gelu(z1), z2 = a W2 + b2       */
/*   G2 = lnbwd(z2, xv - xk),  G1 = (G2 W2^T) * gelu'(z1)                     */
/*   per token in order: W1 -= eta xk^T G1, b1 -= eta G1,                     */
/*                       W2 -= eta a^T G2,  b2 -= eta G2,                      */
/*                       o = xq + LN(gelu(xq W1 + b1) W2 + b2)                */
/* ------------------------------------------------------------------------ */
static void mlp_primal_seq(job_t *j, int n, int h, double *scratch)
{
    const int d = j->d, L = j->L, H = j->H, m = 4 * d;
    const size_t seq = (size_t)n * H + h;
    const double *xq = j->XQ + seq * L * d, *xk = j->XK + seq * L * d;
    const double *xv = j->XV + seq * L * d, *eta = j->eta + seq * L;
    const double *gamma = j->gamma + (size_t)h * d, *beta = j->beta + (size_t)h * d;
    double *o = j->O + seq * L * d;
    const int mc = j->max_chunk;

    double *W1 = scratch;
    double *b1 = W1 + (size_t)d * m;
    double *W2 = b1 + m;
    double *b2 = W2 + (size_t)m * d;
    double *A = b2 + d;                 /* mc x m  activations a_s       */
    double *G1 = A + (size_t)mc * m;    /* mc x m                        */
    double *G2 = G1 + (size_t)mc * m;   /* mc x d                        */
    double *z1 = G2 + (size_t)mc * d;   /* m                             */
    double *a = z1 + m;                 /* m                             */
    double *z2 = a + m;                 /* d                             */
    double *tau = z2 + d;               /* d                             */
    double *y = tau + d;                /* d                             */
    double *W1c = y + d;                /* d x m: chunk-start W1 (decay) */
    double *W2c = W1c + (size_t)d * m;  /* m x d: chunk-start W2 (decay) */

    const size_t bn = j->w0_batched ? (size_t)n : 0;
    memcpy(W1, j->W0 + (bn * H + h) * (size_t)d * m, sizeof(double) * d * m);
    memcpy(b1, j->b0 + (bn * H + h) * (size_t)m, sizeof(double) * m);
    memcpy(W2, j->W2_0 + (bn * H + h) * (size_t)m * d, sizeof(double) * m * d);
    memcpy(b2, j->b2_0 + (bn * H + h) * (size_t)d, sizeof(double) * d);

    int t0 = 0;
    for (int c = 0; c < j->nchunks; ++c) {
        const int len = j->chunk_len[c];
        for (int s = 0; s < len; ++s) {
            const double *k = xk + (size_t)(t0 + s) * d, *v = xv + (size_t)(t0 + s) * d;
            for (int q = 0; q < m; ++q) {
                double acc = b1[q];
                for (int i = 0; i < d; ++i) acc += k[i] * W1[(size_t)i * m + q];
                z1[q] = acc;
                A[(size_t)s * m + q] = gelu(acc);
            }
            for (int jj = 0; jj < d; ++jj) {
                double acc = b2[jj];
                for (int q = 0; q < m; ++q) acc += A[(size_t)s * m + q] * W2[(size_t)q * d + jj];
                z2[jj] = acc;
                tau[jj] = v[jj] - k[jj];
            }
            if (j->loss == 1)
                ln_ip_grad_row(d, z2, v, gamma, j->eps, G2 + (size_t)s * d);
            else
                ln_l2_grad_row(d, z2, tau, gamma, beta, j->eps, G2 + (size_t)s * d);
            for (int q = 0; q < m; ++q) {
                double acc = 0.0;
                for (int jj = 0; jj < d; ++jj) acc += G2[(size_t)s * d + jj] * W2[(size_t)q * d + jj];
                G1[(size_t)s * m + q] = acc * gelu_prime(z1[q]);
            }
        }
        /* weight decay: lambda * W1 and lambda * W2 at the chunk-start state
           join every token's gradient (the biases are not decayed) */
        if (j->wd != 0.0) {
            memcpy(W1c, W1, sizeof(double) * d * m);
            memcpy(W2c, W2, sizeof(double) * m * d);
        }
        for (int s = 0; s < len; ++s) {
            const int t = t0 + s;
            const double *k = xk + (size_t)t * d, *qv = xq + (size_t)t * d;
            const double e = eta[t];
            const double *g1 = G1 + (size_t)s * m, *g2 = G2 + (size_t)s * d, *as = A + (size_t)s * m;
            for (int i = 0; i < d; ++i)
                for (int q = 0; q < m; ++q) {
                    double gw = k[i] * g1[q];
                    if (j->wd != 0.0) gw += j->wd * W1c[(size_t)i * m + q];
                    W1[(size_t)i * m + q] -= e * gw;
                }
            for (int q = 0; q < m; ++q) b1[q] -= e * g1[q];
            for (int q = 0; q < m; ++q)
                for (int jj = 0; jj < d; ++jj) {
                    double gw = as[q] * g2[jj];
                    if (j->wd != 0.0) gw += j->wd * W2c[(size_t)q * d + jj];
                    W2[(size_t)q * d + jj] -= e * gw;
                }
            for (int jj = 0; jj < d; ++jj) b2[jj] -= e * g2[jj];
            for (int q = 0; q < m; ++q) {
                double acc = b1[q];
                for (int i = 0; i < d; ++i) acc += qv[i] * W1[(size_t)i * m + q];
                a[q] = gelu(acc);
            }
            for (int jj = 0; jj < d; ++jj) {
                double acc = b2[jj];
                for (int q = 0; q < m; ++q) acc += a[q] * W2[(size_t)q * d + jj];
                z2[jj] = acc;
            }
            ln_row(d, z2, gamma, beta, j->eps, y);
            for (int jj = 0; jj < d; ++jj) o[(size_t)t * d + jj] = qv[jj] + y[jj];
        }
        t0 += len;
    }
    if (j->W_out) memcpy(j->W_out + seq * d * m, W1, sizeof(double) * d * m);
    if (j->b_out) memcpy(j->b_out + seq * m, b1, sizeof(double) * m);
    if (j->W2_out) memcpy(j->W2_out + seq * m * d, W2, sizeof(double) * m * d);
    if (j->b2_out) memcpy(j->b2_out + seq * d, b2, sizeof(double) * d);
}

int oracle_mlp_forward(int B, int H, int L, int d, int nchunks, const int *chunk_len,
                       double eps, const double *XQ, const double *XK, const double *XV,
                       const double *eta, const double *W1_0, const double *b1_0,
                       const double *W2_0, const double *b2_0, int w0_batched,
                       const double *gamma, const double *beta, double *O,
                       double *W1_out, double *b1_out, double *W2_out, double *b2_out,
                       int nthreads)
{
    if (B < 0 || H < 0 || L < 0 || d <= 0) return ORACLE_E_ARG;
    job_t j;
    memset(&j, 0, sizeof j);
    int st = check_schedule(L, nchunks, chunk_len, &j.max_chunk);
    if (st) return st;
    j.B = B; j.H = H; j.L = L; j.d = d; j.nchunks = nchunks; j.chunk_len = chunk_len;
    j.eps = eps; j.XQ = XQ; j.XK = XK; j.XV = XV; j.eta = eta;
    j.W0 = W1_0; j.b0 = b1_0; j.W2_0 = W2_0; j.b2_0 = b2_0; j.w0_batched = w0_batched;
    j.gamma = gamma; j.beta = beta; j.O = O;
    j.W_out = W1_out; j.b_out = b1_out; j.W2_out = W2_out; j.b2_out = b2_out;
    j.nthreads = nthreads;
    const size_t m = 4 * (size_t)d;
    size_t scratch = 4 * (size_t)d * m + m + d + (size_t)j.max_chunk * (2 * m + d) + 2 * m + 3 * (size_t)d;
    return run_pool(&j, mlp_primal_seq, scratch);
}

/*
 * TTT-MLP with the same Modular-TTT options as TTT-Linear: loss = 1 scores
 * x + LN(f_res(x)) against v by -< ., v > (ln_ip_grad_row at the second
 * layer's output); weight_decay = lambda adds lambda/2 (||W1||^2 + ||W2||^2)
 * to every token's loss (the biases b1, b2 are not decayed). Every gradient,
 * the decay term included, is taken at the chunk-start state.
 */
int oracle_mlp_forward_opts(int B, int H, int L, int d, int nchunks, const int *chunk_len,
                            double eps, const double *XQ, const double *XK, const double *XV,
                            const double *eta, const double *W1_0, const double *b1_0,
                            const double *W2_0, const double *b2_0, int w0_batched,
                            const double *gamma, const double *beta, int loss,
                            double weight_decay, double *O, double *W1_out, double *b1_out,
                            double *W2_out, double *b2_out, int nthreads)
{
    if (B < 0 || H < 0 || L < 0 || d <= 0 || (loss != 0 && loss != 1)) return ORACLE_E_ARG;
    job_t j;
    memset(&j, 0, sizeof j);
    int st = check_schedule(L, nchunks, chunk_len, &j.max_chunk);
    if (st) return st;
    j.B = B; j.H = H; j.L = L; j.d = d; j.nchunks = nchunks; j.chunk_len = chunk_len;
    j.eps = eps; j.XQ = XQ; j.XK = XK; j.XV = XV; j.eta = eta;
    j.W0 = W1_0; j.b0 = b1_0; j.W2_0 = W2_0; j.b2_0 = b2_0; j.w0_batched = w0_batched;
    j.gamma = gamma; j.beta = beta; j.O = O;
    j.W_out = W1_out; j.b_out = b1_out; j.W2_out = W2_out; j.b2_out = b2_out;
    j.nthreads = nthreads;
    j.loss = loss; j.wd = weight_decay;
    const size_t m = 4 * (size_t)d;
    size_t scratch = 4 * (size_t)d * m + m + d + (size_t)j.max_chunk * (2 * m + d) + 2 * m + 3 * (size_t)d;
    return run_pool(&j, mlp_primal_seq, scratch);
}

/* ------------------------------------------------------------------------ */
/* TTT-MLP, dual form. Same function as the primal form in exact arithmetic. */
/*   Zbar1_t = xq_t W1 + b1 - sum_{s<=t} eta_s (xq_t . xk_s + 1) G1_s         */
/*   abar_t  = gelu(Zbar1_t)                                                  */
/*   Zbar2_t = abar_t W2 + b2 - sum_{s<=t} eta_s (abar_t . a_s + 1) G2_s      */
/*   then the chunk's summed update of W1, b1, W2, b2.                        */
/* ------------------------------------------------------------------------ */
static void mlp_dual_seq(job_t *j, int n, int h, double *scratch)
{
    const int d = j->d, L = j->L, H = j->H, m = 4 * d;
    const size_t seq = (size_t)n * H + h;
    const double *xq = j->XQ + seq * L * d, *xk = j->XK + seq * L * d;
    const double *xv = j->XV + seq * L * d, *eta = j->eta + seq * L;
    const double *gamma = j->gamma + (size_t)h * d, *beta = j->beta + (size_t)h * d;
    double *o = j->O + seq * L * d;
    const int mc = j->max_chunk;

    double *W1 = scratch;
    double *b1 = W1 + (size_t)d * m;
    double *W2 = b1 + m;
    double *b2 = W2 + (size_t)m * d;
    double *A = b2 + d;
    double *G1 = A + (size_t)mc * m;
    double *G2 = G1 + (size_t)mc * m;
    double *Ab = G2 + (size_t)mc * d;   /* mc x m : abar */
    double *z1 = Ab + (size_t)mc * m;
    double *z2 = z1 + m;
    double *tau = z2 + d;
    double *y = tau + d;

    const size_t bn = j->w0_batched ? (size_t)n : 0;
    memcpy(W1, j->W0 + (bn * H + h) * (size_t)d * m, sizeof(double) * d * m);
    memcpy(b1, j->b0 + (bn * H + h) * (size_t)m, sizeof(double) * m);
    memcpy(W2, j->W2_0 + (bn * H + h) * (size_t)m * d, sizeof(double) * m * d);
    memcpy(b2, j->b2_0 + (bn * H + h) * (size_t)d, sizeof(double) * d);

    int t0 = 0;
    for (int c = 0; c < j->nchunks; ++c) {
        const int len = j->chunk_len[c];
        for (int s = 0; s < len; ++s) {
            const double *k = xk + (size_t)(t0 + s) * d, *v = xv + (size_t)(t0 + s) * d;
            for (int q = 0; q < m; ++q) {
                double acc = b1[q];
                for (int i = 0; i < d; ++i) acc += k[i] * W1[(size_t)i * m + q];
                z1[q] = acc;
                A[(size_t)s * m + q] = gelu(acc);
            }
            for (int jj = 0; jj < d; ++jj) {
                double acc = b2[jj];
                for (int q = 0; q < m; ++q) acc += A[(size_t)s * m + q] * W2[(size_t)q * d + jj];
                z2[jj] = acc;
                tau[jj] = v[jj] - k[jj];
            }
            if (j->loss == 1)
                ln_ip_grad_row(d, z2, v, gamma, j->eps, G2 + (size_t)s * d);
            else
                ln_l2_grad_row(d, z2, tau, gamma, beta, j->eps, G2 + (size_t)s * d);
            for (int q = 0; q < m; ++q) {
                double acc = 0.0;
                for (int jj = 0; jj < d; ++jj) acc += G2[(size_t)s * d + jj] * W2[(size_t)q * d + jj];
                G1[(size_t)s * m + q] = acc * gelu_prime(z1[q]);
            }
        }
        for (int t = 0; t < len; ++t) {
            const double *qv = xq + (size_t)(t0 + t) * d;
            for (int q = 0; q < m; ++q) {
                double acc = b1[q];
                for (int i = 0; i < d; ++i) acc += qv[i] * W1[(size_t)i * m + q];
                z1[q] = acc;
            }
            for (int s = 0; s <= t; ++s) {
                const double *k = xk + (size_t)(t0 + s) * d;
                double dot = 0.0;
                for (int i = 0; i < d; ++i) dot += qv[i] * k[i];
                const double mm = eta[t0 + s] * (dot + 1.0);
                for (int q = 0; q < m; ++q) z1[q] -= mm * G1[(size_t)s * m + q];
            }
            for (int q = 0; q < m; ++q) Ab[(size_t)t * m + q] = gelu(z1[q]);
            for (int jj = 0; jj < d; ++jj) {
                double acc = b2[jj];
                for (int q = 0; q < m; ++q) acc += Ab[(size_t)t * m + q] * W2[(size_t)q * d + jj];
                z2[jj] = acc;
            }
            for (int s = 0; s <= t; ++s) {
                double dot = 0.0;
                for (int q = 0; q < m; ++q) dot += Ab[(size_t)t * m + q] * A[(size_t)s * m + q];
                const double mm = eta[t0 + s] * (dot + 1.0);
                for (int jj = 0; jj < d; ++jj) z2[jj] -= mm * G2[(size_t)s * d + jj];
            }
            ln_row(d, z2, gamma, beta, j->eps, y);
            for (int jj = 0; jj < d; ++jj) o[(size_t)(t0 + t) * d + jj] = qv[jj] + y[jj];
        }
        for (int i = 0; i < d; ++i)
            for (int q = 0; q < m; ++q) {
                double acc = 0.0;
                for (int s = 0; s < len; ++s)
                    acc += eta[t0 + s] * xk[(size_t)(t0 + s) * d + i] * G1[(size_t)s * m + q];
                W1[(size_t)i * m + q] -= acc;
            }
        for (int q = 0; q < m; ++q) {
            double acc = 0.0;
            for (int s = 0; s < len; ++s) acc += eta[t0 + s] * G1[(size_t)s * m + q];
            b1[q] -= acc;
        }
        for (int q = 0; q < m; ++q)
            for (int jj = 0; jj < d; ++jj) {
                double acc = 0.0;
                for (int s = 0; s < len; ++s)
                    acc += eta[t0 + s] * A[(size_t)s * m + q] * G2[(size_t)s * d + jj];
                W2[(size_t)q * d + jj] -= acc;
            }
        for (int jj = 0; jj < d; ++jj) {
            double acc = 0.0;
            for (int s = 0; s < len; ++s) acc += eta[t0 + s] * G2[(size_t)s * d + jj];
            b2[jj] -= acc;
        }
        t0 += len;
    }
    if (j->W_out) memcpy(j->W_out + seq * d * m, W1, sizeof(double) * d * m);
    if (j->b_out) memcpy(j->b_out + seq * m, b1, sizeof(double) * m);
    if (j->W2_out) memcpy(j->W2_out + seq * m * d, W2, sizeof(double) * m * d);
    if (j->b2_out) memcpy(j->b2_out + seq * d, b2, sizeof(double) * d);
}

int oracle_mlp_dual(int B, int H, int L, int d, int nchunks, const int *chunk_len,
                    double eps, const double *XQ, const double *XK, const double *XV,
                    const double *eta, const double *W1_0, const double *b1_0,
                    const double *W2_0, const double *b2_0, int w0_batched,
                    const double *gamma, const double *beta, double *O,
                    double *W1_out, double *b1_out, double *W2_out, double *b2_out,
                    int nthreads)
{
    if (B < 0 || H < 0 || L < 0 || d <= 0) return ORACLE_E_ARG;
    job_t j;
    memset(&j, 0, sizeof j);
    int st = check_schedule(L, nchunks, chunk_len, &j.max_chunk);
    if (st) return st;
    j.B = B; j.H = H; j.L = L; j.d = d; j.nchunks = nchunks; j.chunk_len = chunk_len;
    j.eps = eps; j.XQ = XQ; j.XK = XK; j.XV = XV; j.eta = eta;
    j.W0 = W1_0; j.b0 = b1_0; j.W2_0 = W2_0; j.b2_0 = b2_0; j.w0_batched = w0_batched;
    j.gamma = gamma; j.beta = beta; j.O = O;
    j.W_out = W1_out; j.b_out = b1_out; j.W2_out = W2_out; j.b2_out = b2_out;
    j.nthreads = nthreads;
    const size_t m = 4 * (size_t)d;
    size_t scratch = 2 * (size_t)d * m + m + d + (size_t)j.max_chunk * (3 * m + d) + m + 3 * (size_t)d;
    return run_pool(&j, mlp_dual_seq, scratch);
}

/*
 * Input projections of the layer ([Y] §2.2: the outer loop learns the
 * projections theta_K, theta_V, theta_Q that make the key, value and query
 * views of each token; [D] §4.2 feeds those views, XK, XV, XQ, to the inner
 * loop). Reading taken where the pages are silent: each view is a linear map
 * of the layer input x_t (width d_model) to H heads of width d, with the
 * weight stored output-major like a linear layer's, so that
 *     XQ[b,h,t,j] = sum_k X[b,t,k] * theta[0][h*d + j][k]
 *     XK[b,h,t,j] = sum_k X[b,t,k] * theta[1][h*d + j][k]
 *     XV[b,h,t,j] = sum_k X[b,t,k] * theta[2][h*d + j][k]
 * X : [B,L,d_model]   theta : [3, H*d, d_model]   XQ, XK, XV : [B,H,L,d]
 * The sum runs over k in increasing order, in fp64.
 */
int oracle_qkv_project(int B, int L, int dm, int H, int d, const double *X,
                       const double *theta, double *XQ, double *XK, double *XV)
{
    if (B < 0 || L < 0 || dm <= 0 || H < 0 || d <= 0) return ORACLE_E_ARG;
    double *outs[3] = {XQ, XK, XV};
    const size_t hd = (size_t)H * d;
    for (int v = 0; v < 3; ++v)
        for (int b = 0; b < B; ++b)
            for (int h = 0; h < H; ++h)
                for (int t = 0; t < L; ++t)
                    for (int j = 0; j < d; ++j) {
                        const double *x = X + ((size_t)b * L + t) * dm;
                        const double *w = theta + ((size_t)v * hd + (size_t)h * d + j) * dm;
                        double s = 0.0;
                        for (int k = 0; k < dm; ++k) s += x[k] * w[k];
                        outs[v][(((size_t)b * H + h) * L + t) * d + j] = s;
                    }
    return ORACLE_OK;
}

/* The same sums at n chosen outputs: idx[5*i .. 5*i+4] = (view, b, h, t, j),
 * view 0 = XQ, 1 = XK, 2 = XV; out[i] receives that output. */
int oracle_qkv_project_at(int B, int L, int dm, int H, int d, const double *X,
                          const double *theta, int n, const int *idx, double *out)
{
    if (B < 0 || L < 0 || dm <= 0 || H < 0 || d <= 0 || n < 0) return ORACLE_E_ARG;
    const size_t hd = (size_t)H * d;
    for (int i = 0; i < n; ++i) {
        const int v = idx[5 * i], b = idx[5 * i + 1], h = idx[5 * i + 2], t = idx[5 * i + 3],
                  j = idx[5 * i + 4];
        if (v < 0 || v > 2 || b < 0 || b >= B || h < 0 || h >= H || t < 0 || t >= L || j < 0 || j >= d)
            return ORACLE_E_ARG;
        const double *x = X + ((size_t)b * L + t) * dm;
        const double *w = theta + ((size_t)v * hd + (size_t)h * d + j) * dm;
        double s = 0.0;
        for (int k = 0; k < dm; ++k) s += x[k] * w[k];
        out[i] = s;
    }
    return ORACLE_OK;
}
