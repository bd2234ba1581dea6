/*
 * Oracle for the selective state-space scan (S6) and its one-token decode step.
 *
 * TEST INFRASTRUCTURE ONLY. This file is the slow, obviously correct CPU
 * definition that the GPU library is checked against. Only the tests, the
 * smoke check and the CPU-baseline leg of the benchmark may load it; the
 * product path never does. It shares no code, header, table or helper with
 * the HIP library.
 *
 * Everything is IEEE double precision with libm exp/log1p, in the plain order
 * the pages give: a sequential loop over time t for each (batch, channel) row,
 * the state dimension n innermost. Rows are independent, so they are handed
 * out to threads in contiguous blocks; that changes no arithmetic.
 *
 * What is computed, per row (b, d), starting from h = h0 (zero unless given):
 *
 *   delta_t = softplus(delta_raw[b,d,t] + dt_bias[d])
 *       "State Space Models and Mamba" (multigrid.ai), section "Selective
 *       state: the change that made it work on text": the step size is the
 *       softplus of a per-token projection; "Mamba: Linear-Time Sequence
 *       Modeling with Selective State Spaces" (azimuth.plus), the list of the
 *       three input-dependent parameters of S6. The projection itself arrives
 *       as the input delta_raw; dt_bias is a per-channel additive bias.
 *
 *   Abar = exp(delta_t * A[d,n]);   h[n] = Abar * h[n] + delta_t * B[b,n,t] * x[b,d,t]
 *       multigrid.ai, same section: the discretised decay and the input term.
 *       A is diagonal with negative real entries (section "It is a linear
 *       recurrence").
 *
 *   y[b,d,t] = (sum_n C[b,n,t] * h[n] + D[d] * x[b,d,t]) * silu(z[b,d,t])
 *       readout by C ("It is a linear recurrence"); the D feed-through is one
 *       of the four SSM matrices named in "State space models and Mamba:
 *       reading long sequences without attention" (ai-trend.me), section
 *       "Core idea: one notepad page instead of full meeting minutes"; the
 *       multiplicative SiLU gate branch is in multigrid.ai, section "What a
 *       Mamba block actually contains". silu(z) = z / (1 + exp(-z)).
 *
 *   last_state[b,d,n] = h[n] after the last token (the fixed-size state of
 *       multigrid.ai, section "The state, in bytes, against a KV cache").
 *
 * Error scales. Alongside each output the oracle carries the same recurrence
 * on absolute values:  habs[n] = Abar * habs[n] + |delta_t * B * x|  (habs
 * starts from |h0|), and
 *   y_scale = (sum_n |C| * habs[n] + |D * x|) * |silu(z)|.
 * Each is the sum of the magnitudes of the terms that make up the output, the
 * natural yardstick for the rounding error of any evaluation order, and is
 * what relative errors are measured against.
 *
 * Layouts (all row-major, contiguous): x, delta, z, y: [batch, dim, seqlen];
 * B, C: [batch, dstate, seqlen]; A: [dim, dstate]; D, dt_bias: [dim];
 * states: [batch, dim, dstate]. Null D, z or dt_bias mean D = 0, no gate,
 * bias 0.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* softplus(u) = ln(1 + e^u), written in the overflow-free form
 * max(u, 0) + ln(1 + e^{-|u|}), which is the same function. */
static double softplus(double u) { return fmax(u, 0.0) + log1p(exp(-fabs(u))); }

/* silu(z) = z * sigmoid(z) = z / (1 + e^{-z}). */
static double silu(double z) { return z / (1.0 + exp(-z)); }

typedef struct {
    /* inputs */
    const double *x, *delta, *A, *B, *C, *D, *z, *dt_bias, *h0, *h0_scale;
    int64_t batch, seqlen, dim, dstate;
    const int64_t *rows; /* NULL: row i is b*dim+d = i */
    /* outputs, indexed by position in the row list */
    double *y, *last_state, *y_scale, *state_scale;
    /* work split */
    int64_t row_begin, row_end;
} fwd_job;

static void fwd_rows(const fwd_job *j)
{
    const int64_t L = j->seqlen, N = j->dstate;
    double *h = (double *)malloc(sizeof(double) * (size_t)N);
    double *habs = (double *)malloc(sizeof(double) * (size_t)N);
    for (int64_t i = j->row_begin; i < j->row_end; ++i) {
        const int64_t row = j->rows ? j->rows[i] : i;
        const int64_t b = row / j->dim, d = row % j->dim;
        const double *x = j->x + row * L;
        const double *dr = j->delta + row * L;
        const double *z = j->z ? j->z + row * L : NULL;
        const double *Bb = j->B + b * N * L;
        const double *Cb = j->C + b * N * L;
        const double *Ad = j->A + d * N;
        const double Dd = j->D ? j->D[d] : 0.0;
        const double bias = j->dt_bias ? j->dt_bias[d] : 0.0;
        for (int64_t n = 0; n < N; ++n) {
            h[n] = j->h0 ? j->h0[row * N + n] : 0.0;
            habs[n] = j->h0 ? (j->h0_scale ? j->h0_scale[row * N + n] : fabs(h[n])) : 0.0;
        }
        for (int64_t t = 0; t < L; ++t) {
            const double dl = softplus(dr[t] + bias);
            for (int64_t n = 0; n < N; ++n) {
                const double abar = exp(dl * Ad[n]);
                const double bx = dl * Bb[n * L + t] * x[t];
                h[n] = abar * h[n] + bx;
                habs[n] = abar * habs[n] + fabs(bx);
            }
            double acc = 0.0, acc_abs = 0.0;
            for (int64_t n = 0; n < N; ++n) {
                acc += Cb[n * L + t] * h[n];
                acc_abs += fabs(Cb[n * L + t]) * habs[n];
            }
            double yv = acc + Dd * x[t];
            double sv = acc_abs + fabs(Dd * x[t]);
            if (z) {
                const double g = silu(z[t]);
                yv *= g;
                sv *= fabs(g);
            }
            j->y[i * L + t] = yv;
            if (j->y_scale) j->y_scale[i * L + t] = sv;
        }
        for (int64_t n = 0; n < N; ++n) {
            if (j->last_state) j->last_state[i * N + n] = h[n];
            if (j->state_scale) j->state_scale[i * N + n] = habs[n];
        }
    }
    free(h);
    free(habs);
}

static void *fwd_thread(void *p)
{
    fwd_job *j = (fwd_job *)p;
    fwd_rows(j);
    return NULL;
}

/* Return codes: 0 ok, -1 null required pointer, -2 bad sizes, -3 thread failure. */
int ssm_ref_fwd(const double *x, const double *delta, const double *A, const double *B,
                const double *C, const double *D, const double *z, const double *dt_bias,
                const double *h0, const double *h0_scale,
                int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate,
                const int64_t *rows, int64_t nrows,
                double *y, double *last_state, double *y_scale, double *state_scale,
                int nthreads)
{
    if (!x || !delta || !A || !B || !C || !y) return -1;
    if (batch <= 0 || seqlen < 0 || dim <= 0 || dstate <= 0) return -2;
    if (!rows) nrows = batch * dim;
    if (nrows < 0) return -2;
    if (rows)
        for (int64_t i = 0; i < nrows; ++i)
            if (rows[i] < 0 || rows[i] >= batch * dim) return -2;
    if (nthreads < 1) nthreads = 1;
    if (nthreads > nrows) nthreads = nrows > 0 ? (int)nrows : 1;

    fwd_job base;
    memset(&base, 0, sizeof base);
    base.x = x; base.delta = delta; base.A = A; base.B = B; base.C = C;
    base.D = D; base.z = z; base.dt_bias = dt_bias; base.h0 = h0; base.h0_scale = h0_scale;
    base.batch = batch; base.seqlen = seqlen; base.dim = dim; base.dstate = dstate;
    base.rows = rows; base.y = y; base.last_state = last_state;
    base.y_scale = y_scale; base.state_scale = state_scale;

    fwd_job *jobs = (fwd_job *)calloc((size_t)nthreads, sizeof(fwd_job));
    pthread_t *tid = (pthread_t *)calloc((size_t)nthreads, sizeof(pthread_t));
    int rc = 0;
    for (int k = 0; k < nthreads; ++k) {
        jobs[k] = base;
        jobs[k].row_begin = nrows * k / nthreads;
        jobs[k].row_end = nrows * (k + 1) / nthreads;
    }
    int started = 0;
    for (int k = 1; k < nthreads; ++k) {
        if (pthread_create(&tid[k], NULL, fwd_thread, &jobs[k]) != 0) { rc = -3; break; }
        started = k;
    }
    if (rc == 0) fwd_rows(&jobs[0]);
    for (int k = 1; k <= started; ++k) pthread_join(tid[k], NULL);
    free(jobs);
    free(tid);
    return rc;
}

/*
 * One decode step: the same update for a single token, continuing from a
 * state (multigrid.ai, section "Why a linear recurrence can be trained in
 * parallel": at inference the layer runs as the recurrence, one token at a
 * time, with a fixed-size state). The step takes delta already biased:
 * delta_t = softplus(delta[b,d]). state and state_scale are updated in place.
 * x, delta, z, y: [batch, dim]; B, C: [batch, dstate]; state: [batch, dim, dstate].
 */
int ssm_ref_step(double *state, double *state_scale,
                 const double *x, const double *delta, const double *A, const double *B,
                 const double *C, const double *D, const double *z,
                 int64_t batch, int64_t dim, int64_t dstate,
                 double *y, double *y_scale)
{
    if (!state || !x || !delta || !A || !B || !C || !y) return -1;
    if (batch <= 0 || dim <= 0 || dstate <= 0) return -2;
    const int64_t N = dstate;
    for (int64_t b = 0; b < batch; ++b) {
        for (int64_t d = 0; d < dim; ++d) {
            const int64_t row = b * dim + d;
            double *h = state + row * N;
            double *habs = state_scale ? state_scale + row * N : NULL;
            const double xv = x[row];
            const double dl = softplus(delta[row]);
            double acc = 0.0, acc_abs = 0.0;
            for (int64_t n = 0; n < N; ++n) {
                const double abar = exp(dl * A[d * N + n]);
                const double bx = dl * B[b * N + n] * xv;
                h[n] = abar * h[n] + bx;
                acc += C[b * N + n] * h[n];
                if (habs) {
                    habs[n] = abar * habs[n] + fabs(bx);
                    acc_abs += fabs(C[b * N + n]) * habs[n];
                } else {
                    acc_abs += fabs(C[b * N + n] * h[n]);
                }
            }
            const double Dd = D ? D[d] : 0.0;
            double yv = acc + Dd * xv;
            double sv = acc_abs + fabs(Dd * xv);
            if (z) {
                const double g = silu(z[row]);
                yv *= g;
                sv *= fabs(g);
            }
            y[row] = yv;
            if (y_scale) y_scale[row] = sv;
        }
    }
    return 0;
}

/*
 * The short causal convolution in front of the selective SSM, and its decode
 * step.
 *
 * "State Space Models and Mamba" (multigrid.ai), section "What a Mamba block
 * actually contains": the SSM branch is a depthwise conv1d of kernel width 4,
 * then SiLU, then the selective SSM; the four-position convolution gives the
 * block direct access to the few tokens just before the current one. "Mamba:
 * Linear-Time Sequence Modeling with Selective State Spaces" (azimuth.plus),
 * the block architecture: projection, then a short 1D convolution (kernel
 * size 4), then SiLU, then the selective SSM. Depthwise: each channel d has
 * its own K taps w[d, 0..K-1] (and bias[d]). It must be causal, since the
 * same block runs one token at a time at inference: token t sees inputs
 * t-K+1 .. t only. For each row (b, d) and token t:
 *
 *   pre = bias[d] + sum_{k=0}^{K-1} w[d,k] * xx(t - (K-1) + k)
 *   out[b,d,t] = silu(pre) = pre / (1 + exp(-pre))
 *
 * with xx(s) = x[b,d,s] for s >= 0 and, for s < 0, x_prev[b,d,K-1+s]: the
 * K-1 inputs that came before token 0 (zeros when x_prev is null). x_last
 * receives the last K-1 entries of the sequence x_prev ++ x, i.e. the x_prev
 * of a call that continues where this one stops.
 *
 * Error scale: out_scale = |bias| + sum_k |w[d,k] * xx(...)|, the magnitude
 * sum of the terms of pre; silu is 1.1-Lipschitz, so it bounds the rounding
 * error of out for any evaluation order.
 *
 * Layouts: x, out, out_scale: [batch, dim, seqlen]; w: [dim, K]; bias: [dim];
 * x_prev, x_last: [batch, dim, K-1].
 */
int ssm_ref_conv1d(const double *x, const double *w, const double *bias, const double *x_prev,
                   int64_t batch, int64_t seqlen, int64_t dim, int64_t K,
                   double *out, double *out_scale, double *x_last)
{
    if (!x || !w || !out) return -1;
    if (batch < 0 || seqlen < 0 || dim < 0 || K < 1) return -2;
    for (int64_t b = 0; b < batch; ++b) {
        for (int64_t d = 0; d < dim; ++d) {
            const int64_t row = b * dim + d;
            const double *xr = x + row * seqlen;
            const double *pr = x_prev ? x_prev + row * (K - 1) : NULL;
            for (int64_t t = 0; t < seqlen; ++t) {
                double pre = bias ? bias[d] : 0.0;
                double sc = fabs(pre);
                for (int64_t k = 0; k < K; ++k) {
                    const int64_t s = t - (K - 1) + k;
                    const double xv = s >= 0 ? xr[s] : (pr ? pr[K - 1 + s] : 0.0);
                    pre += w[d * K + k] * xv;
                    sc += fabs(w[d * K + k] * xv);
                }
                out[row * seqlen + t] = silu(pre);
                if (out_scale) out_scale[row * seqlen + t] = sc;
            }
            if (x_last) {
                for (int64_t k = 0; k < K - 1; ++k) {
                    const int64_t s = seqlen - (K - 1) + k;
                    x_last[row * (K - 1) + k] = s >= 0 ? xr[s] : (pr ? pr[K - 1 + s] : 0.0);
                }
            }
        }
    }
    return 0;
}

/*
 * One decode step of the convolution: the same formula for a single token x
 * [batch, dim] with the K-1 previous inputs held in conv_state [batch, dim,
 * K-1] (oldest first), which is then shifted by one and takes x as its
 * newest entry.
 */
int ssm_ref_conv1d_step(double *conv_state, const double *x, const double *w, const double *bias,
                        int64_t batch, int64_t dim, int64_t K, double *out, double *out_scale)
{
    if (!conv_state || !x || !w || !out) return -1;
    if (batch < 0 || dim < 0 || K < 1) return -2;
    for (int64_t b = 0; b < batch; ++b) {
        for (int64_t d = 0; d < dim; ++d) {
            const int64_t row = b * dim + d;
            double *st = conv_state + row * (K - 1);
            double pre = bias ? bias[d] : 0.0;
            double sc = fabs(pre);
            for (int64_t k = 0; k < K - 1; ++k) {
                pre += w[d * K + k] * st[k];
                sc += fabs(w[d * K + k] * st[k]);
            }
            pre += w[d * K + K - 1] * x[row];
            sc += fabs(w[d * K + K - 1] * x[row]);
            out[row] = silu(pre);
            if (out_scale) out_scale[row] = sc;
            for (int64_t k = 0; k + 1 < K - 1; ++k) st[k] = st[k + 1];
            if (K > 1) st[K - 2] = x[row];
        }
    }
    return 0;
}
