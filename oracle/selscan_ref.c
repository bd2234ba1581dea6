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
 * Gradients of the convolution + SiLU above for an output gradient dout
 * [batch, dim, seqlen]: the chain rule through its definition, written out.
 *   pre[t] = bias + sum_k w[k] xx(t - (K-1) + k),   out[t] = silu(pre[t])
 *   g[t]   = dout[t] * silu'(pre[t]),  silu'(u) = sig(u) (1 + u (1 - sig(u)))
 *   dxx(s) = sum_k w[k] g[s + (K-1) - k]   over the t = s + (K-1) - k in [0, L)
 *   dx[t] = dxx(t) (t >= 0);  dx_prev[j] = dxx(j - (K-1))  (j < K-1)
 *   dw[d,k] = sum_{b,t} g[t] xx(t - (K-1) + k);   dbias[d] = sum_{b,t} g[t]
 * Scales: the same sums on magnitudes, silu' taken as the sum of its two
 * terms' magnitudes, sig(u) (1 + |u| (1 - sig(u))), and pre as its terms'.
 * dx_prev, dbias and their scales may be null (not wanted). dw, dbias: sums
 * over batch entries in order.
 */
int ssm_ref_conv1d_bwd(const double *x, const double *w, const double *bias, const double *x_prev,
                       const double *dout, int64_t batch, int64_t seqlen, int64_t dim, int64_t K,
                       double *dx, double *dx_prev, double *dw, double *dbias,
                       double *sdx, double *sdx_prev, double *sdw, double *sdbias)
{
    if (!x || !w || !dout || !dx || !dw || !sdx || !sdw) return -1;
    if ((dx_prev && !sdx_prev) || (dbias && !sdbias)) return -1;
    if (batch < 0 || seqlen < 0 || dim < 0 || K < 1) return -2;
    const int64_t L = seqlen, H = K - 1;
    double *g = malloc(sizeof(double) * (size_t)(2 * (L + 1)));
    if (!g) return -3;
    double *ga = g + L + 1;
    for (int64_t i = 0; i < dim * K; ++i) dw[i] = sdw[i] = 0.0;
    if (dbias) for (int64_t d = 0; d < dim; ++d) dbias[d] = sdbias[d] = 0.0;
    for (int64_t b = 0; b < batch; ++b) {
        for (int64_t d = 0; d < dim; ++d) {
            const int64_t row = b * dim + d;
            const double *xr = x + row * L, *dr = dout + row * L;
            const double *pr = x_prev ? x_prev + row * H : NULL;
            const double *wd = w + d * K;
            #define XX(s) ((s) >= 0 ? xr[s] : (pr ? pr[H + (s)] : 0.0))
            for (int64_t t = 0; t < L; ++t) {
                double pre = bias ? bias[d] : 0.0, pa = fabs(pre);
                for (int64_t k = 0; k < K; ++k) {
                    pre += wd[k] * XX(t - H + k);
                    pa += fabs(wd[k] * XX(t - H + k));
                }
                const double sg = 1.0 / (1.0 + exp(-pre));
                g[t] = dr[t] * sg * (1.0 + pre * (1.0 - sg));
                ga[t] = fabs(dr[t]) * sg * (1.0 + pa * (1.0 - sg));
                for (int64_t k = 0; k < K; ++k) {
                    dw[d * K + k] += g[t] * XX(t - H + k);
                    sdw[d * K + k] += ga[t] * fabs(XX(t - H + k));
                }
                if (dbias) { dbias[d] += g[t]; sdbias[d] += ga[t]; }
            }
            for (int64_t s = -H; s < L; ++s) {
                double v = 0.0, va = 0.0;
                for (int64_t k = 0; k < K; ++k) {
                    const int64_t t = s + H - k;
                    if (t >= 0 && t < L) { v += wd[k] * g[t]; va += fabs(wd[k]) * ga[t]; }
                }
                if (s >= 0) { dx[row * L + s] = v; sdx[row * L + s] = va; }
                else if (dx_prev) { dx_prev[row * H + H + s] = v; sdx_prev[row * H + H + s] = va; }
            }
            #undef XX
        }
    }
    free(g);
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

/*
 * Backward pass: gradients of a scalar loss whose gradient with respect to y
 * is dy, through the forward pass defined above (from h = 0).
 *
 * "Mamba: Linear-Time Sequence Modeling with Selective State Spaces"
 * (azimuth.plus), hardware-aware algorithm, recomputation: the backward pass
 * does not keep the per-token states of the forward pass but recomputes
 * them; "Mamba State Space Models: Fixed State, Linear Time" (deepnoodle.ai)
 * likewise. Here the oracle simply recomputes the forward states of a row
 * into a buffer and walks back through them; the gradients are the chain
 * rule applied to the definition, written out:
 *
 *   g = silu(z), s_t = sum_n C h + D x, y = s g
 *   dz   = dy * s * silu'(z),  silu'(z) = sig(z) (1 + z (1 - sig(z)))
 *   ds   = dy * g;  dD += ds * x
 *   going back in t, with carry[n] = dlast[n] after the last token (the
 *   gradient flowing into the final state; 0 when none is given):
 *     dh[n] = ds * C[n,t] + carry[n]           (total gradient of h_t[n])
 *     abar  = exp(dl * A[n]);  q = dh * abar * h_{t-1}[n]
 *     dA[n] += q * dl;   ddl += q * A[n]        (through the decay)
 *     dB[n,t] += dh * dl * x;  ddl += dh * B x;  dx += dh * dl * B   (input term)
 *     dC[n,t] += ds * h_t[n]
 *     carry[n] = abar * dh
 *   dx += ds * D;  ddelta = ddl * sig(u)  (softplus' = sigmoid);  ddt_bias += ddelta
 *   dh0[n] = carry[n] after the first token (h_{-1} = h0, the initial state;
 *   0 when none is given)
 * dA, dD and ddt_bias sum over batch and time; dB and dC sum over channels.
 *
 * Error scales: the same computation on magnitudes (|dy|, |x|, the forward
 * habs, ...), one per output, as for the forward outputs.
 *
 * Layouts as the forward; dA: [dim, dstate]; dD, ddt_bias: [dim];
 * dB, dC: [batch, dstate, seqlen]. D, z, dt_bias may be null (then dD, dz,
 * ddt_bias are not written). h0, dlast and dh0: [batch, dim, dstate], each
 * may be null. Batch entries are split over threads; the
 * per-channel sums are added in batch order afterwards.
 */
typedef struct {
    const double *x, *delta, *A, *B, *C, *D, *z, *dt_bias, *dy, *h0, *dlast;
    double *dh0, *sdh0;
    int64_t batch, L, dim, N;
    double *dx, *ddelta, *dA, *dB, *dC, *dD, *dz, *ddt;       /* values */
    double *sdx, *sddelta, *sdA, *sdB, *sdC, *sdD, *sdz, *sddt; /* scales */
    double *pA, *psA, *pD, *psD, *pT, *psT;                    /* per-batch partials */
    int64_t b0, b1;
    int rc;
} bwd_job;

static double sigmoid(double v) { return 1.0 / (1.0 + exp(-v)); }

static void bwd_batches(bwd_job *j)
{
    const int64_t L = j->L, N = j->N, dim = j->dim;
    double *H = malloc(sizeof(double) * (size_t)(L + 1) * (size_t)N);
    double *HA = malloc(sizeof(double) * (size_t)(L + 1) * (size_t)N);
    double *carry = malloc(sizeof(double) * (size_t)N * 2);
    if (!H || !HA || !carry) { j->rc = -3; free(H); free(HA); free(carry); return; }
    double *carry_abs = carry + N;
    for (int64_t b = j->b0; b < j->b1; ++b) {
        const double *Bb = j->B + b * N * L, *Cb = j->C + b * N * L;
        double *dBb = j->dB + b * N * L, *dCb = j->dC + b * N * L;
        double *sdBb = j->sdB + b * N * L, *sdCb = j->sdC + b * N * L;
        for (int64_t i = 0; i < N * L; ++i) dBb[i] = dCb[i] = sdBb[i] = sdCb[i] = 0.0;
        for (int64_t d = 0; d < dim; ++d) {
            const int64_t row = b * dim + d;
            const double *x = j->x + row * L, *dr = j->delta + row * L, *dy = j->dy + row * L;
            const double *z = j->z ? j->z + row * L : NULL;
            const double *Ad = j->A + d * N;
            const double bias = j->dt_bias ? j->dt_bias[d] : 0.0;
            const double Dd = j->D ? j->D[d] : 0.0;
            /* forward: H[t+1] = h_t, H[0] = h_{-1} = h0 (or 0) */
            for (int64_t n = 0; n < N; ++n) {
                H[n] = j->h0 ? j->h0[row * N + n] : 0.0;
                HA[n] = fabs(H[n]);
            }
            for (int64_t t = 0; t < L; ++t) {
                const double dl = softplus(dr[t] + bias);
                for (int64_t n = 0; n < N; ++n) {
                    const double abar = exp(dl * Ad[n]);
                    const double bx = dl * Bb[n * L + t] * x[t];
                    H[(t + 1) * N + n] = abar * H[t * N + n] + bx;
                    HA[(t + 1) * N + n] = abar * HA[t * N + n] + fabs(bx);
                }
            }
            double dD = 0.0, sD = 0.0, dT = 0.0, sT = 0.0;
            for (int64_t n = 0; n < N; ++n) {
                carry[n] = j->dlast ? j->dlast[row * N + n] : 0.0;
                carry_abs[n] = fabs(carry[n]);
            }
            for (int64_t t = L - 1; t >= 0; --t) {
                const double u = dr[t] + bias;
                const double dl = softplus(u);
                const double *h = H + (t + 1) * N, *hp = H + t * N;
                const double *ha = HA + (t + 1) * N, *hpa = HA + t * N;
                double s = 0.0, sabs = 0.0;
                for (int64_t n = 0; n < N; ++n) {
                    s += Cb[n * L + t] * h[n];
                    sabs += fabs(Cb[n * L + t]) * ha[n];
                }
                s += Dd * x[t];
                sabs += fabs(Dd * x[t]);
                double g = 1.0;
                if (z) {
                    const double sz = sigmoid(z[t]);
                    const double gp = sz * (1.0 + z[t] * (1.0 - sz));
                    g = silu(z[t]);
                    if (j->dz) {
                        /* silu'(z) is formed as sig + z sig (1 - sig), a sum that
                           crosses zero (near z = -1.28): its scale is the sum of
                           the magnitudes of those two terms. */
                        const double gpa = sz * (1.0 + fabs(z[t]) * (1.0 - sz));
                        j->dz[row * L + t] = dy[t] * s * gp;
                        j->sdz[row * L + t] = fabs(dy[t]) * sabs * gpa;
                    }
                }
                const double ds = dy[t] * g, dsa = fabs(ds);
                dD += ds * x[t];
                sD += fabs(ds * x[t]);
                double ddl = 0.0, ddla = 0.0, accB = 0.0, accBa = 0.0;
                for (int64_t n = 0; n < N; ++n) {
                    const double Bv = Bb[n * L + t], Cv = Cb[n * L + t];
                    const double dh = ds * Cv + carry[n];
                    const double dha = dsa * fabs(Cv) + carry_abs[n];
                    const double abar = exp(dl * Ad[n]);
                    const double q = dh * abar * hp[n];
                    const double qa = dha * abar * hpa[n];
                    j->pA[(b * dim + d) * N + n] += q * dl;
                    j->psA[(b * dim + d) * N + n] += qa * dl;
                    ddl += q * Ad[n];
                    ddla += qa * fabs(Ad[n]);
                    dBb[n * L + t] += dh * dl * x[t];
                    sdBb[n * L + t] += dha * fabs(dl * x[t]);
                    accB += dh * Bv;
                    accBa += dha * fabs(Bv);
                    dCb[n * L + t] += ds * h[n];
                    sdCb[n * L + t] += dsa * ha[n];
                    carry[n] = abar * dh;
                    carry_abs[n] = abar * dha;
                }
                ddl += accB * x[t];
                ddla += accBa * fabs(x[t]);
                j->dx[row * L + t] = ds * Dd + dl * accB;
                j->sdx[row * L + t] = fabs(ds * Dd) + dl * accBa;
                const double sg = sigmoid(u);
                j->ddelta[row * L + t] = ddl * sg;
                j->sddelta[row * L + t] = ddla * sg;
                dT += ddl * sg;
                sT += ddla * sg;
            }
            if (j->dh0)
                for (int64_t n = 0; n < N; ++n) {
                    j->dh0[row * N + n] = carry[n];
                    j->sdh0[row * N + n] = carry_abs[n];
                }
            j->pD[b * dim + d] = dD;
            j->psD[b * dim + d] = sD;
            j->pT[b * dim + d] = dT;
            j->psT[b * dim + d] = sT;
        }
    }
    free(H); free(HA); free(carry);
}

static void *bwd_thread(void *p)
{
    bwd_batches((bwd_job *)p);
    return NULL;
}

int ssm_ref_bwd(const double *x, const double *delta, const double *A, const double *B,
                const double *C, const double *D, const double *z, const double *dt_bias,
                const double *dy, const double *h0, const double *dlast,
                int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate,
                double *dx, double *ddelta, double *dA, double *dB, double *dC, double *dD,
                double *dz, double *ddt_bias, double *dh0,
                double *sdx, double *sddelta, double *sdA, double *sdB, double *sdC, double *sdD,
                double *sdz, double *sddt_bias, double *sdh0, int nthreads)
{
    if (!x || !delta || !A || !B || !C || !dy || !dx || !ddelta || !dA || !dB || !dC) return -1;
    if (!sdx || !sddelta || !sdA || !sdB || !sdC) return -1;
    if (D && (!dD || !sdD)) return -1;
    if (dt_bias && (!ddt_bias || !sddt_bias)) return -1;
    if (z && (!dz || !sdz)) return -1;
    if (dh0 && !sdh0) return -1;
    if (batch < 0 || seqlen < 0 || dim < 0 || dstate <= 0) return -2;
    const int64_t N = dstate;
    const size_t nb = (size_t)(batch * dim);
    double *part = calloc(nb * (size_t)(2 * N + 4) + 1, sizeof(double));
    if (!part) return -3;
    if (nthreads < 1) nthreads = 1;
    if (nthreads > batch) nthreads = (int)(batch > 0 ? batch : 1);
    bwd_job proto = {x, delta, A, B, C, D, z, dt_bias, dy, h0, dlast, dh0, sdh0,
                     batch, seqlen, dim, N,
                     dx, ddelta, dA, dB, dC, dD, dz, ddt_bias,
                     sdx, sddelta, sdA, sdB, sdC, sdD, sdz, sddt_bias,
                     part, part + nb * N, part + 2 * nb * N, part + 2 * nb * N + nb,
                     part + 2 * nb * N + 2 * nb, part + 2 * nb * N + 3 * nb, 0, 0, 0};
    bwd_job *jobs = malloc(sizeof(bwd_job) * (size_t)nthreads);
    pthread_t *th = malloc(sizeof(pthread_t) * (size_t)nthreads);
    if (!jobs || !th) { free(part); free(jobs); free(th); return -3; }
    int rc = 0;
    for (int i = 0; i < nthreads; ++i) {
        jobs[i] = proto;
        jobs[i].b0 = batch * i / nthreads;
        jobs[i].b1 = batch * (i + 1) / nthreads;
    }
    int started = 0;
    for (int i = 1; i < nthreads; ++i) {
        if (pthread_create(&th[i], NULL, bwd_thread, &jobs[i]) != 0) { rc = -3; break; }
        started = i;
    }
    if (rc == 0) bwd_batches(&jobs[0]);
    for (int i = 1; i <= started; ++i) pthread_join(th[i], NULL);
    for (int i = 0; i <= started && rc == 0; ++i)
        if (jobs[i].rc) rc = jobs[i].rc;
    /* per-channel sums over batch, in batch order */
    for (int64_t d = 0; d < dim; ++d) {
        for (int64_t n = 0; n < N; ++n) {
            double v = 0.0, s = 0.0;
            for (int64_t b = 0; b < batch; ++b) {
                v += proto.pA[(b * dim + d) * N + n];
                s += proto.psA[(b * dim + d) * N + n];
            }
            dA[d * N + n] = v;
            sdA[d * N + n] = s;
        }
        double vD = 0.0, sD = 0.0, vT = 0.0, sT = 0.0;
        for (int64_t b = 0; b < batch; ++b) {
            vD += proto.pD[b * dim + d]; sD += proto.psD[b * dim + d];
            vT += proto.pT[b * dim + d]; sT += proto.psT[b * dim + d];
        }
        if (D) { dD[d] = vD; sdD[d] = sD; }
        if (dt_bias) { ddt_bias[d] = vT; sddt_bias[d] = sT; }
    }
    free(part); free(jobs); free(th);
    return rc;
}

/*
 * The state space dual (SSD) layer of Mamba-2: the selective SSM restricted
 * so that the decay is one scalar per head and token.
 *
 * "State Space Models Explained: How Mamba Works and How It Compares to
 * Transformers" (mernstackdev.com), section "From S4 to Mamba"; "State
 * space models and Mamba: reading long sequences without attention"
 * (ai-trend.me), section "How it developed: from S4 to Mamba and Mamba-2";
 * "Mamba State Space Models: Fixed State, Linear Time" (deepnoodle.ai). In
 * short: when the decay is restricted enough, the layer's sequence map is a
 * masked product y = (Lmask o C B^T)(delta x) + D x with a semiseparable
 * mask, so matrix products can evaluate it. The restriction read here is the one under which the sequence
 * map is such a matrix: A_t = exp(delta_t A_h) times the identity, one
 * scalar per (token, head); the P channels of a head share delta_t, and B_t,
 * C_t (N entries) are shared by all heads. Per batch entry b and head h, from
 * the state S = h0[b,h] (N x P; zero when h0 is null):
 *
 *   delta_t = softplus(delta_raw[b,t,h] + dt_bias[h])
 *   S[n,p]  = exp(delta_t A_h) S[n,p] + delta_t B[b,t,n] x[b,t,h,p]
 *   y[b,t,h,p] = sum_n C[b,t,n] S[n,p] + D_h x[b,t,h,p]
 *   last_state[b,h,n,p] = S[n,p] after the last token
 *
 * (This is the recurrence; the duality is that y = (Lmask o C B^T)(delta x)
 * + D x with Lmask[t,s] = exp(A_h sum_{s<k<=t} delta_k) for s <= t, which the
 * tests check it against.) Scales as for the selective scan: the same
 * recurrence on magnitudes.
 *
 * Layouts: x, y: [batch, seqlen, heads, headdim]; delta_raw: [batch, seqlen,
 * heads]; A, D, dt_bias: [heads]; B, C: [batch, seqlen, dstate];
 * last_state, h0: [batch, heads, dstate, headdim]. (b, h) pairs are split
 * over threads. One token from a given state is the layer's decode step.
 */
typedef struct {
    const double *x, *delta, *A, *B, *C, *D, *dt_bias, *h0;
    int64_t batch, L, H, P, N;
    double *y, *ys, *hs, *hss;
    int64_t i0, i1;
} ssd_job;

static void ssd_pairs(const ssd_job *j)
{
    const int64_t L = j->L, H = j->H, P = j->P, N = j->N;
    double *S = malloc(sizeof(double) * (size_t)(N * P) * 2);
    if (!S) return;
    double *Sa = S + N * P;
    for (int64_t i = j->i0; i < j->i1; ++i) {
        const int64_t b = i / H, h = i % H;
        for (int64_t k = 0; k < N * P; ++k) {
            S[k] = j->h0 ? j->h0[i * N * P + k] : 0.0;
            Sa[k] = fabs(S[k]);
        }
        const double Ah = j->A[h], Dh = j->D ? j->D[h] : 0.0, bias = j->dt_bias ? j->dt_bias[h] : 0.0;
        for (int64_t t = 0; t < L; ++t) {
            const double dl = softplus(j->delta[(b * L + t) * H + h] + bias);
            const double a = exp(dl * Ah);
            const double *xt = j->x + ((b * L + t) * H + h) * P;
            const double *Bt = j->B + (b * L + t) * N, *Ct = j->C + (b * L + t) * N;
            for (int64_t n = 0; n < N; ++n)
                for (int64_t p = 0; p < P; ++p) {
                    const double in = dl * Bt[n] * xt[p];
                    S[n * P + p] = a * S[n * P + p] + in;
                    Sa[n * P + p] = a * Sa[n * P + p] + fabs(in);
                }
            double *yt = j->y + ((b * L + t) * H + h) * P;
            double *yst = j->ys ? j->ys + ((b * L + t) * H + h) * P : NULL;
            for (int64_t p = 0; p < P; ++p) {
                double acc = 0.0, accs = 0.0;
                for (int64_t n = 0; n < N; ++n) {
                    acc += Ct[n] * S[n * P + p];
                    accs += fabs(Ct[n]) * Sa[n * P + p];
                }
                yt[p] = acc + Dh * xt[p];
                if (yst) yst[p] = accs + fabs(Dh * xt[p]);
            }
        }
        if (j->hs)
            for (int64_t k = 0; k < N * P; ++k) j->hs[i * N * P + k] = S[k];
        if (j->hss)
            for (int64_t k = 0; k < N * P; ++k) j->hss[i * N * P + k] = Sa[k];
    }
    free(S);
}

static void *ssd_thread(void *p)
{
    ssd_pairs((const ssd_job *)p);
    return NULL;
}

int ssm_ref_ssd(const double *x, const double *delta, const double *A, const double *B,
                const double *C, const double *D, const double *dt_bias, const double *h0,
                int64_t batch, int64_t seqlen, int64_t heads, int64_t headdim, int64_t dstate,
                double *y, double *y_scale, double *last_state, double *state_scale, int nthreads)
{
    if (!x || !delta || !A || !B || !C || !y) return -1;
    if (batch < 0 || seqlen < 0 || heads < 0 || headdim <= 0 || dstate <= 0) return -2;
    const int64_t pairs = batch * heads;
    if (nthreads < 1) nthreads = 1;
    if (nthreads > pairs) nthreads = pairs > 0 ? (int)pairs : 1;
    ssd_job base = {x, delta, A, B, C, D, dt_bias, h0, batch, seqlen, heads, headdim, dstate,
                    y, y_scale, last_state, state_scale, 0, 0};
    ssd_job *jobs = calloc((size_t)nthreads, sizeof(ssd_job));
    pthread_t *tid = calloc((size_t)nthreads, sizeof(pthread_t));
    if (!jobs || !tid) { free(jobs); free(tid); return -3; }
    int rc = 0, started = 0;
    for (int k = 0; k < nthreads; ++k) {
        jobs[k] = base;
        jobs[k].i0 = pairs * k / nthreads;
        jobs[k].i1 = pairs * (k + 1) / nthreads;
    }
    for (int k = 1; k < nthreads; ++k) {
        if (pthread_create(&tid[k], NULL, ssd_thread, &jobs[k]) != 0) { rc = -3; break; }
        started = k;
    }
    if (rc == 0) ssd_pairs(&jobs[0]);
    for (int k = 1; k <= started; ++k) pthread_join(tid[k], NULL);
    free(jobs);
    free(tid);
    return rc;
}
