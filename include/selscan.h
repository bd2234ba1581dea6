/*
 * libselscan: the selective state-space scan (S6) and its one-token decode step
 * on AMD Instinct MI355X (gfx950).
 *
 * C ABI. Every tensor argument is a pointer to contiguous, caller-owned DEVICE
 * memory, 16-byte aligned (any torch/hipMalloc allocation is). The library
 * never frees or keeps a caller buffer. All work is enqueued on the caller's
 * stream (a hipStream_t passed as void*; NULL is the default stream) and the
 * calls return as soon as it is enqueued.
 *
 * Shapes: B = batch, L = seqlen, d = dim (channels, "d_inner"), N = dstate.
 * dtype (selscan_dtype_t) is the storage type of x, delta, z, B, C and y:
 * fp32 or bfloat16. A, D, dt_bias and every state are always fp32, and all
 * arithmetic is fp32.
 *
 * Error handling: every argument check runs on the host before any HIP call,
 * and a failed check returns its negative code with nothing enqueued. A launch
 * that the runtime rejects returns SELSCAN_ERR_LAUNCH. Faults inside a kernel
 * surface at the caller's next synchronisation. No value checks are made on
 * the data: NaN and Inf propagate through the arithmetic.
 */
#ifndef SELSCAN_H
#define SELSCAN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { SELSCAN_F32 = 0, SELSCAN_BF16 = 1 } selscan_dtype_t;

typedef struct {
    int64_t batch;   /* B >= 0 */
    int64_t seqlen;  /* 0 <= L < 2^27 (ignored by selscan_step) */
    int64_t dim;     /* d >= 0 */
    int64_t dstate;  /* N; this version supports N == 16 */
    int32_t dtype;   /* selscan_dtype_t */
} selscan_dims_t;

/* Return codes. */
#define SELSCAN_OK 0
#define SELSCAN_ERR_NULL (-1)   /* a required pointer is NULL */
#define SELSCAN_ERR_DIMS (-2)   /* a size is negative, or a size/offset overflows */
#define SELSCAN_ERR_DSTATE (-3) /* dstate other than 16 */
#define SELSCAN_ERR_DTYPE (-4)  /* dtype not a selscan_dtype_t */
#define SELSCAN_ERR_LAUNCH (-5) /* the HIP runtime rejected a launch */
#define SELSCAN_ERR_ALLOC (-6)  /* workspace allocation on the stream failed */
#define SELSCAN_ERR_ALIGN (-7)  /* a pointer is not 16-byte aligned */
#define SELSCAN_ERR_ALIAS (-8)  /* an output overlaps an input or another output */
#define SELSCAN_ERR_CONFIG (-9) /* selscan_fwd_ex launch options out of range */

/*
 * selscan_fwd — the selective scan over whole sequences.
 *
 * Defined by: "State Space Models and Mamba" (multigrid.ai), section
 * "Selective state: the change that made it work on text" (input-dependent
 * step size delta = softplus(projection), decay exp(delta*A), input term
 * delta*B*x) and section "It is a linear recurrence" (readout by C; diagonal
 * A of negative reals); the D feed-through of "State space models and Mamba:
 * reading long sequences without attention" (ai-trend.me), section "Core
 * idea: one notepad page instead of full meeting minutes"; the SiLU gate
 * branch of multigrid.ai, section "What a Mamba block actually contains"; and
 * the fused evaluation that keeps the state on chip of "Mamba: Linear-Time
 * Sequence Modeling with Selective State Spaces" (azimuth.plus), hardware-aware
 * algorithm (kernel fusion, parallel scan).
 *
 * For every row (b, d), from h = 0:
 *   delta_t = softplus(delta[b,d,t] + dt_bias[d])
 *   h[n]    = exp(delta_t * A[d,n]) * h[n] + delta_t * B[b,n,t] * x[b,d,t]
 *   y[b,d,t] = (sum_n C[b,n,t] * h[n] + D[d] * x[b,d,t]) * silu(z[b,d,t])
 *   last_state[b,d,n] = h[n] after token L-1
 *
 * Arguments (device pointers):
 *   x, delta, z, y : [B, d, L] of dtype (L contiguous)
 *   B, C           : [B, N, L] of dtype
 *   A              : [d, N] fp32, the negative reals themselves (not a log)
 *   D, dt_bias     : [d] fp32; NULL means 0
 *   z              : NULL means no gate (y is the SSM output itself)
 *   last_state     : [B, d, N] fp32 output; NULL means not wanted
 * Owns nothing. Long sequences with few rows use a temporary workspace of
 * about 2 * segments * B * d * N * 4 bytes, taken with hipMallocAsync on the
 * stream and released with hipFreeAsync on it (SELSCAN_ERR_ALLOC if that
 * fails). y and last_state must not overlap any input or each other.
 * Deterministic: the same inputs give the same bits.
 */
int selscan_fwd(const void* x, const void* delta, const float* A, const void* B, const void* C,
                const float* D, const void* z, const float* dt_bias, void* y, float* last_state,
                const selscan_dims_t* dims, void* stream);

/*
 * selscan_fwd_ex — selscan_fwd with explicit launch choices (for tuning and
 * for testing one evaluation order against another). Same semantics and
 * results up to rounding.
 *   segments : number of sequence segments scanned in parallel (1 = one pass
 *              per row; > 1 = chunk states, a carry pass, then the output
 *              pass); 0 = automatic. At most 65536, and the segment length is
 *              rounded up to the kernel's time tile.
 *   groups   : waves per 64-row block, each taking N/groups states: 1, 2 or
 *              4; 0 = automatic.
 */
int selscan_fwd_ex(const void* x, const void* delta, const float* A, const void* B, const void* C,
                   const float* D, const void* z, const float* dt_bias, void* y,
                   float* last_state, const selscan_dims_t* dims, int32_t segments,
                   int32_t groups, void* stream);

/*
 * selscan_step — one decode step, updating the state in place.
 *
 * Defined by: "State Space Models and Mamba" (multigrid.ai), section "Why a
 * linear recurrence can be trained in parallel" (at inference the layer runs
 * the recurrence one token at a time on a fixed-size state) and the same
 * update as selscan_fwd for a single token.
 *
 * For every row (b, d):
 *   delta_t = softplus(delta[b,d])         (the channel bias, if any, is
 *                                            already added by the caller)
 *   state[b,d,n] = exp(delta_t * A[d,n]) * state[b,d,n] + delta_t * B[b,n] * x[b,d]
 *   y[b,d] = (sum_n C[b,n] * state[b,d,n] + D[d] * x[b,d]) * silu(z[b,d])
 *
 * Arguments (device pointers):
 *   state       : [B, d, N] fp32, read and written in place
 *   x, delta, z : [B, d] of dtype; y: [B, d] of dtype (output)
 *   B, C        : [B, N] of dtype; A: [d, N] fp32; D: [d] fp32 or NULL
 *   z           : NULL means no gate
 * dims->seqlen is ignored. y must not overlap any input or the state.
 * Running L steps with delta = delta_raw[..., t] + dt_bias equals
 * selscan_fwd over the L tokens.
 */
int selscan_step(float* state, const void* x, const void* delta, const float* A, const void* B,
                 const void* C, const float* D, const void* z, void* y,
                 const selscan_dims_t* dims, void* stream);

/* A static, human-readable message for a return code. */
const char* selscan_strerror(int code);

/* Library version as major*10000 + minor*100 + patch. */
int selscan_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SELSCAN_H */
