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
#define SELSCAN_ERR_CONFIG (-9) /* options out of range, or workspace too small */
#define SELSCAN_ERR_SCRATCH (-10) /* selscan_fwd_noalloc: the call needs more workspace
                                     than SELSCAN_NOALLOC_SCRATCH_BYTES */

/* Size of the device scratch array behind selscan_fwd_noalloc (per GPU). */
#define SELSCAN_NOALLOC_SCRATCH_BYTES (64u << 20)

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
 * Owns nothing. The call needs a device workspace (B and C repacked as fp32,
 * B * ceil(L/32)*32 * 128 bytes, plus per-segment states when a long sequence
 * with few rows is split: selscan_fwd_workspace_size); selscan_fwd takes it
 * with hipMallocAsync on the stream and returns it with hipFreeAsync on it
 * (SELSCAN_ERR_ALLOC if that fails). selscan_fwd_ex can be handed a caller's
 * workspace instead. y and last_state must not overlap any input or each
 * other. Deterministic: the same inputs and launch choices give the same bits.
 */
int selscan_fwd(const void* x, const void* delta, const float* A, const void* B, const void* C,
                const float* D, const void* z, const float* dt_bias, void* y, float* last_state,
                const selscan_dims_t* dims, void* stream);

/*
 * Options of selscan_fwd_ex. Zero-initialise, then set what is wanted.
 *
 *   h0        : [B, d, N] fp32, the state entering token 0 (a stored prefix
 *               state, so that a long sequence can be fed in pieces: the scan
 *               is a linear recurrence, "State Space Models and Mamba"
 *               (multigrid.ai), section "It is a linear recurrence", and a
 *               state is all that is kept between tokens, section "The state,
 *               in bytes, against a KV cache"). NULL means zeros. Read only;
 *               it may be the same memory as last_state (read before written
 *               by the same row's lanes) but must not overlap y.
 *   workspace : caller-owned device memory of workspace_bytes bytes, 256-byte
 *               aligned, at least selscan_fwd_workspace_size(); NULL means
 *               the library takes and returns its own on the stream. The
 *               contents on entry do not matter; the call uses it until its
 *               work on the stream completes. It must not overlap any input
 *               or output (SELSCAN_ERR_ALIAS).
 *   segments  : sequence segments scanned in parallel (1 = one pass per row;
 *               > 1 = segment states, a carry pass, then the output pass);
 *               0 = automatic. At most 65536; the segment length is rounded
 *               up to the kernels' 32-token tile. Results agree to rounding.
 *   groups    : waves per 64-row block, each taking N/groups states: 1, 2,
 *               4 or 8; 0 = automatic. Results agree to rounding.
 *   ckpt      : NULL, or a [ceil(L/16), B, d, N] fp32 output: the state
 *               entering tokens 0, 16, 32, ... of every row (token 0's is h0
 *               or zeros), for a later selscan_bwd_ex over the same inputs,
 *               which then need not recompute them ("Mamba: Linear-Time
 *               Sequence Modeling with Selective State Spaces" (azimuth.plus),
 *               hardware-aware algorithm: the backward recomputes states
 *               rather than storing all L of them; these are 1/16 of them).
 *               Requires groups 0 or 4. Must not overlap any input or output.
 *   conv_w    : NULL, or [d, 4] fp32 taps of the block's causal depthwise
 *               convolution + SiLU (the definition of selscan_conv1d), which
 *               is then applied to x on the fly: the scan's input is
 *               silu(conv_b[d] + sum_k conv_w[d,k] xx(t - 3 + k)), never
 *               written to memory (x is the convolution's input, and D
 *               multiplies the convolved input). Requires groups 0 or 4 and
 *               no ckpt.
 *   conv_b    : [d] fp32 or NULL (0); only with conv_w.
 *   conv_x_prev, conv_x_last : [B, d, 3] fp32 or NULL, as selscan_conv1d's
 *               x_prev and x_last; only with conv_w. x_last may be x_prev.
 *   variant   : which forward kernel: 0 = automatic; 1 = the per-wave kernel
 *               (every wave both streams its tokens and scans); 2 = the
 *               warp-specialised kernel (scan waves fed through LDS by io
 *               waves that stream x, delta, z and store y), groups then
 *               being its scan waves, 0 (automatic), 4 or 8; 3 = 2, with the
 *               io waves also loading each chunk's B/C operands into the
 *               scalar cache a chunk ahead of the scan waves. 2 and 3 need
 *               L % 4 == 0 and no ckpt or conv_w.
 *               Results agree to rounding.
 */
typedef struct {
    const float* h0;
    void* workspace;
    uint64_t workspace_bytes;
    int32_t segments;
    int32_t groups;
    float* ckpt;
    const float* conv_w;
    const float* conv_b;
    const float* conv_x_prev;
    float* conv_x_last;
    int32_t variant;
} selscan_fwd_opts_t;

/*
 * selscan_fwd_ex — selscan_fwd with an initial state, a caller workspace and
 * explicit launch choices (opts may be NULL: all defaults, which is
 * selscan_fwd). With h0 the recurrence starts from h0 instead of zero:
 * splitting a sequence at any token and passing the first part's last_state
 * as h0 of the second gives the unsplit result up to rounding.
 * Errors as selscan_fwd, plus SELSCAN_ERR_CONFIG for options out of range or
 * a workspace that is too small or misaligned.
 */
int selscan_fwd_ex(const void* x, const void* delta, const float* A, const void* B, const void* C,
                   const float* D, const void* z, const float* dt_bias, void* y,
                   float* last_state, const selscan_dims_t* dims,
                   const selscan_fwd_opts_t* opts, void* stream);

/*
 * selscan_fwd_noalloc — selscan_fwd for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation. Same arguments, results and errors as selscan_fwd, and
 * the same kernels and launch plan; the workspace is a file-scope device array
 * of SELSCAN_NOALLOC_SCRATCH_BYTES (64 MiB) instead of an allocation, so no
 * hipMalloc, hipMallocAsync or hipFree is made. Each GPU the library runs on
 * holds its own copy of the array from first use until the process ends; its
 * device address is looked up on the first call on a device (that device
 * current; the stream must belong to the current device).
 * A call that needs more workspace than the array holds (selscan_fwd_workspace_size
 * with NULL opts: B and C repacked as B * ceil(L/32)*32 * 128 bytes, plus
 * per-segment states) returns SELSCAN_ERR_SCRATCH with nothing enqueued,
 * e.g. batch * L above about 500,000 tokens.
 * Every call on a GPU shares that GPU's array: calls that overlap in time on
 * one GPU (on different streams, or from several threads without ordering on
 * one stream) race on it and must not be made. Calls ordered on one stream
 * are safe; nothing in the array needs to start at zero (each call writes
 * every byte it reads before reading it).
 */
int selscan_fwd_noalloc(const void* x, const void* delta, const float* A, const void* B,
                        const void* C, const float* D, const void* z, const float* dt_bias,
                        void* y, float* last_state, const selscan_dims_t* dims, void* stream);

/*
 * Bytes of workspace selscan_fwd_ex needs for these dims and options (h0 and
 * the workspace fields of opts are ignored; opts may be NULL). Host only.
 * Returns SELSCAN_OK and sets *bytes, or an argument error.
 */
int selscan_fwd_workspace_size(const selscan_dims_t* dims, const selscan_fwd_opts_t* opts,
                               uint64_t* bytes);

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

/*
 * Options of selscan_step_ex. Zero-initialise and set what is wanted.
 *   conv_w     : NULL, or [d, 4] fp32 taps of the block's causal depthwise
 *                convolution + SiLU (the definition of selscan_conv1d_step),
 *                applied to x first in the same kernel: x is then the
 *                convolution's input, and the step's input (also the one D
 *                multiplies) is u = silu(conv_b[d] + conv_w[d,0..2] .
 *                conv_state[b,d,0..2] + conv_w[d,3] x[b,d]), kept in fp32
 *                (never rounded to the dtype or written to memory).
 *   conv_b     : [d] fp32 or NULL (0); only with conv_w.
 *   conv_state : [B, d, 3] fp32, the three previous inputs of every row
 *                (oldest first), read and shifted in place with x appended;
 *                required with conv_w, which it must not overlap, nor any
 *                other argument.
 * The fields exist for "State Space Models and Mamba" (multigrid.ai),
 * section "What a Mamba block actually contains": in the block the
 * convolution sits right in front of the selective SSM, so a decode step of
 * the block is one launch instead of two.
 */
typedef struct {
    const float* conv_w;
    const float* conv_b;
    float* conv_state;
} selscan_step_opts_t;

/*
 * selscan_step_ex — selscan_step with options (opts may be NULL: selscan_step).
 * Errors as selscan_step, plus SELSCAN_ERR_CONFIG for conv_b or conv_state
 * without conv_w, or conv_w without conv_state.
 */
int selscan_step_ex(float* state, const void* x, const void* delta, const float* A, const void* B,
                    const void* C, const float* D, const void* z, void* y,
                    const selscan_dims_t* dims, const selscan_step_opts_t* opts, void* stream);

/*
 * selscan_bwd — gradients of the forward pass (from a zero state) for an
 * output gradient dy.
 *
 * Defined by: the chain rule through the recurrence of selscan_fwd ("State
 * Space Models and Mamba" (multigrid.ai), section "Selective state: the
 * change that made it work on text"), evaluated as "Mamba: Linear-Time
 * Sequence Modeling with Selective State Spaces" (azimuth.plus), hardware-
 * aware algorithm, prescribes: the per-token states are recomputed in the
 * backward pass rather than stored (here from a checkpoint every 16 tokens).
 * With g = silu(z), s = sum_n C h + D x, y = s g, and going back in time with
 * dh[n] = dy g C[n,t] + exp(delta_{t+1} A[n]) dh_{t+1}[n]:
 *   dz      = dy * s * silu'(z)
 *   dx      = dy g D + delta sum_n dh[n] B[n,t]
 *   ddelta  = (x sum_n dh[n] B[n,t] + sum_n dh[n] exp(delta A[n]) h_{t-1}[n] A[n])
 *             * sigmoid(delta_raw + dt_bias)             (gradient of delta_raw)
 *   dA[d,n] = sum_{b,t} dh[n] exp(delta A[n]) h_{t-1}[n] delta
 *   dB[b,n,t] = sum_d dh[n] delta x;   dC[b,n,t] = sum_d dy g h_t[n]
 *   dD[d]   = sum_{b,t} dy g x;   ddt_bias[d] = sum_{b,t} ddelta
 *
 * Arguments (device pointers), inputs exactly as selscan_fwd, plus:
 *   dy                 : [B, d, L] of dtype
 *   dx, ddelta         : [B, d, L] of dtype (outputs)
 *   dz                 : [B, d, L] of dtype, required when z is given, else NULL
 *   dB, dC             : [B, N, L] of dtype (outputs)
 *   dA                 : [d, N] fp32 (output)
 *   dD, ddt_bias       : [d] fp32 outputs, NULL when not wanted (computed
 *                        whether or not D / dt_bias are given)
 * Workspace: about (B d ceil(L/16) + 2 B ceil(d/64) ceil(L/16) 16) * 64 bytes
 * (checkpoints and per-row-block partial sums; 0.4 GB at B 8, L 2048, d 4096),
 * taken with hipMallocAsync on the stream and returned with hipFreeAsync
 * (selscan_bwd_ex takes caller-owned workspace instead).
 * Outputs must not overlap inputs or each other. Deterministic.
 */
int selscan_bwd(const void* x, const void* delta, const float* A, const void* B, const void* C,
                const float* D, const void* z, const float* dt_bias, const void* dy, void* dx,
                void* ddelta, float* dA, void* dB, void* dC, float* dD, void* dz, float* ddt_bias,
                const selscan_dims_t* dims, void* stream);

/*
 * Options of selscan_bwd_ex (zero-initialise, then set what is wanted).
 *   h0          : [B, d, N] fp32, the state the forward started from (as
 *                 selscan_fwd_ex's h0); NULL = zeros.
 *   dlast_state : [B, d, N] fp32, the gradient flowing into the forward's
 *                 last_state (a later chunk's dh0 when a sequence is trained
 *                 in pieces); NULL = zeros. The adjoint carry starts from it.
 *   dh0         : [B, d, N] fp32 output, the gradient of h0 (the adjoint
 *                 carry leaving the first token); NULL = not wanted. With
 *                 L = 0 it is dlast_state (or zeros).
 *   ckpt        : [ceil(L/16), B, d, N] fp32, the checkpoints a
 *                 selscan_fwd_ex over the same inputs (and h0) wrote; the
 *                 call then skips recomputing them (and takes no workspace
 *                 for them). NULL = recompute.
 *   segments : sequence segments swept in parallel. 1 = one reverse sweep per
 *              row; > 1 = the states entering the segments (a forward state
 *              pass and carries), the checkpoint pass over all segments, a
 *              reverse carry sweep of every segment but the first and its
 *              composition, then the reverse sweep of all segments at once;
 *              0 = automatic (segments only when rows are too few to fill the
 *              chip). At most 65536; the segment length is rounded up to 32
 *              tokens, so fewer segments may run. Results agree to rounding;
 *              each choice is deterministic.
 *   workspace : caller-owned device memory of workspace_bytes bytes, 256-byte
 *               aligned, at least selscan_bwd_workspace_size(); NULL means
 *               the library takes and returns its own on the stream. The
 *               contents on entry do not matter; the call uses it until its
 *               work on the stream completes. It must not overlap any input
 *               or output.
 */
typedef struct {
    const float* h0;
    const float* dlast_state;
    float* dh0;
    int32_t segments;
    const float* ckpt;
    void* workspace;
    uint64_t workspace_bytes;
} selscan_bwd_opts_t;

/*
 * selscan_bwd_ex — selscan_bwd with an initial state, a gradient flowing
 * into the final state, the gradient of the initial state, and explicit
 * launch choices (opts may be NULL: all defaults, which is selscan_bwd).
 * Defined by the same chain rule as selscan_bwd with the loss adding
 * sum(dlast_state * last_state) and the recurrence starting from h0: the
 * adjoint carry after the last token is dlast_state, and dh0 is the carry
 * after the first token. Splitting a sequence at a token, running the
 * second part's backward with h0 = the first part's last_state and the first
 * part's with dlast_state = the second part's dh0 gives the unsplit
 * gradients (dA, dD, ddt_bias as the sum of the parts') up to rounding.
 * h0, dlast_state, dh0 and ckpt must be 16-byte aligned; dh0 must not
 * overlap any input or other output. A segmented call takes, beyond the workspace above,
 * 2 S B d 16 fp32 states, S B d doubles and S-fold dA/dD/ddt_bias partial
 * sums. Errors as selscan_bwd, plus SELSCAN_ERR_CONFIG for segments out of
 * range or a caller workspace that is misaligned or smaller than
 * selscan_bwd_workspace_size(), and SELSCAN_ERR_ALIAS for one that overlaps
 * an input or output.
 */
int selscan_bwd_ex(const void* x, const void* delta, const float* A, const void* B, const void* C,
                   const float* D, const void* z, const float* dt_bias, const void* dy, void* dx,
                   void* ddelta, float* dA, void* dB, void* dC, float* dD, void* dz,
                   float* ddt_bias, const selscan_dims_t* dims, const selscan_bwd_opts_t* opts,
                   void* stream);

/*
 * Bytes of workspace selscan_bwd_ex needs for these dims and options (only
 * opts->segments and whether opts->ckpt is set matter; opts may be NULL).
 * Host only. Returns SELSCAN_OK and sets *bytes, or an argument error.
 */
int selscan_bwd_workspace_size(const selscan_dims_t* dims, const selscan_bwd_opts_t* opts,
                               uint64_t* bytes);

/*
 * selscan_ssd_fwd — Mamba-2's state space dual (SSD) layer: the selective SSM
 * restricted to one scalar decay per token and head, evaluated chunk-wise
 * with matrix products.
 *
 * Defined by: "State Space Models Explained: How Mamba Works and How It
 * Compares to Transformers" (mernstackdev.com), section "From S4 to Mamba",
 * and "State space models and Mamba: reading long sequences without
 * attention" (ai-trend.me), section "How it developed: from S4 to Mamba and
 * Mamba-2". With one decay per token and head, the layer's output over a
 * chunk equals y = (Lmask o C B^T)(delta x) + D x, Lmask[t,s] the product of
 * the decays after s up to t (a semiseparable matrix), so it can be formed
 * with matrix products instead of a token-by-token loop. Per batch entry b
 * and head h, from a zero state S (dstate x headdim):
 *   delta_t = softplus(delta[b,t,h] + dt_bias[h])
 *   S = exp(delta_t A[h]) S + delta_t B[b,t,:]^T x[b,t,h,:]
 *   y[b,t,h,:] = C[b,t,:] S + D[h] x[b,t,h,:];   last_state[b,h] = S at the end
 *
 * Arguments (device pointers; bfloat16 only in this version):
 *   x, y       : [B, L, H, P] bf16 (token-major, as a projection writes them)
 *   delta      : [B, L, H] bf16 (before softplus; dt_bias is added first)
 *   A          : [H] fp32, negative; D, dt_bias: [H] fp32 or NULL (0)
 *   B, C       : [B, L, N] bf16, shared by all heads
 *   last_state : [B, H, N, P] fp32 output or NULL
 * dims: batch B, seqlen L (< 2^27), heads H, headdim P (64), dstate N (64 or
 * 128), dtype SELSCAN_BF16 (anything else: SELSCAN_ERR_DTYPE; other P or N:
 * SELSCAN_ERR_DSTATE). No workspace: one workgroup per (batch, head) walks
 * the 64-token chunks in order with the state on chip. Outputs must not
 * overlap inputs. Products in bf16 with fp32 sums (the within-chunk scores,
 * the decay-weighted B and the carried state are rounded to bf16 as
 * matrix-core operands; the state is accumulated in fp32). Deterministic.
 */
typedef struct {
    int64_t batch;
    int64_t seqlen;
    int64_t heads;
    int64_t headdim;
    int64_t dstate;
    int32_t dtype;
} selscan_ssd_dims_t;

int selscan_ssd_fwd(const void* x, const void* delta, const float* A, const void* B, const void* C,
                    const float* D, const float* dt_bias, void* y, float* last_state,
                    const selscan_ssd_dims_t* dims, void* stream);

/*
 * selscan_ssd_fwd_ex — selscan_ssd_fwd from a given state: S starts as
 * h0[b,h] ([B, H, N, P] fp32; NULL means zeros) instead of zero. A state is
 * all the layer keeps between tokens ("State Space Models and Mamba"
 * (multigrid.ai), section "The state, in bytes, against a KV cache"), so a
 * sequence run in two pieces, the second from the first's last_state, gives
 * the unsplit result up to rounding (the state enters the first chunk's
 * products as bf16, like the carried state between chunks). h0 may be
 * last_state itself, but must not overlap y. With L = 0, last_state = h0.
 */
int selscan_ssd_fwd_ex(const void* x, const void* delta, const float* A, const void* B,
                       const void* C, const float* D, const float* dt_bias, const float* h0,
                       void* y, float* last_state, const selscan_ssd_dims_t* dims, void* stream);

/*
 * selscan_ssd_step — one decode step of the SSD layer, the state updated in
 * place: the recurrence of selscan_ssd_fwd for a single token ("State Space
 * Models and Mamba" (multigrid.ai), section "Why a linear recurrence can be
 * trained in parallel": at inference the layer runs the recurrence one token
 * at a time on a fixed-size state). Per (b, h):
 *   delta = softplus(delta[b,h] + dt_bias[h])
 *   state[b,h] = exp(delta A[h]) state[b,h] + delta B[b,:]^T x[b,h,:]
 *   y[b,h,:] = C[b,:] state[b,h] + D[h] x[b,h,:]
 * Arguments (device pointers): state [B, H, N, P] fp32 (read and written);
 * x, y [B, H, P] bf16; delta [B, H] bf16; B, C [B, N] bf16; A [H] fp32; D,
 * dt_bias [H] fp32 or NULL. dims->seqlen is ignored; P 64, N 64 or 128, bf16.
 * Fully fp32 arithmetic (no matrix-core rounding). y and state must not
 * overlap any input or each other. Running L steps equals selscan_ssd_fwd_ex
 * over the L tokens up to that call's bf16 operand rounding.
 */
int selscan_ssd_step(float* state, const void* x, const void* delta, const float* A, const void* B,
                     const void* C, const float* D, const float* dt_bias, void* y,
                     const selscan_ssd_dims_t* dims, void* stream);

/*
 * selscan_conv1d — the short causal convolution in front of the scan: a
 * depthwise conv1d of width SELSCAN_CONV_WIDTH (4), then SiLU.
 *
 * Defined by: "State Space Models and Mamba" (multigrid.ai), section "What a
 * Mamba block actually contains" (the SSM branch is a depthwise conv1d of
 * kernel 4, SiLU, then the selective SSM; the short convolution gives direct
 * access to the last few tokens) and "Mamba: Linear-Time Sequence Modeling
 * with Selective State Spaces" (azimuth.plus), the block architecture
 * (projection, 1D convolution of kernel size 4, SiLU, selective SSM). Causal,
 * since the block also runs one token at a time (selscan_conv1d_step).
 *
 * For every row (b, d) and token t:
 *   out[b,d,t] = silu(bias[d] + sum_{k=0..3} w[d,k] * xx(t - 3 + k))
 *   xx(s) = x[b,d,s] for s >= 0, x_prev[b,d,3+s] for s < 0
 *   x_last[b,d,0..2] = the last three entries of x_prev[b,d,:] ++ x[b,d,:]
 *
 * Arguments (device pointers):
 *   x, out  : [B, d, L] of dtype (L contiguous)
 *   w       : [d, 4] fp32 (tap k multiplies the input 3 - k tokens back)
 *   bias    : [d] fp32; NULL means 0
 *   x_prev  : [B, d, 3] fp32, the three inputs before token 0 (oldest first);
 *             NULL means zeros (the start of a sequence)
 *   x_last  : [B, d, 3] fp32 output, NULL means not wanted; it is the x_prev
 *             of a call that continues this sequence, and the conv_state of
 *             selscan_conv1d_step. It may be x_prev itself.
 * dims->dstate is ignored. out must not overlap any input or x_last. No
 * workspace. Errors as selscan_fwd.
 */
#define SELSCAN_CONV_WIDTH 4
int selscan_conv1d(const void* x, const float* w, const float* bias, const float* x_prev,
                   void* out, float* x_last, const selscan_dims_t* dims, void* stream);

/*
 * selscan_conv1d_bwd — gradients of selscan_conv1d for an output gradient
 * dout: the chain rule through its definition (the training face of the
 * block's convolution; same sources as selscan_conv1d). With
 * pre[t] = bias + sum_k w[k] xx(t - 3 + k) and g[t] = dout[t] silu'(pre[t]):
 *   dx[b,d,s]      = sum_k w[d,k] g[s + 3 - k]   (terms with 0 <= s + 3 - k < L)
 *   dx_prev[b,d,j] = the same sum for s = j - 3 (the inputs before token 0)
 *   dw[d,k] = sum_{b,t} g[t] xx(t - 3 + k);   dbias[d] = sum_{b,t} g[t]
 * Arguments (device pointers): x, dout, dx [B, d, L] of dtype; w [d, 4] fp32;
 * bias [d] fp32 or NULL; x_prev [B, d, 3] fp32 or NULL (zeros); dw [d, 4]
 * fp32 (output); dbias [d], dx_prev [B, d, 3] fp32 outputs or NULL (not
 * wanted). dims->dstate is ignored. Outputs must not overlap inputs or each
 * other. A workspace of 20 bytes per workgroup of the gradient kernel (at
 * most 20 * max(d, 16384) bytes) is taken with hipMallocAsync on the stream.
 * dw and dbias are sums in a fixed order: deterministic.
 */
int selscan_conv1d_bwd(const void* x, const float* w, const float* bias, const float* x_prev,
                       const void* dout, void* dx, float* dw, float* dbias, float* dx_prev,
                       const selscan_dims_t* dims, void* stream);

/*
 * selscan_conv1d_step — one decode step of the convolution, with the three
 * previous inputs of every row in conv_state [B, d, 3] fp32 (oldest first),
 * updated in place (shifted by one, x appended). Same sources as
 * selscan_conv1d. For every row (b, d):
 *   out[b,d] = silu(bias[d] + w[d,0]*s0 + w[d,1]*s1 + w[d,2]*s2 + w[d,3]*x[b,d])
 *   conv_state[b,d,:] = (s1, s2, x[b,d])
 * x, out: [B, d] of dtype. dims->seqlen and dims->dstate are ignored. Running
 * L steps from conv_state = x_prev equals selscan_conv1d over the L tokens.
 */
int selscan_conv1d_step(float* conv_state, const void* x, const float* w, const float* bias,
                        void* out, const selscan_dims_t* dims, void* stream);

/*
 * Kernel timing for measurement harnesses. selscan_timing_start(capacity)
 * creates capacity pairs of HIP events (once, reused) and from then on every
 * selscan_fwd / selscan_fwd_ex call records one pair on its stream around its
 * output-pass kernel (the kernel that writes y; the B/C repack and, for a
 * split sequence, the state and carry passes are outside the pair) and every
 * selscan_step call around its kernel, until capacity pairs are used.
 * selscan_timing_stop waits for the recorded events, writes the summed
 * elapsed milliseconds and the number of recorded launches, and stops
 * recording. Not thread-safe: one measuring thread at a time.
 * Errors: SELSCAN_ERR_CONFIG (capacity outside 1..65536, or stop without
 * start), SELSCAN_ERR_NULL, SELSCAN_ERR_LAUNCH (a HIP event call failed).
 */
int selscan_timing_start(int32_t capacity);
int selscan_timing_stop(double* total_ms, int32_t* launches);

/* A static, human-readable message for a return code. */
const char* selscan_strerror(int code);

/* Library version as major*10000 + minor*100 + patch. */
int selscan_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SELSCAN_H */
