// Host-side launchers of the HIP kernels (internal to libselscan).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace selscan {

enum class DType : int { F32 = 0, BF16 = 1 };

// Device pointers of one forward call. x/delta/z/y: [batch, dim, L];
// B/C: [batch, N, L]; A: [dim, N]; D/dt_bias: [dim]; last_state: [batch, dim, N].
struct FwdTensors {
    const void* x;
    const void* delta;
    const void* z;  // null: no gate
    const float* A;
    const void* B;
    const void* C;
    const float* D;        // null: 0
    const float* dt_bias;  // null: 0
    void* y;
    float* last_state;  // null: not wanted
    const float* h0;    // [batch, dim, N] state entering token 0; null: zeros
    float* ckpt;        // [ceil(L/16)][batch*dim][N] states before every 16th token; null: none
    // The block's causal depthwise convolution (width 4) + SiLU applied to x
    // first (null conv_w: none): taps [dim, 4], bias [dim] or null, the 3
    // inputs before token 0 [batch*dim, 3] or null (zeros), and the last 3
    // inputs out [batch*dim, 3] or null.
    const float* conv_w = nullptr;
    const float* conv_b = nullptr;
    const float* conv_x_prev = nullptr;
    float* conv_x_last = nullptr;
};

struct FwdShape {
    int64_t batch, L, dim;
    DType dtype;
};

// How the sequence axis is cut: `segments` runs of `seg_len` tokens each
// (seg_len a multiple of the time tile when segments > 1); `groups` waves per
// 64-row block, each holding N / groups states.
struct FwdPlan {
    int32_t segments;
    int64_t seg_len;
    int32_t groups;  // waves per block of the per-wave kernel; scan waves of the specialised one
    bool vec;  // 16-byte vector access to rows is valid (L * elem_size % 16 == 0)
    // The warp-specialised kernel (scan waves and io waves) instead of the
    // per-wave one; pref: its io waves also load the B/C records of the next
    // chunk into the scalar cache.
    bool ws = false, pref = false;
    // When set, recorded on the stream right before and after the output-pass
    // kernel (measurement only).
    hipEvent_t ev_begin = nullptr, ev_end = nullptr;
};

// Time tile (tokens per chunk) of the forward kernels.
constexpr int kChunk = 32;

// Bytes of workspace a plan needs (0 when segments == 1).
size_t fwd_workspace_bytes(const FwdShape& s, const FwdPlan& p);

// Enqueue the forward pass. `workspace` must hold fwd_workspace_bytes bytes
// (ignored when segments == 1).
hipError_t launch_fwd(const FwdTensors& t, const FwdShape& s, const FwdPlan& p, void* workspace,
                      hipStream_t stream);

// Checkpoint pass of the backward: packs B/C into `packed` (the forward's
// record layout, fwd_workspace_bytes of a one-segment plan), then runs the
// forward recurrence from t.h0 (null: zeros) storing the state before every
// 16th token in ckpt [ceil(L/16)][batch*dim][N] (recompute = false: the pack
// only, the checkpoints being given). 4 waves. With segments > 1
// (seg_len a multiple of kChunk, every segment non-empty) the states entering
// the segments come first, from a state pass into seg_state [segments][rows][N]
// and seg_lsum [segments][rows] and the carries into carry [segments][rows][N].
hipError_t launch_fwd_ckpt(const FwdTensors& t, float* ckpt, const FwdShape& s, float* packed,
                           int32_t segments, int64_t seg_len, float* seg_state, double* seg_lsum,
                           float* carry, bool recompute, hipStream_t stream);

// Carries of a segmented scan, per (row, n): carry[0] = h0 (or 0),
// carry[s+1] = 2^(A[row % dim, n] * seg_lsum[s]) carry[s] + seg_state[s].
hipError_t launch_carry(const float* A, const float* seg_state, const double* seg_lsum,
                        const float* h0, float* carry, int64_t rows, int64_t dim, int32_t segments,
                        hipStream_t stream);

struct StepTensors {
    float* state;
    const void* x;
    const void* delta;
    const float* A;
    const void* B;
    const void* C;
    const float* D;  // null: 0
    const void* z;   // null: no gate
    void* y;
    // The block's convolution (width 4) + SiLU applied to x first (null
    // conv_w: none): taps [dim, 4], bias [dim] or null, and the three previous
    // inputs of every row [rows, 3], shifted in place.
    const float* conv_w = nullptr;
    const float* conv_b = nullptr;
    float* conv_state = nullptr;
};

hipError_t launch_step(const StepTensors& t, int64_t batch, int64_t dim, DType dtype,
                       hipStream_t stream, hipEvent_t ev_begin = nullptr,
                       hipEvent_t ev_end = nullptr);

// Backward pass. x/delta/z/dy and dx/ddelta/dz: [batch, dim, L]; B/C and
// dB/dC: [batch, N, L] (all of the dtype); A/dA: [dim, N]; D/dD, dt_bias/ddt_bias:
// [dim] fp32. z/dz, D/dD, dt_bias/ddt_bias are null together. h0 (the
// forward's initial state), dlast (the gradient flowing into its final state)
// and dh0: [batch, dim, N] fp32, each may be null.
struct BwdTensors {
    const void* x;
    const void* delta;
    const float* A;
    const void* B;
    const void* C;
    const float* D;
    const void* z;
    const float* dt_bias;
    const void* dy;
    void* dx;
    void* ddelta;
    float* dA;
    void* dB;
    void* dC;
    float* dD;
    void* dz;
    float* ddt_bias;
    const float* h0;
    const float* dlast;
    float* dh0;
    const float* ckpt;  // checkpoints from the forward (null: recomputed)
};
// segments > 1: the sequence is cut into segments of seg_len tokens (a
// multiple of kChunk, every segment non-empty), swept in parallel.
size_t bwd_workspace_bytes(int64_t batch, int64_t L, int64_t dim, int32_t segments,
                           bool ckpt_given);
hipError_t launch_bwd(const BwdTensors& t, int64_t batch, int64_t L, int64_t dim, DType dtype,
                      int32_t segments, int64_t seg_len, void* workspace, hipStream_t stream);

// Mamba-2 SSD layer (bf16). x/y: [batch, L, heads, 64]; delta: [batch, L, heads];
// A, D, dt_bias: [heads] fp32; B, C: [batch, L, dstate]; last_state and h0
// (the state entering token 0): [batch, heads, dstate, 64] fp32 or null.
// dstate 64 or 128.
struct SsdTensors {
    const void* x;
    const void* delta;
    const float* A;
    const void* B;
    const void* C;
    const float* D;
    const float* dt_bias;
    void* y;
    float* last_state;
    const float* h0;
};
hipError_t launch_ssd(const SsdTensors& t, int64_t batch, int64_t L, int64_t heads, int64_t dstate,
                      hipStream_t stream);

// One decode step of the SSD layer: state [batch, heads, dstate, 64] fp32 in
// place; x/y: [batch, heads, 64], delta: [batch, heads], B/C: [batch, dstate]
// (bf16); A, D, dt_bias: [heads] fp32 (D, dt_bias may be null).
struct SsdStepTensors {
    float* state;
    const void* x;
    const void* delta;
    const float* A;
    const void* B;
    const void* C;
    const float* D;
    const float* dt_bias;
    void* y;
};
hipError_t launch_ssd_step(const SsdStepTensors& t, int64_t batch, int64_t heads, int64_t dstate,
                           hipStream_t stream);

// Causal depthwise conv (width 4) + SiLU. x/out: [rows, L]; w: [dim, 4];
// bias: [dim] or null; x_prev/x_last: [rows, 3] fp32 or null.
struct ConvTensors {
    const void* x;
    const float* w;
    const float* bias;
    const float* x_prev;
    void* out;
    float* x_last;
};
hipError_t launch_conv(const ConvTensors& t, int64_t rows, int64_t L, int64_t dim, DType dtype,
                       hipStream_t stream);

// Gradients of the convolution + SiLU for dout: dx [rows, L] of the dtype,
// dw [dim, 4] fp32, dbias [dim] fp32 or null, dx_prev [rows, 3] fp32 or null
// (the inputs before token 0).
struct ConvBwdTensors {
    const void* x;
    const float* w;
    const float* bias;
    const float* x_prev;
    const void* dout;
    void* dx;
    float* dw;
    float* dbias;
    float* dx_prev;
};
// Work split of the gradient kernel: per channel, `bgroups` groups of batch
// entries times `pieces` pieces of the sequence, one workgroup each.
struct ConvBwdPlan {
    int32_t bgroups, pieces;
};
ConvBwdPlan conv_bwd_plan(int64_t batch, int64_t L, int64_t dim, DType dtype);
// part: dim * bgroups * pieces * 5 floats of workspace.
hipError_t launch_conv_bwd(const ConvBwdTensors& t, int64_t batch, int64_t L, int64_t dim,
                           DType dtype, float* part, ConvBwdPlan plan, hipStream_t stream);

// x_last[r] = the last three entries of x_prev[r] ++ x[r] (x: [rows, L] of the
// dtype; x_prev, x_last: [rows, 3] fp32, x_prev may be null, x_last may be x_prev).
hipError_t launch_conv_last(const void* x, const float* x_prev, float* x_last, int64_t rows,
                            int64_t L, DType dtype, hipStream_t stream);

struct ConvStepTensors {
    float* state;  // [rows, 3], oldest first, updated in place
    const void* x;
    const float* w;
    const float* bias;
    void* out;
};
hipError_t launch_conv_step(const ConvStepTensors& t, int64_t rows, int64_t dim, DType dtype,
                            hipStream_t stream);

}  // namespace selscan
