// One-token decode step of the selective scan (S6) for gfx950.
//
// "State Space Models and Mamba" (multigrid.ai), section "Why a linear
// recurrence can be trained in parallel": at inference time the layer runs the
// recurrence one token at a time on a fixed-size state. Per (b, d) row:
//     delta = softplus(delta_in)
//     h_n  <- exp(delta A_dn) h_n + delta B_n x
//     y     = (sum_n C_n h_n + D_d x) silu(z)
//
// The step is bound by HBM: the fp32 state (64 bytes per row) is read and
// written once; everything else is a few bytes per row. Four consecutive lanes
// share a row, each owning four states as one 16-byte vector, so every wave
// streams 1 KiB of contiguous state in and out, with non-temporal accesses
// (the state is touched once per step, and between two steps of a layer the
// rest of the model runs). The per-row scalars (softplus, silu) are recomputed
// by the four lanes rather than exchanged; the readout is reduced across the
// quad with two cross-lane adds. Each thread takes two quads (measured against
// one and four: 38 and 40 us per step at batch 256 x d_inner 5120 with cached
// state accesses, 35 us non-temporal at two), of one channel in two batch
// entries (below).
//
// With the block's convolution fused in front ("State Space Models and
// Mamba" (multigrid.ai), section "What a Mamba block actually contains": a
// width-4 causal depthwise conv1d and a SiLU feed the selective SSM), the
// step's input is u = silu(b_d + w_d . (s0, s1, s2, x)) from the row's three
// previous inputs s, which lane 0 of the quad then shifts (s1, s2, x); u is
// kept in fp32 and D multiplies it.
#include "common.hpp"
#include "launch.hpp"

namespace selscan {
namespace {

typedef float f32x4v __attribute__((ext_vector_type(4)));

// A block takes 64 channels d (4 lanes each) of R consecutive batch entries:
// each thread owns the quad (lane q of 4) of channel d in R rows
// (b, d), ..., (b + R - 1, d), so the channel's A (and the convolution's
// taps) are loaded once for R rows, and every wave's state access is 1 KiB
// of contiguous memory per row set. All of a thread's loads are issued before
// any arithmetic. Measured at batch 256 x d_inner 5120 (bf16): 32.3 us per
// step back to back and 35.3 cold, against 33.6 / 36.6 with the thread's two
// quads in consecutive channels of one batch entry (A loaded twice).
template <typename T, bool GATE, bool CONV, int R>
__global__ __launch_bounds__(256) void step_kernel(float* __restrict__ state,
                                                   const T* __restrict__ x,
                                                   const T* __restrict__ delta,
                                                   const float* __restrict__ A,
                                                   const T* __restrict__ B,
                                                   const T* __restrict__ C,
                                                   const float* __restrict__ D,
                                                   const T* __restrict__ z, T* __restrict__ y,
                                                   const float* __restrict__ conv_w,
                                                   const float* __restrict__ conv_b,
                                                   float* __restrict__ conv_state, int64_t batch,
                                                   int64_t dim) {
    const int64_t dblocks = (dim + 63) / 64;
    const int64_t db = blockIdx.x % dblocks, bg = blockIdx.x / dblocks;
    const int q = int(threadIdx.x & 3);
    const int64_t d0 = db * 64 + (threadIdx.x >> 2);
    const bool d_ok = d0 < dim;
    const int64_t d = d_ok ? d0 : dim - 1;  // clamped: every lane reads valid memory
    const float4 a4 = *reinterpret_cast<const float4*>(A + d * kN + q * 4);
    const float Dd = D ? D[d] : 0.0f;
    float4 cw = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    float cb = 0.0f;
    if constexpr (CONV) {
        cw = *reinterpret_cast<const float4*>(conv_w + d * 4);
        cb = conv_b ? conv_b[d] : 0.0f;
    }
    float4 h[R];
    float bv[R][4], cv[R][4], xv[R], dv[R], zv[R], cs[R][3];
    int64_t rr[R];
    bool ok[R];
#pragma unroll
    for (int k = 0; k < R; ++k) {
        const int64_t b0 = bg * R + k;
        ok[k] = d_ok && b0 < batch;
        const int64_t b = b0 < batch ? b0 : batch - 1;
        const int64_t r = b * dim + d;
        rr[k] = r;
        { const f32x4v hv = __builtin_nontemporal_load(reinterpret_cast<const f32x4v*>(state + r * kN + q * 4)); h[k] = make_float4(hv.x, hv.y, hv.z, hv.w); }
        if constexpr (sizeof(T) == 4) {
            const float4 b4 = *reinterpret_cast<const float4*>(B + b * kN + q * 4);
            const float4 c4 = *reinterpret_cast<const float4*>(C + b * kN + q * 4);
            bv[k][0] = b4.x; bv[k][1] = b4.y; bv[k][2] = b4.z; bv[k][3] = b4.w;
            cv[k][0] = c4.x; cv[k][1] = c4.y; cv[k][2] = c4.z; cv[k][3] = c4.w;
        } else {
            const uint2 b2 = *reinterpret_cast<const uint2*>(B + b * kN + q * 4);
            const uint2 c2 = *reinterpret_cast<const uint2*>(C + b * kN + q * 4);
            bv[k][0] = bf16_lo(b2.x); bv[k][1] = bf16_hi(b2.x); bv[k][2] = bf16_lo(b2.y); bv[k][3] = bf16_hi(b2.y);
            cv[k][0] = bf16_lo(c2.x); cv[k][1] = bf16_hi(c2.x); cv[k][2] = bf16_lo(c2.y); cv[k][3] = bf16_hi(c2.y);
        }
        xv[k] = to_f32(x[r]);
        dv[k] = to_f32(delta[r]);
        zv[k] = GATE ? to_f32(z[r]) : 0.0f;
        if constexpr (CONV) {
            cs[k][0] = conv_state[r * 3 + 0];
            cs[k][1] = conv_state[r * 3 + 1];
            cs[k][2] = conv_state[r * 3 + 2];
        }
    }
#pragma unroll
    for (int k = 0; k < R; ++k) {
        if constexpr (CONV) {
            const float xr = xv[k];
            xv[k] = silu(fmaf(cw.w, xr, fmaf(cw.z, cs[k][2], fmaf(cw.y, cs[k][1], fmaf(cw.x, cs[k][0], cb)))));
            if (ok[k] && q == 0) {
                conv_state[rr[k] * 3 + 0] = cs[k][1];
                conv_state[rr[k] * 3 + 1] = cs[k][2];
                conv_state[rr[k] * 3 + 2] = xr;
            }
        }
        const float l = softplus_log2(dv[k]);
        const float w = l * kLn2 * xv[k];
        h[k].x = fmaf(exp2_hw(l * a4.x), h[k].x, w * bv[k][0]);
        h[k].y = fmaf(exp2_hw(l * a4.y), h[k].y, w * bv[k][1]);
        h[k].z = fmaf(exp2_hw(l * a4.z), h[k].z, w * bv[k][2]);
        h[k].w = fmaf(exp2_hw(l * a4.w), h[k].w, w * bv[k][3]);
        if (ok[k]) { f32x4v hv = {h[k].x, h[k].y, h[k].z, h[k].w}; __builtin_nontemporal_store(hv, reinterpret_cast<f32x4v*>(state + rr[k] * kN + q * 4)); }
        float yp = fmaf(cv[k][3], h[k].w, fmaf(cv[k][2], h[k].z, fmaf(cv[k][1], h[k].y, cv[k][0] * h[k].x)));
        yp += __shfl_xor(yp, 1);
        yp += __shfl_xor(yp, 2);
        if (ok[k] && q == 0) {
            float yv = yp + Dd * xv[k];
            if constexpr (GATE) yv *= silu(zv[k]);
            y[rr[k]] = from_f32<T>(yv);
        }
    }
}

constexpr int kStepR = 2;

template <typename T, bool GATE, bool CONV>
hipError_t launch_v(const StepTensors& t, int64_t batch, int64_t dim, hipStream_t st) {
    const int64_t blocks = (dim + 63) / 64 * ((batch + kStepR - 1) / kStepR);
    if (blocks > int64_t(0xffffffff)) return hipErrorInvalidValue;
    hipLaunchKernelGGL((step_kernel<T, GATE, CONV, kStepR>), dim3(unsigned(blocks)), dim3(256), 0, st,
                       t.state, static_cast<const T*>(t.x), static_cast<const T*>(t.delta), t.A,
                       static_cast<const T*>(t.B), static_cast<const T*>(t.C), t.D,
                       static_cast<const T*>(t.z), static_cast<T*>(t.y), t.conv_w, t.conv_b,
                       t.conv_state, batch, dim);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_t(const StepTensors& t, int64_t batch, int64_t dim, hipStream_t st) {
    if (t.conv_w)
        return t.z ? launch_v<T, true, true>(t, batch, dim, st) : launch_v<T, false, true>(t, batch, dim, st);
    return t.z ? launch_v<T, true, false>(t, batch, dim, st) : launch_v<T, false, false>(t, batch, dim, st);
}

}  // namespace

hipError_t launch_step(const StepTensors& t, int64_t batch, int64_t dim, DType dtype,
                       hipStream_t stream, hipEvent_t ev_begin, hipEvent_t ev_end) {
    if (ev_begin && hipEventRecord(ev_begin, stream) != hipSuccess) return hipGetLastError();
    const hipError_t e = dtype == DType::BF16 ? launch_t<bf16_bits>(t, batch, dim, stream)
                                              : launch_t<float>(t, batch, dim, stream);
    if (e != hipSuccess) return e;
    if (ev_end && hipEventRecord(ev_end, stream) != hipSuccess) return hipGetLastError();
    return hipSuccess;
}

}  // namespace selscan
