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
// streams 1 KiB of contiguous state in and out. The per-row scalars (softplus,
// silu) are recomputed by the four lanes rather than exchanged; the readout is
// reduced across the quad with two cross-lane adds.
#include "common.hpp"
#include "launch.hpp"

namespace selscan {
namespace {

template <typename T, bool GATE>
__global__ __launch_bounds__(256) void step_kernel(float* __restrict__ state,
                                                   const T* __restrict__ x,
                                                   const T* __restrict__ delta,
                                                   const float* __restrict__ A,
                                                   const T* __restrict__ B,
                                                   const T* __restrict__ C,
                                                   const float* __restrict__ D,
                                                   const T* __restrict__ z, T* __restrict__ y,
                                                   int64_t rows, int64_t dim) {
    const int64_t gid = int64_t(blockIdx.x) * 256 + threadIdx.x;
    const int64_t row = gid >> 2;
    const int q = int(gid & 3);
    const bool ok = row < rows;
    const int64_t r = ok ? row : rows - 1;  // clamped: every lane reads valid memory
    const int64_t b = r / dim, d = r % dim;

    float4 h = *reinterpret_cast<const float4*>(state + r * kN + q * 4);
    const float4 a4 = *reinterpret_cast<const float4*>(A + d * kN + q * 4);
    float bv[4], cv[4];
    if constexpr (sizeof(T) == 4) {
        const float4 b4 = *reinterpret_cast<const float4*>(B + b * kN + q * 4);
        const float4 c4 = *reinterpret_cast<const float4*>(C + b * kN + q * 4);
        bv[0] = b4.x; bv[1] = b4.y; bv[2] = b4.z; bv[3] = b4.w;
        cv[0] = c4.x; cv[1] = c4.y; cv[2] = c4.z; cv[3] = c4.w;
    } else {
        const uint2 b2 = *reinterpret_cast<const uint2*>(B + b * kN + q * 4);
        const uint2 c2 = *reinterpret_cast<const uint2*>(C + b * kN + q * 4);
        bv[0] = bf16_lo(b2.x); bv[1] = bf16_hi(b2.x); bv[2] = bf16_lo(b2.y); bv[3] = bf16_hi(b2.y);
        cv[0] = bf16_lo(c2.x); cv[1] = bf16_hi(c2.x); cv[2] = bf16_lo(c2.y); cv[3] = bf16_hi(c2.y);
    }
    const float xv = to_f32(x[r]);
    const float l = softplus_log2(to_f32(delta[r]));
    const float w = l * kLn2 * xv;

    h.x = fmaf(exp2_hw(l * a4.x), h.x, w * bv[0]);
    h.y = fmaf(exp2_hw(l * a4.y), h.y, w * bv[1]);
    h.z = fmaf(exp2_hw(l * a4.z), h.z, w * bv[2]);
    h.w = fmaf(exp2_hw(l * a4.w), h.w, w * bv[3]);
    float yp = fmaf(cv[3], h.w, fmaf(cv[2], h.z, fmaf(cv[1], h.y, cv[0] * h.x)));
    if (ok) *reinterpret_cast<float4*>(state + r * kN + q * 4) = h;

    yp += __shfl_xor(yp, 1);
    yp += __shfl_xor(yp, 2);
    if (ok && q == 0) {
        float yv = yp + (D ? D[d] : 0.0f) * xv;
        if constexpr (GATE) yv *= silu(to_f32(z[r]));
        y[r] = from_f32<T>(yv);
    }
}

template <typename T>
hipError_t launch_t(const StepTensors& t, int64_t rows, int64_t dim, hipStream_t st) {
    const int64_t blocks = (rows * 4 + 255) / 256;
    if (t.z)
        hipLaunchKernelGGL((step_kernel<T, true>), dim3(unsigned(blocks)), dim3(256), 0, st,
                           t.state, static_cast<const T*>(t.x), static_cast<const T*>(t.delta), t.A,
                           static_cast<const T*>(t.B), static_cast<const T*>(t.C), t.D,
                           static_cast<const T*>(t.z), static_cast<T*>(t.y), rows, dim);
    else
        hipLaunchKernelGGL((step_kernel<T, false>), dim3(unsigned(blocks)), dim3(256), 0, st,
                           t.state, static_cast<const T*>(t.x), static_cast<const T*>(t.delta), t.A,
                           static_cast<const T*>(t.B), static_cast<const T*>(t.C), t.D,
                           static_cast<const T*>(nullptr), static_cast<T*>(t.y), rows, dim);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_step(const StepTensors& t, int64_t batch, int64_t dim, DType dtype,
                       hipStream_t stream) {
    const int64_t rows = batch * dim;
    return dtype == DType::BF16 ? launch_t<bf16_bits>(t, rows, dim, stream)
                                : launch_t<float>(t, rows, dim, stream);
}

}  // namespace selscan
