// Device helpers shared by the selective-scan kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace selscan {

using bf16_bits = uint16_t;  // bfloat16 storage: the upper half of an fp32

constexpr int kWave = 64;    // CDNA wavefront width
constexpr int kN = 16;       // supported state size

constexpr float kLog2e = 1.44269504088896340736f;
constexpr float kLn2 = 0.69314718055994530942f;

// ---- storage conversions -------------------------------------------------

__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(bf16_bits v) { return __uint_as_float(uint32_t(v) << 16); }

template <typename T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }
// Round to nearest even through the hardware conversion (v_cvt_pk_bf16_f32).
template <> __device__ __forceinline__ bf16_bits from_f32<bf16_bits>(float v) {
    return __builtin_bit_cast(bf16_bits, (__bf16)v);
}

// Workgroups are handed to the 8 XCDs (each with its own L2) round robin:
// workgroup i runs on XCD i % 8. xcd_tile renumbers them so that consecutive
// tile numbers run on one XCD: of n = 8 q + r workgroups, XCD x takes the
// tiles from x q + min(x, r) on, q + 1 of them if x < r, else q. Tiles that
// read the same data (the row blocks of one batch entry and segment, which
// share its B/C records) then share an L2.
__device__ __forceinline__ int64_t xcd_tile(int64_t i, int64_t n) {
    const int64_t q = n / 8, r = n % 8, x = i % 8;
    return x * q + (x < r ? x : r) + i / 8;
}

// Two floats rounded to bfloat16 (nearest even) and packed low, high into a
// 32-bit word: one v_cvt_pk_bf16_f32.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, v);
}

// The two bfloat16 halves of a 32-bit word, as fp32.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// ---- the scalar functions of the method -----------------------------------
//
// The hardware transcendentals work in base 2: v_exp_f32 is 2^x, v_log_f32 is
// log2(x), v_rcp_f32 is 1/x. The step size is therefore carried in log2 units,
// l = softplus(u) / ln 2, so that the decay exp(delta * A) is 2^(l * A) with a
// single multiply, and delta itself is l * ln 2.

__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float log2_hw(float x) { return __builtin_amdgcn_logf(x); }
__device__ __forceinline__ float rcp_hw(float x) { return __builtin_amdgcn_rcpf(x); }

// softplus(u) / ln 2 = max(u, 0)/ln 2 + log2(1 + e^{-|u|}), from ul = u / ln 2.
// log2(1 + e) is taken from w = fl(1 + e) plus a first-order correction for
// the rounding of w: with c = e - (w - 1) (exact), ln(1 + e) = ln(w) + c/w
// + O(c^2). The factor 1/w is dropped: the term it changes is below
// 2^-24 * log2(e) * (1 - 1/w), under one ulp of the result whether e is near
// 1 (result >= 1) or small (then 1 - 1/w is about e, a relative 2^-24). This
// keeps the relative accuracy of small step sizes (u very negative), where
// 1 + e rounds to 1.
__device__ __forceinline__ float softplus_log2_of(float ul) {
    const float e = exp2_hw(-fabsf(ul));
    const float w = 1.0f + e;
    const float c = e - (w - 1.0f);
    return fmaxf(ul, 0.0f) + fmaf(c, kLog2e, log2_hw(w));
}
__device__ __forceinline__ float softplus_log2(float u) { return softplus_log2_of(u * kLog2e); }

// silu(z) = z * sigmoid(z) = z / (1 + e^{-z}); saturates cleanly at both ends.
__device__ __forceinline__ float silu(float z) {
    return z * rcp_hw(1.0f + exp2_hw(-z * kLog2e));
}

// silu'(z) = sig(z) (1 + z (1 - sig(z))), sig(z) = 1 / (1 + e^{-z}).
__device__ __forceinline__ float silu_grad(float z) {
    const float sg = rcp_hw(1.0f + exp2_hw(-z * kLog2e));
    return sg * fmaf(z, 1.0f - sg, 1.0f);
}

}  // namespace selscan
