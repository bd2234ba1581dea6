// Copy kernels of known size for calibrating the HBM byte counters against
// the access patterns of the scan kernels (see include/selscan_calib.h).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/selscan_calib.h"

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int64_t kRowBytes = 4096;   // mode 2: one row
constexpr int64_t kPiece = 64;        // mode 2: bytes of a row per step (4 lanes x 16 B)

template <bool NT>
__global__ __launch_bounds__(256) void copy_flat(const u32x4* __restrict__ src,
                                                 u32x4* __restrict__ dst, int64_t n) {
    const int64_t stride = int64_t(gridDim.x) * 256;
    for (int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x; i < n; i += stride) {
        if constexpr (NT) {
            __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
        } else {
            dst[i] = src[i];
        }
    }
}

// Block = 64 rows; thread (r, q) = (tid / 4, tid % 4) copies bytes
// [k*64 + q*16, +16) of row r for k = 0..63.
__global__ __launch_bounds__(256) void copy_rows(const unsigned char* __restrict__ src,
                                                 unsigned char* __restrict__ dst) {
    const int r = threadIdx.x / 4, q = threadIdx.x % 4;
    const int64_t base = (int64_t(blockIdx.x) * 64 + r) * kRowBytes + q * 16;
    for (int64_t k = 0; k < kRowBytes / kPiece; ++k) {
        const u32x4* s = reinterpret_cast<const u32x4*>(src + base + k * kPiece);
        u32x4* d = reinterpret_cast<u32x4*>(dst + base + k * kPiece);
        __builtin_nontemporal_store(__builtin_nontemporal_load(s), d);
    }
}

typedef float f32x16 __attribute__((ext_vector_type(16)));
__device__ __forceinline__ f32x16 sload64(const float* p) {
    using CP = const __attribute__((address_space(4))) f32x16*;
    return *(CP)(reinterpret_cast<uintptr_t>(p));
}

// The forward kernel's inner loop alone, from on-chip operands: per lane 4
// states, per token and state one multiply (l*A), one v_exp_f32, one multiply
// (w*B, B a scalar operand) and two FMAs (state, readout). B and C come from
// a small hot buffer by s_load_dwordx16 one 4-token sub-block ahead, (l, w)
// from LDS, exactly as in the forward kernel; no HBM traffic, no barriers.
// Its rate is the measured ceiling of this instruction mix.
__global__ __launch_bounds__(256) void scan_mix(const float* __restrict__ rec, float* __restrict__ out,
                                                int32_t nsub) {
    constexpr int NG = 4, SB = 4;
    __shared__ float2 lw[16][64];
    const int tid = threadIdx.x, lane = tid % 64;
    const int wv = __builtin_amdgcn_readfirstlane(tid / 64);
    if (tid < 64)
        for (int e = 0; e < 16; ++e)
            lw[e][lane] = make_float2(-0.01f * float(1 + (e + lane) % 7), 0.001f * float(e + 1));
    __syncthreads();
    float An[NG], h[NG];
    for (int j = 0; j < NG; ++j) {
        An[j] = -1.0f - float(j) - float(lane) * 1e-3f;
        h[j] = 0.0f;
    }
    f32x16 B0 = sload64(rec + wv * 32), C0 = sload64(rec + wv * 32 + 16), B1, C1;
    float2 l0[SB], l1[SB];
    for (int e = 0; e < SB; ++e) l0[e] = lw[e][lane];
    float tot = 0.0f;
    auto half = [&](int sb, const f32x16& Bc, const f32x16& Cc, const float2* lc, f32x16& Bn,
                    f32x16& Cn, float2* ln) {
        __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
        __builtin_amdgcn_sched_barrier(0);
        const float* nr = rec + ((sb + 1) & 63) * 128 + wv * 32;
        Bn = sload64(nr);
        Cn = sload64(nr + 16);
        for (int e = 0; e < SB; ++e) ln[e] = lw[((sb + 1) * SB + e) & 15][lane];
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int e = 0; e < SB; ++e) {
            float acc = 0.0f;
#pragma unroll
            for (int j = 0; j < NG; ++j) {
                const float dA = __builtin_amdgcn_exp2f(lc[e].x * An[j]);
                h[j] = fmaf(dA, h[j], lc[e].y * Bc[j * SB + e]);
                acc = fmaf(Cc[j * SB + e], h[j], acc);
            }
            tot += acc;
        }
    };
#pragma unroll 1
    for (int sb = 0; sb < nsub; sb += 2) {
        half(sb, B0, C0, l0, B1, C1, l1);
        half(sb + 1, B1, C1, l1, B0, C0, l0);
    }
    float s = tot;
    for (int j = 0; j < NG; ++j) s += h[j];
    out[int64_t(blockIdx.x) * 256 + tid] = s;
}

}  // namespace

extern "C" int selscan_calib_scan_mix(const float* rec, float* out, int32_t blocks, int32_t nsub,
                                      void* stream) {
    if (!rec || !out) return -1;
    if (blocks < 1 || nsub < 2 || nsub % 2) return -2;
    hipLaunchKernelGGL(scan_mix, dim3(unsigned(blocks)), dim3(256), 0, static_cast<hipStream_t>(stream),
                       rec, out, nsub);
    return hipGetLastError() == hipSuccess ? 0 : -5;
}

extern "C" int selscan_calib_copy(const void* src, void* dst, int64_t bytes, int32_t mode,
                                  void* stream) {
    if (!src || !dst) return -1;
    if (bytes <= 0 || bytes % 16) return -2;
    if ((reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst)) & 15u) return -7;
    hipStream_t st = static_cast<hipStream_t>(stream);
    const int64_t n = bytes / 16;
    const auto* s = static_cast<const u32x4*>(src);
    auto* d = static_cast<u32x4*>(dst);
    const int64_t blocks = n / 256 < 8192 ? (n + 255) / 256 : 8192;
    switch (mode) {
        case 0: hipLaunchKernelGGL(copy_flat<false>, dim3(unsigned(blocks)), dim3(256), 0, st, s, d, n); break;
        case 1: hipLaunchKernelGGL(copy_flat<true>, dim3(unsigned(blocks)), dim3(256), 0, st, s, d, n); break;
        case 2: {
            if (bytes % (64 * kRowBytes)) return -2;
            const int64_t rblocks = bytes / (64 * kRowBytes);
            hipLaunchKernelGGL(copy_rows, dim3(unsigned(rblocks)), dim3(256), 0, st,
                               static_cast<const unsigned char*>(src), static_cast<unsigned char*>(dst));
            break;
        }
        default: return -9;
    }
    return hipGetLastError() == hipSuccess ? 0 : -5;
}
