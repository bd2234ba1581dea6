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

}  // namespace

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
