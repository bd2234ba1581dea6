// Mamba-2's state space dual (SSD) layer on gfx950 matrix cores.
//
// The restricted selective SSM of the state space duality ("State Space
// Models Explained: How Mamba Works and How It Compares to Transformers"
// (mernstackdev.com), section "From S4 to Mamba"; "State space models and
// Mamba: reading long sequences without attention" (ai-trend.me), section
// "How it developed: from S4 to Mamba and Mamba-2"): one scalar decay
// a_t = exp(delta_t A_h) per token and head, heads of P channels, B and C
// shared by the heads. Per batch entry and head, with S the N x P state:
//     S_t = a_t S_{t-1} + delta_t B_t x_t^T,   y_t = C_t^T S_t + D_h x_t.
// Its dual is a masked matrix product, y = (L o C B^T)(delta x) + D x with
// L[t,s] = a_{s+1} ... a_t, a semiseparable matrix; cutting the sequence into
// chunks of Q tokens splits it into diagonal blocks (small dense products)
// and low-rank off-diagonal parts carried by the chunk states. That is what
// makes the layer matrix-multiply work:
//   chunk_state: S_c = sum_{s in c} exp(cum_end - cum_s) delta_s B_s x_s^T
//   state_pass:  H_{c+1} = exp(cum_end(c)) H_c + S_c       (sequential in c)
//   chunk_scan:  y_t = sum_{s<=t in c} [C_t.B_s] exp(cum_t - cum_s) delta_s x_s
//                      + exp(cum_t) C_t^T H_c + D x_t
// with cum the running sum of delta A within the chunk (base 2 here). The
// products run on v_mfma_f32_32x32x16_bf16: bf16 operands (the inputs, and
// the masked-and-scaled score and scaled C rounded to bf16), fp32 sums.
//
// One workgroup (4 waves) per (batch, head, chunk of 64 tokens); headdim 64,
// dstate 64 or 128. Tiles are staged in LDS with rows padded by 16 bytes so
// that the 16-byte operand reads of 32 lanes on 32 rows spread over the banks.
#include "common.hpp"
#include "launch.hpp"

namespace selscan {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kQ = 64;   // tokens per chunk
constexpr int kP = 64;   // headdim

__device__ __forceinline__ f32x16 mfma(const bf16x8& a, const bf16x8& b, const f32x16& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
// 8 consecutive bf16 from LDS (16 bytes, aligned).
__device__ __forceinline__ bf16x8 lds8(const bf16_bits* p) {
    return *reinterpret_cast<const bf16x8*>(p);
}
__device__ __forceinline__ bf16_bits tobf(float v) { return from_f32<bf16_bits>(v); }

// 8 bf16 (16 bytes) from global memory, or zeros.
__device__ __forceinline__ uint4 ld8(const bf16_bits* p, bool ok) {
    return ok ? *reinterpret_cast<const uint4*>(p) : make_uint4(0, 0, 0, 0);
}
__device__ __forceinline__ bf16_bits lo16(uint32_t w) { return bf16_bits(w & 0xffffu); }
__device__ __forceinline__ bf16_bits hi16(uint32_t w) { return bf16_bits(w >> 16); }
// The 8 values of a 16-byte piece, as bf16 bits, in order.
__device__ __forceinline__ void split8(const uint4& v, bf16_bits* o) {
    o[0] = lo16(v.x); o[1] = hi16(v.x); o[2] = lo16(v.y); o[3] = hi16(v.y);
    o[4] = lo16(v.z); o[5] = hi16(v.z); o[6] = lo16(v.w); o[7] = hi16(v.w);
}
__device__ __forceinline__ float bfval(bf16_bits v) { return __uint_as_float(uint32_t(v) << 16); }

struct SsdArgs {
    const bf16_bits* x;     // [batch, L, H, P]
    const bf16_bits* delta; // [batch, L, H]
    const float* A;         // [H]
    const bf16_bits* B;     // [batch, L, N]
    const bf16_bits* C;     // [batch, L, N]
    const float* D;         // [H] or null
    const float* dt_bias;   // [H] or null
    bf16_bits* y;           // [batch, L, H, P]
    float* last_state;      // [batch, H, N, P] or null
    float* S;               // [batch*H*nc][P][N] chunk states (transposed)
    float* tot;             // [batch*H*nc] base-2 log of the chunk's total decay
    bf16_bits* Hin;         // [batch*H*nc][P][N] state entering each chunk (transposed)
    int64_t batch, L, H;
    int32_t nc;
};

// delta_t and the running sum of log2-decays of the chunk's tokens, into LDS;
// tokens past L get delta 0 (an identity step). One wave computes the scan.
template <int N>
__device__ __forceinline__ void chunk_decays(const SsdArgs& a, int64_t b, int64_t h, int c, float* dts,
                                             float* cum) {
    const int tid = threadIdx.x;
    if (tid < kQ) {
        const int64_t t = int64_t(c) * kQ + tid;
        float dt = 0.0f;
        if (t < a.L) {
            const float u = to_f32(a.delta[(b * a.L + t) * a.H + h]) + (a.dt_bias ? a.dt_bias[h] : 0.0f);
            dt = softplus_log2(u) * kLn2;
        }
        float v = dt * a.A[h] * kLog2e;  // log2 of this token's decay
#pragma unroll
        for (int o = 1; o < kQ; o <<= 1) {
            const float w = __shfl_up(v, o, kQ);
            if (tid >= o) v += w;
        }
        dts[tid] = dt;
        cum[tid] = v;
    }
}

// ---- chunk_state: S_c^T[p][n] = sum_s x[s][p] w_s B[s][n], w_s = 2^(cum_end - cum_s) delta_s ----
template <int N>
__global__ __launch_bounds__(256) void ssd_chunk_state(SsdArgs a) {
    constexpr int QR = kQ + 8;
    __shared__ alignas(16) bf16_bits Bt[N * QR];    // B^T: [n][s]
    __shared__ alignas(16) bf16_bits Xt[kP * QR];   // (w x)^T: [p][s]
    __shared__ float dts[kQ], cum[kQ];
    const int tid = threadIdx.x, lane = tid % 64, wv = tid / 64;
    const int c = int(blockIdx.x % unsigned(a.nc));
    const int64_t bh = blockIdx.x / unsigned(a.nc);
    const int64_t b = bh / a.H, h = bh % a.H;
    chunk_decays<N>(a, b, h, c, dts, cum);
    __syncthreads();
    const float cend = cum[kQ - 1];
    // Stage B^T and (w x)^T, both transposed: a thread loads a 16-byte piece
    // (8 consecutive n, or p) of one token's row and writes it down a column;
    // consecutive threads take consecutive tokens, so the 2-byte LDS writes
    // of a wave fall in distinct banks.
    for (int i = tid; i < kQ * (N / 8); i += 256) {
        const int s = i % kQ, q8 = i / kQ;
        const int64_t t = int64_t(c) * kQ + s;
        bf16_bits v[8];
        split8(ld8(a.B + (b * a.L + t) * N + q8 * 8, t < a.L), v);
#pragma unroll
        for (int e = 0; e < 8; ++e) Bt[(q8 * 8 + e) * QR + s] = v[e];
    }
    for (int i = tid; i < kQ * (kP / 8); i += 256) {
        const int s = i % kQ, q8 = i / kQ;
        const int64_t t = int64_t(c) * kQ + s;
        const bool ok = t < a.L;
        const float w = ok ? exp2_hw(cend - cum[s]) * dts[s] : 0.0f;
        bf16_bits v[8];
        split8(ld8(a.x + ((b * a.L + t) * a.H + h) * kP + q8 * 8, ok), v);
#pragma unroll
        for (int e = 0; e < 8; ++e) Xt[(q8 * 8 + e) * QR + s] = tobf(w * bfval(v[e]));
    }
    __syncthreads();
    // S^T [P x N] = Xt [P x Q] . Bt^T [Q x N]; tiles of 32 x 32: (P/32) x (N/32), split over 4 waves
    constexpr int TI = kP / 32, TJ = N / 32, TILES = TI * TJ, PER = TILES / 4;
    const int64_t base = (bh * a.nc + c) * int64_t(kP) * N;
#pragma unroll
    for (int u = 0; u < PER; ++u) {
        const int tile = wv * PER + u;
        const int ti = tile / TJ, tj = tile % TJ;
        f32x16 acc = {};
#pragma unroll
        for (int ks = 0; ks < kQ / 16; ++ks) {
            const int k0 = ks * 16 + 8 * (lane / 32);
            const bf16x8 av = lds8(&Xt[(ti * 32 + lane % 32) * QR + k0]);
            const bf16x8 bv = lds8(&Bt[(tj * 32 + lane % 32) * QR + k0]);
            acc = mfma(av, bv, acc);
        }
        // acc[r] = S^T[ti*32 + 8*(r/4) + 4*(lane/32) + r%4][tj*32 + lane%32]
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int p = ti * 32 + 8 * (r / 4) + 4 * (lane / 32) + r % 4;
            const int n = tj * 32 + lane % 32;
            a.S[base + int64_t(p) * N + n] = acc[r];
        }
    }
    if (tid == 0) a.tot[bh * a.nc + c] = cend;
}

// ---- state_pass: H_in[c] = state entering chunk c; H <- 2^tot_c H + S_c ----
template <int N>
__global__ __launch_bounds__(256) void ssd_state_pass(SsdArgs a) {
    constexpr int E = kP * N / 256;  // elements per thread
    const int64_t bh = blockIdx.x;
    const int tid = threadIdx.x;
    float H[E];
#pragma unroll
    for (int e = 0; e < E; ++e) H[e] = 0.0f;
    for (int c = 0; c < a.nc; ++c) {
        const int64_t base = (bh * a.nc + c) * int64_t(kP) * N;
        const float g = exp2_hw(a.tot[bh * a.nc + c]);
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const int64_t i = int64_t(e) * 256 + tid;
            a.Hin[base + i] = tobf(H[e]);
            H[e] = fmaf(g, H[e], a.S[base + i]);
        }
    }
    if (a.last_state) {
        const int64_t b = bh / a.H, h = bh % a.H;
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const int i = e * 256 + tid;      // = p * N + n
            const int p = i / N, n = i % N;
            a.last_state[((b * a.H + h) * N + n) * kP + p] = H[e];
        }
    }
}

// ---- chunk_scan: y = (L o C B^T)(delta x) + (2^cum o C) H_in + D x ----
template <int N>
__global__ __launch_bounds__(256) void ssd_chunk_scan(SsdArgs a) {
    constexpr int NR = N + 8;
    constexpr int QR = kQ + 8;
    __shared__ alignas(16) bf16_bits Cs[kQ * NR];   // C rows [t][n]
    __shared__ alignas(16) bf16_bits Cw[kQ * NR];   // 2^cum_t C rows [t][n]
    __shared__ alignas(16) bf16_bits Bs[kQ * NR];   // B rows [s][n]
    __shared__ alignas(16) bf16_bits Xt[kP * QR];   // x^T [p][s]
    __shared__ alignas(16) bf16_bits Ms[kQ * QR];   // masked, scaled scores [t][s]
    __shared__ float dts[kQ], cum[kQ];
    const int tid = threadIdx.x, lane = tid % 64, wv = tid / 64;
    const int c = int(blockIdx.x % unsigned(a.nc));
    const int64_t bh = blockIdx.x / unsigned(a.nc);
    const int64_t b = bh / a.H, h = bh % a.H;
    chunk_decays<N>(a, b, h, c, dts, cum);
    __syncthreads();
    // C and B rows as they are (16-byte pieces, consecutive threads on
    // consecutive pieces of a row), C scaled by 2^cum_t as well; x transposed
    // (consecutive threads on consecutive tokens).
    for (int i = tid; i < kQ * (N / 8); i += 256) {
        const int s = i / (N / 8), q8 = i % (N / 8);
        const int64_t t = int64_t(c) * kQ + s;
        const bool ok = t < a.L;
        const uint4 cv = ld8(a.C + (b * a.L + t) * N + q8 * 8, ok);
        *reinterpret_cast<uint4*>(&Cs[s * NR + q8 * 8]) = cv;
        *reinterpret_cast<uint4*>(&Bs[s * NR + q8 * 8]) = ld8(a.B + (b * a.L + t) * N + q8 * 8, ok);
        const float gw = exp2_hw(cum[s]);
        bf16_bits v[8];
        split8(cv, v);
        uint32_t wv4[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
            wv4[e] = uint32_t(tobf(gw * bfval(v[2 * e]))) | (uint32_t(tobf(gw * bfval(v[2 * e + 1]))) << 16);
        *reinterpret_cast<uint4*>(&Cw[s * NR + q8 * 8]) = make_uint4(wv4[0], wv4[1], wv4[2], wv4[3]);
    }
    for (int i = tid; i < kQ * (kP / 8); i += 256) {
        const int s = i % kQ, q8 = i / kQ;
        const int64_t t = int64_t(c) * kQ + s;
        bf16_bits v[8];
        split8(ld8(a.x + ((b * a.L + t) * a.H + h) * kP + q8 * 8, t < a.L), v);
#pragma unroll
        for (int e = 0; e < 8; ++e) Xt[(q8 * 8 + e) * QR + s] = v[e];
    }
    __syncthreads();
    // scores G = C B^T [Q x Q], one 32 x 32 tile per wave: (t block, s block)
    {
        const int tb = wv / 2, sb = wv % 2;
        f32x16 g = {};
        if (sb <= tb) {
#pragma unroll
            for (int ks = 0; ks < N / 16; ++ks) {
                const int k0 = ks * 16 + 8 * (lane / 32);
                g = mfma(lds8(&Cs[(tb * 32 + lane % 32) * NR + k0]), lds8(&Bs[(sb * 32 + lane % 32) * NR + k0]), g);
            }
        }
        // M[t][s] = G[t][s] 2^(cum_t - cum_s) delta_s for s <= t, else 0
        const int s = sb * 32 + lane % 32;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int t = tb * 32 + 8 * (r / 4) + 4 * (lane / 32) + r % 4;
            const float m = s <= t ? g[r] * exp2_hw(cum[t] - cum[s]) * dts[s] : 0.0f;
            Ms[t * QR + s] = tobf(m);
        }
    }
    __syncthreads();
    // y [Q x P]: one 32 x 32 tile per wave (t block, p block)
    const int tb = wv / 2, pb = wv % 2;
    f32x16 acc = {};
#pragma unroll
    for (int ks = 0; ks < kQ / 16; ++ks) {   // + M x
        const int k0 = ks * 16 + 8 * (lane / 32);
        acc = mfma(lds8(&Ms[(tb * 32 + lane % 32) * QR + k0]), lds8(&Xt[(pb * 32 + lane % 32) * QR + k0]), acc);
    }
    const bf16_bits* Hc = a.Hin + (bh * a.nc + c) * int64_t(kP) * N + int64_t(pb * 32 + lane % 32) * N;
#pragma unroll
    for (int ks = 0; ks < N / 16; ++ks) {    // + (2^cum o C) H_in
        const int k0 = ks * 16 + 8 * (lane / 32);
        acc = mfma(lds8(&Cw[(tb * 32 + lane % 32) * NR + k0]), *reinterpret_cast<const bf16x8*>(Hc + k0), acc);
    }
    const float Dh = a.D ? a.D[h] : 0.0f;
    const int p = pb * 32 + lane % 32;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int tl = tb * 32 + 8 * (r / 4) + 4 * (lane / 32) + r % 4;
        const int64_t t = int64_t(c) * kQ + tl;
        if (t < a.L) {
            const int64_t o = ((b * a.L + t) * a.H + h) * kP + p;
            a.y[o] = tobf(fmaf(Dh, to_f32(Xt[p * QR + tl]), acc[r]));
        }
    }
}

template <int N>
hipError_t ssd_n(const SsdArgs& k, hipStream_t st) {
    const int64_t pairs = k.batch * k.H;
    const dim3 block(256);
    hipLaunchKernelGGL((ssd_chunk_state<N>), dim3(unsigned(pairs * k.nc)), block, 0, st, k);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((ssd_state_pass<N>), dim3(unsigned(pairs)), block, 0, st, k);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((ssd_chunk_scan<N>), dim3(unsigned(pairs * k.nc)), block, 0, st, k);
    return hipGetLastError();
}

size_t al256s(size_t v) { return (v + 255) & ~size_t(255); }

}  // namespace

size_t ssd_workspace_bytes(int64_t batch, int64_t L, int64_t heads, int64_t dstate) {
    const size_t blocks = size_t(batch) * size_t(heads) * size_t((L + kQ - 1) / kQ);
    return al256s(blocks * kP * size_t(dstate) * 4) + al256s(blocks * 4) +
           al256s(blocks * kP * size_t(dstate) * 2);
}

hipError_t launch_ssd(const SsdTensors& t, int64_t batch, int64_t L, int64_t heads, int64_t dstate,
                      void* workspace, hipStream_t stream) {
    SsdArgs k{};
    k.x = static_cast<const bf16_bits*>(t.x);
    k.delta = static_cast<const bf16_bits*>(t.delta);
    k.A = t.A;
    k.B = static_cast<const bf16_bits*>(t.B);
    k.C = static_cast<const bf16_bits*>(t.C);
    k.D = t.D;
    k.dt_bias = t.dt_bias;
    k.y = static_cast<bf16_bits*>(t.y);
    k.last_state = t.last_state;
    k.batch = batch; k.L = L; k.H = heads;
    k.nc = int32_t((L + kQ - 1) / kQ);
    const size_t blocks = size_t(batch) * size_t(heads) * size_t(k.nc);
    unsigned char* w = static_cast<unsigned char*>(workspace);
    k.S = reinterpret_cast<float*>(w);
    w += al256s(blocks * kP * size_t(dstate) * 4);
    k.tot = reinterpret_cast<float*>(w);
    w += al256s(blocks * 4);
    k.Hin = reinterpret_cast<bf16_bits*>(w);
    return dstate == 64 ? ssd_n<64>(k, stream) : ssd_n<128>(k, stream);
}

}  // namespace selscan
