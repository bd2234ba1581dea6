// Backward pass of the selective scan (S6) for gfx950.
//
// The gradients of the forward pass (from a zero state) for an output
// gradient dy, by the chain rule through the recurrence of "State Space
// Models and Mamba" (multigrid.ai), section "Selective state: the change that
// made it work on text". Following "Mamba: Linear-Time Sequence Modeling with
// Selective State Spaces" (azimuth.plus), hardware-aware algorithm,
// recomputation, the per-token states are never stored: a checkpoint pass
// (the forward kernel's third mode) keeps the state before every 16th token
// (1/16 of the states) and computes dz; this file's reverse pass then walks
// the 16-token chunks from last to first, recomputing each chunk's states and
// decays into registers from its checkpoint and sweeping back through them.
//
// Per (b, d) row, going back in t with carry[n] = 0 after the last token:
//     ds = dy * silu(z)
//     dh[n] = ds C[n,t] + carry[n];   carry[n] = abar[n,t] dh[n]
//     q = carry[n] h_{t-1}[n]                  (= dh * abar * h_{t-1})
//     dA[n] += q delta;  ddelta_t += q A[n] + x dh[n] B[n,t]
//     dx_t  += dh[n] delta B[n,t];  dB[n,t] += dh[n] delta x;  dC[n,t] += ds h_t[n]
//     dx_t  += ds D;  draw_t = ddelta_t * sigmoid(delta_raw + dt_bias);  ddt_bias += draw_t
//
// Mapping, as in the forward kernel: a workgroup owns 64 rows of one batch
// entry, one lane per row, and its 4 waves own 4 states each. B and C
// (packed by the checkpoint pass, B times ln 2) are staged per chunk in LDS
// and read as broadcasts (scalar operands would need more SGPRs than the
// reverse sweep leaves). The
// per-token work (softplus, the gate, the sums over states into dx and
// ddelta) is spread over all 256 threads by token slices and shared through
// LDS. dB and dC sum over the 64 rows of a wave: each 4-token sub-block's 16
// values per lane are reduced across the wave with the gfx950 lane-swap
// instructions (v_permlane32_swap, v_permlane16_swap) and row rotations
// (DPP), then the row blocks' partial sums are added in a fixed order by a
// second kernel, as are the per-channel sums (dA, dD, ddt_bias) over the
// batch. Every sum has a fixed order: the results are deterministic.
#include "common.hpp"
#include "launch.hpp"

namespace selscan {
namespace {

constexpr int kBCH = 16;                // tokens per reverse chunk (= checkpoint spacing)
constexpr int kBG = 4;                  // waves per 64-row block
constexpr int kBNG = kN / kBG;          // states per wave
constexpr int kBSB = 4;                 // tokens per packed sub-block (= waves)
constexpr int kBNSB = kBCH / kBSB;      // sub-blocks per chunk
constexpr int kBTS = kBCH / kBG;        // tokens per thread in the per-token phases
constexpr int kRecF = 32;               // floats per packed (b, sub-block, wave) record

struct BwdKArgs {
    const void* x;
    const void* delta;
    const void* z;
    const void* dy;
    const float* A;
    const float* P;      // packed B (times ln 2) / C records, as in the forward
    const float* D;
    const float* dt_bias;
    const float* ckpt;   // [nck][batch*dim][N]
    void* dx;
    void* ddelta;
    void* dz;            // [batch, dim, L] (gated only)
    float* pB;           // [row_blocks][batch][Lp][N]: sum over the block's rows of dh * l x
    float* pC;           // [row_blocks][batch][Lp][N]: sum over the block's rows of ds * h
    float* pA;           // [segments][batch*dim][N]: sum over the segment's t of q * l
    float* pD;           // [segments][batch*dim]
    float* pT;           // [segments][batch*dim]
    // Segments along t (a multiple of 32 tokens each). In the reverse pass,
    // carry_in[S-1-k] is the carry entering segment k from the right (null:
    // zero). The carry pass writes, for segment k, the carry a
    // sweep over it from zero leaves at its start to rc_state[S-1-k] and its
    // summed log2 step sizes to rc_lsum[S-1-k], both [S][batch*dim](*N).
    const float* carry_in;
    float* rc_state;
    double* rc_lsum;
    float* dh0;  // [batch*dim][N]: the carry leaving token 0 (null: not wanted)
    int64_t batch, L, dim, Lp, psub, seg_len;
    int32_t row_blocks, nck, segments, seg0;
};

// LDS: per-token l, w and ds of the chunk for the scan waves, and the waves'
// per-token partial sums over their states (sum q A, sum dh B', and, gated,
// sum C h). Every array holds 4 tokens per 16-byte piece, 64 bytes per row,
// and every access is a 16-byte one, at a piece index swizzled so that no
// access conflicts. On gfx950 a 16-byte read is served 16 lanes at a time
// from 64 banks (so 16 lanes must hit 16 distinct pieces mod 16) and a
// 16-byte write 8 lanes at a time from 32 banks (8 distinct pieces mod 8):
// * quad_in: written by the per-token threads (4 per row; 8 lanes = 2 rows x
//   4 pieces), read by them (16 lanes = 4 rows x 4 pieces) and by the scan
//   lanes (one row each, 16 rows, one piece);
// * quad_out: written by the scan lanes (8 rows, one piece), read by the
//   per-token threads.
struct alignas(16) BwdSmem {
    float ql[kWave * kBCH];        // l = log2-unit step size
    float qw[kWave * kBCH];        // w = l x
    float qd[kWave * kBCH];        // ds = dy silu(z)
    float pa[kBG][kWave * kBCH];   // per wave: sum over its states of q A
    float pb[kBG][kWave * kBCH];   // sum of dh B'
    float py[kBG][kWave * kBCH];   // sum of C h (gated)
    float bc[kBNSB * kBG * kRecF];  // the chunk's packed B/C records, as laid out in P
};
__device__ __forceinline__ int quad_in(int row, int k) { return row * 4 + (k ^ ((row >> 2) & 3)); }
__device__ __forceinline__ int quad_out(int row, int k) { return row * 4 + (k ^ ((row >> 1) & 3)); }
__device__ __forceinline__ float4& piece(float* base, int i) { return reinterpret_cast<float4*>(base)[i]; }

// 4 consecutive tokens of type T as one load: 16 bytes (fp32) or 8 (bf16),
// at any element-aligned address (rows need not start on a vector boundary:
// gfx950's global loads and stores take unaligned addresses whole).
template <typename T> struct Quad;
template <> struct Quad<float> {
    using V = uint4;
    static __device__ __forceinline__ V load(const float* p) { V v; __builtin_memcpy(&v, p, sizeof(V)); return v; }
    static __device__ __forceinline__ void unpack(const V& v, float* o) {
        o[0] = __uint_as_float(v.x); o[1] = __uint_as_float(v.y);
        o[2] = __uint_as_float(v.z); o[3] = __uint_as_float(v.w);
    }
    static __device__ __forceinline__ V pack(const float* f) {
        return make_uint4(__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]),
                          __float_as_uint(f[3]));
    }
    static __device__ __forceinline__ void store(float* p, const V& v) { __builtin_memcpy(p, &v, sizeof(V)); }
};
template <> struct Quad<bf16_bits> {
    using V = uint2;
    static __device__ __forceinline__ V load(const bf16_bits* p) { V v; __builtin_memcpy(&v, p, sizeof(V)); return v; }
    static __device__ __forceinline__ void unpack(const V& v, float* o) {
        o[0] = bf16_lo(v.x); o[1] = bf16_hi(v.x); o[2] = bf16_lo(v.y); o[3] = bf16_hi(v.y);
    }
    static __device__ __forceinline__ V pack(const float* f) {
        auto p = [](float a, float b) {
            return pack_bf16x2(a, b);
        };
        return make_uint2(p(f[0], f[1]), p(f[2], f[3]));
    }
    static __device__ __forceinline__ void store(bf16_bits* p, const V& v) { __builtin_memcpy(p, &v, sizeof(V)); }
};

// Sum of a over lanes {l, l^32} in lanes 0..31 and of b in lanes 32..63.
__device__ __forceinline__ float fold32(float a, float b) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// Sum of a over lanes {l, l^16} in even 16-lane rows and of b in odd rows.
__device__ __forceinline__ float fold16(float a, float b) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// Sum over the 16 lanes of a row, in every lane of it (rotations by 8, 4, 2, 1).
__device__ __forceinline__ float rowsum16(float v) {
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x128, 0xf, 0xf, false));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x124, 0xf, 0xf, false));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x122, 0xf, 0xf, false));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x121, 0xf, 0xf, false));
    return v;
}
// v[4e + j] (token e, state j) summed over the 64 lanes of the wave. Lane l
// returns, in o[0..3], the sums of token e = l / 16 for states 0..3.
__device__ __forceinline__ void wave_sum16(const float* v, float* o) {
    float u[8], w[4];
#pragma unroll
    for (int i = 0; i < 8; ++i) u[i] = fold32(v[i], v[i + 8]);   // index i + 8*(l/32)
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = fold16(u[i], u[i + 4]);   // index i + 4*((l/16)%2) + 8*(l/32)
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = rowsum16(w[i]);
}

// CARRY: the carry pass of a segmented backward (only the adjoint carry,
// swept back over the segment from zero, and the summed step sizes).
template <typename T, bool GATE, bool CARRY>
__global__ __launch_bounds__(256, 2) void bwd_kernel(BwdKArgs a) {
    using Q = Quad<T>;
    __shared__ BwdSmem sm;
    const T* __restrict__ X = static_cast<const T*>(a.x);
    const T* __restrict__ DL = static_cast<const T*>(a.delta);
    const T* __restrict__ Z = static_cast<const T*>(a.z);
    const T* __restrict__ DY = static_cast<const T*>(a.dy);

    const int tid = threadIdx.x;
    const int wv = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int lane = tid % kWave;
    // block -> (segment, batch entry, 64-row block)
    int64_t blk = xcd_tile(blockIdx.x, gridDim.x);
    const int rb = int(blk % a.row_blocks);
    blk /= a.row_blocks;
    const int64_t b = blk % a.batch;
    const int seg = a.seg0 + int(blk / a.batch);
    const int64_t rows = a.batch * a.dim;
    // this segment's 16-token chunks [c_lo, c_hi)
    const int c_lo = int(int64_t(seg) * a.seg_len / kBCH);
    const int c_hi = int(min(int64_t(a.nck), (int64_t(seg) + 1) * a.seg_len / kBCH));

    // scan mapping: lane = row, wave = 4 states
    const int64_t d0 = int64_t(rb) * kWave;
    const int64_t d = d0 + lane;
    const bool row_ok = d < a.dim;
    const int64_t row = b * a.dim + (row_ok ? d : d0);
    const int n0 = wv * kBNG;
    float An[kBNG];
#pragma unroll
    for (int j = 0; j < kBNG; ++j) An[j] = row_ok ? a.A[d * kN + n0 + j] : 0.0f;

    // per-token mapping: thread (pr, pq) = row pr, tokens [4 pq, 4 pq + 4) of a chunk
    const int pr = tid / kBG, pq = tid % kBG;
    const int64_t dp = d0 + pr;
    const bool prow_ok = dp < a.dim;
    const int64_t prow = b * a.dim + (prow_ok ? dp : d0);
    const float biasl = (a.dt_bias && prow_ok) ? a.dt_bias[dp] * kLog2e : 0.0f;
    const float Dd = (a.D && prow_ok) ? a.D[dp] : 0.0f;

    // A thread's four tokens are one vector load per tensor (at any
    // alignment); a group that runs past the row's end is loaded element by
    // element, zero past the end.
    struct In {
        typename Q::V x, d, z, g;
        float2 bc;  // 8 bytes of the chunk's packed B/C records
    };
    // The chunk's records are one contiguous 2 KiB block of P: 8 bytes a thread.
    const float* Pb = a.P + b * a.psub * kBG * kRecF;
    auto load = [&](int c, In& in) {
        in.bc = reinterpret_cast<const float2*>(Pb + int64_t(c) * (kBNSB * kBG * kRecF))[tid];
        const int64_t t0 = int64_t(c) * kBCH + pq * kBTS;
        const int64_t off = prow * a.L + t0;
        if (t0 + kBTS <= a.L) {
            in.x = Q::load(X + off);
            in.d = Q::load(DL + off);
            if constexpr (GATE) in.z = Q::load(Z + off);
            in.g = Q::load(DY + off);
        } else {
            float fx[4], fd[4], fz[4], fg[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const bool ok = t0 + e < a.L;
                fx[e] = ok ? to_f32(X[off + e]) : 0.0f;
                fd[e] = ok ? to_f32(DL[off + e]) : 0.0f;
                fz[e] = (GATE && ok) ? to_f32(Z[off + e]) : 0.0f;
                fg[e] = ok ? to_f32(DY[off + e]) : 0.0f;
            }
            in.x = Q::pack(fx);
            in.d = Q::pack(fd);
            in.z = Q::pack(fz);
            in.g = Q::pack(fg);
        }
    };
    // Values a per-token thread keeps from its prologue to its epilogue of the
    // same chunk: x, sigmoid(u), and (gated) dy silu'(z). Its l and ds are
    // read back from LDS, where they stay for the scan until the next prologue.
    struct Keep {
        float x[kBTS], sg[kBTS], dzf[GATE ? kBTS : 1];
    };
    double lsum_acc = 0.0;  // carry pass: this thread's tokens' summed step sizes
    // ---- per-token prologue of chunk c: (l, w) and ds to LDS ----
    auto prologue = [&](int c, const In& in, Keep& k) {
        const int64_t t0 = int64_t(c) * kBCH + pq * kBTS;
        float xs[4], us[4], zs[4], gs[4];
        Q::unpack(in.x, xs);
        Q::unpack(in.d, us);
        Q::unpack(in.g, gs);
        if constexpr (GATE) Q::unpack(in.z, zs);
        float l[4], w[4], dsv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const bool ok = prow_ok && t0 + e < a.L;
            const float ul = fmaf(us[e], kLog2e, biasl);
            const float lv = softplus_log2_of(ul);
            l[e] = ok ? lv : 0.0f;
            w[e] = l[e] * xs[e];
            float g = 1.0f;
            if constexpr (GATE) {
                // silu(z) = z sig(z); silu'(z) = sig(z) (1 + z (1 - sig(z)))
                const float sz = rcp_hw(1.0f + exp2_hw(-zs[e] * kLog2e));
                g = zs[e] * sz;
                k.dzf[e] = ok ? gs[e] * (sz * fmaf(zs[e], 1.0f - sz, 1.0f)) : 0.0f;
            }
            dsv[e] = ok ? gs[e] * g : 0.0f;
            k.x[e] = xs[e];
            k.sg[e] = exp2_hw(ul - lv);  // sigmoid(u) = e^u / (1 + e^u)
            if constexpr (CARRY) lsum_acc += double(l[e]);
        }
        const int qi = quad_in(pr, pq);
        piece(sm.ql, qi) = make_float4(l[0], l[1], l[2], l[3]);
        piece(sm.qw, qi) = make_float4(w[0], w[1], w[2], w[3]);
        piece(sm.qd, qi) = make_float4(dsv[0], dsv[1], dsv[2], dsv[3]);
        reinterpret_cast<float2*>(sm.bc)[tid] = in.bc;
    };

    float carry[kBNG], dAacc[kBNG];
#pragma unroll
    for (int j = 0; j < kBNG; ++j) {
        carry[j] = (a.carry_in && row_ok)
                       ? a.carry_in[((int64_t(a.segments) - 1 - seg) * rows + row) * kN + n0 + j]
                       : 0.0f;
        dAacc[j] = 0.0f;
    }

    // ---- the scan waves on chunk c: recompute, then sweep back ----
    // The states of the chunk are recomputed from its checkpoint into
    // registers (h_t for the 16 tokens); the decays are recomputed again on
    // the way back rather than kept. B and C come from LDS (broadcast reads).
    auto scan_chunk = [&](int c) {
        if constexpr (CARRY) {
            // only the adjoint carry: dh = ds C + carry, carry = exp(delta A) dh
#pragma unroll
            for (int sb = kBNSB - 1; sb >= 0; --sb) {
                const float4 L4 = piece(sm.ql, quad_in(lane, sb)), D4 = piece(sm.qd, quad_in(lane, sb));
                const float Lv[4] = {L4.x, L4.y, L4.z, L4.w}, Dv[4] = {D4.x, D4.y, D4.z, D4.w};
                float Cv[16];
                const float4* r = reinterpret_cast<const float4*>(sm.bc + (sb * kBG + wv) * kRecF);
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const float4 w = r[4 + q];
                    Cv[4 * q] = w.x; Cv[4 * q + 1] = w.y; Cv[4 * q + 2] = w.z; Cv[4 * q + 3] = w.w;
                }
#pragma unroll
                for (int e = kBSB - 1; e >= 0; --e) {
                    const float lx = Lv[e], ds = Dv[e];
#pragma unroll
                    for (int j = 0; j < kBNG; ++j) {
                        const float dh = fmaf(ds, Cv[j * kBSB + e], carry[j]);
                        carry[j] = exp2_hw(lx * An[j]) * dh;
                    }
                }
            }
            return;
        }
        const float4 hs4 = *reinterpret_cast<const float4*>(a.ckpt + (int64_t(c) * rows + row) * kN + n0);
        const float hs[kBNG] = {hs4.x, hs4.y, hs4.z, hs4.w};
        auto rec = [&](int sb) { return reinterpret_cast<const float4*>(sm.bc + (sb * kBG + wv) * kRecF); };
        float H[kBCH][kBNG];
        float h[kBNG] = {hs[0], hs[1], hs[2], hs[3]};
#pragma unroll
        for (int sb = 0; sb < kBNSB; ++sb) {
            float Bv[16];
            const float4* r = rec(sb);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float4 v = r[q];
                Bv[4 * q] = v.x; Bv[4 * q + 1] = v.y; Bv[4 * q + 2] = v.z; Bv[4 * q + 3] = v.w;
            }
            const float4 L4 = piece(sm.ql, quad_in(lane, sb)), W4 = piece(sm.qw, quad_in(lane, sb));
            const float Lv[4] = {L4.x, L4.y, L4.z, L4.w}, Wv[4] = {W4.x, W4.y, W4.z, W4.w};
#pragma unroll
            for (int e = 0; e < kBSB; ++e) {
                const int t = sb * kBSB + e;
#pragma unroll
                for (int j = 0; j < kBNG; ++j) {
                    h[j] = fmaf(exp2_hw(Lv[e] * An[j]), h[j], Wv[e] * Bv[j * kBSB + e]);
                    H[t][j] = h[j];
                }
            }
        }
#pragma unroll
        for (int sb = kBNSB - 1; sb >= 0; --sb) {
            float Bv[16], Cv[16];
            const float4* r = rec(sb);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float4 v = r[q], w = r[4 + q];
                Bv[4 * q] = v.x; Bv[4 * q + 1] = v.y; Bv[4 * q + 2] = v.z; Bv[4 * q + 3] = v.w;
                Cv[4 * q] = w.x; Cv[4 * q + 1] = w.y; Cv[4 * q + 2] = w.z; Cv[4 * q + 3] = w.w;
            }
            const int qi = quad_in(lane, sb);
            const float4 L4 = piece(sm.ql, qi), W4 = piece(sm.qw, qi), D4 = piece(sm.qd, qi);
            const float Lv[4] = {L4.x, L4.y, L4.z, L4.w}, Wv[4] = {W4.x, W4.y, W4.z, W4.w};
            const float Dv[4] = {D4.x, D4.y, D4.z, D4.w};
            float vB[16], vC[16], yv[kBSB], av[kBSB], bv[kBSB];
#pragma unroll
            for (int e = kBSB - 1; e >= 0; --e) {
                const int t = sb * kBSB + e;
                const float2 lw = make_float2(Lv[e], Wv[e]);
                const float ds = Dv[e];
                float accA = 0.0f, accB = 0.0f, accY = 0.0f;
#pragma unroll
                for (int j = 0; j < kBNG; ++j) {
                    const float dh = fmaf(ds, Cv[j * kBSB + e], carry[j]);
                    carry[j] = exp2_hw(lw.x * An[j]) * dh;
                    const float q = carry[j] * (t > 0 ? H[t - 1][j] : hs[j]);
                    accA = fmaf(q, An[j], accA);
                    dAacc[j] = fmaf(q, lw.x, dAacc[j]);
                    accB = fmaf(dh, Bv[j * kBSB + e], accB);
                    vB[e * 4 + j] = dh * lw.y;
                    vC[e * 4 + j] = ds * H[t][j];
                    if constexpr (GATE) accY = fmaf(Cv[j * kBSB + e], H[t][j], accY);
                }
                av[e] = accA;
                bv[e] = accB;
                yv[e] = accY;
            }
            const int qo = quad_out(lane, sb);
            piece(sm.pa[wv], qo) = make_float4(av[0], av[1], av[2], av[3]);
            piece(sm.pb[wv], qo) = make_float4(bv[0], bv[1], bv[2], bv[3]);
            if constexpr (GATE) piece(sm.py[wv], qo) = make_float4(yv[0], yv[1], yv[2], yv[3]);
            float sB[4], sC[4];
            wave_sum16(vB, sB);
            wave_sum16(vC, sC);
            if ((lane & 15) == 0) {
                const int64_t t = int64_t(c) * kBCH + sb * kBSB + (lane >> 4);
                const int64_t o = ((int64_t(rb) * a.batch + b) * a.Lp + t) * kN + n0;
                *reinterpret_cast<float4*>(a.pB + o) = make_float4(sB[0], sB[1], sB[2], sB[3]);
                *reinterpret_cast<float4*>(a.pC + o) = make_float4(sC[0], sC[1], sC[2], sC[3]);
            }
        }
    };

    float dDacc = 0.0f, dTacc = 0.0f;
    // ---- per-token epilogue of chunk c: sums over the waves, dx, ddelta ----
    auto epilogue = [&](int c, const Keep& k) {
        if constexpr (CARRY) return;
        const int64_t t0 = int64_t(c) * kBCH + pq * kBTS;
        const float4 L4 = piece(sm.ql, quad_in(pr, pq)), D4 = piece(sm.qd, quad_in(pr, pq));
        const float kl[4] = {L4.x, L4.y, L4.z, L4.w}, kds[4] = {D4.x, D4.y, D4.z, D4.w};
        const int qo = quad_out(pr, pq);
        float dxv[4], ddv[4], dzv[4];
        if constexpr (GATE) {
            // dz = dy silu'(z) (C.h + D x), the waves' partial sums added in order
            float4 y4 = piece(sm.py[0], qo);
#pragma unroll
            for (int g = 1; g < kBG; ++g) {
                const float4 v = piece(sm.py[g], qo);
                y4.x += v.x; y4.y += v.y; y4.z += v.z; y4.w += v.w;
            }
            const float yv[4] = {y4.x, y4.y, y4.z, y4.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) dzv[e] = fmaf(Dd, k.x[e], yv[e]) * k.dzf[e];
        }
        // the waves' (sum q A, sum dh B') of the thread's 4 tokens, added in wave order
        float AAs[4] = {0.0f, 0.0f, 0.0f, 0.0f}, BBs[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int g = 0; g < kBG; ++g) {
            const float4 va = piece(sm.pa[g], qo), vb = piece(sm.pb[g], qo);
            AAs[0] += va.x; AAs[1] += va.y; AAs[2] += va.z; AAs[3] += va.w;
            BBs[0] += vb.x; BBs[1] += vb.y; BBs[2] += vb.z; BBs[3] += vb.w;
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float AA = AAs[e], BB = BBs[e];
            // B was packed times ln 2: BB = ln2 * sum dh B, and delta = l ln 2.
            const float ddl = fmaf(k.x[e] * BB, kLog2e, AA);
            dxv[e] = fmaf(kl[e], BB, kds[e] * Dd);
            ddv[e] = ddl * k.sg[e];
            if (t0 + e < a.L) {
                dDacc = fmaf(kds[e], k.x[e], dDacc);
                dTacc += ddv[e];
            }
        }
        if (!prow_ok) return;
        const int64_t off = prow * a.L + t0;
        T* DXo = static_cast<T*>(a.dx);
        T* DDo = static_cast<T*>(a.ddelta);
        T* DZo = static_cast<T*>(a.dz);
        if (t0 + kBTS <= a.L) {
            Q::store(DXo + off, Q::pack(dxv));
            Q::store(DDo + off, Q::pack(ddv));
            if constexpr (GATE) Q::store(DZo + off, Q::pack(dzv));
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (t0 + e < a.L) {
                    DXo[off + e] = from_f32<T>(dxv[e]);
                    DDo[off + e] = from_f32<T>(ddv[e]);
                    if constexpr (GATE) DZo[off + e] = from_f32<T>(dzv[e]);
                }
        }
    };

    // The segment's chunks from last to first. Inputs are loaded two chunks
    // ahead; the per-token values of chunk c live in the Keep set of its
    // parity.
    In in0, in1;
    Keep k0, k1;
    // As in the forward kernel, the sweep runs at a raised wave priority and
    // the per-token phases at the base one (about 3.5% less time).
    auto step = [&](int c, Keep& kc, Keep& kn, In& inn) {
        // kc: chunk c (prologue done); inn holds chunk c-1's inputs
        __builtin_amdgcn_s_setprio(1);
        scan_chunk(c);
        __syncthreads();
        __builtin_amdgcn_s_setprio(0);
        epilogue(c, kc);
        if (c - 1 >= c_lo) prologue(c - 1, inn, kn);
        if (c - 3 >= c_lo) load(c - 3, inn);
        __syncthreads();
    };
    const int last = c_hi - 1;
    // in[p] holds the chunk of parity p's inputs
    if (last & 1) {
        load(last, in1);
        if (last - 1 >= c_lo) load(last - 1, in0);
        prologue(last, in1, k1);
        if (last - 2 >= c_lo) load(last - 2, in1);
    } else {
        load(last, in0);
        if (last - 1 >= c_lo) load(last - 1, in1);
        prologue(last, in0, k0);
        if (last - 2 >= c_lo) load(last - 2, in0);
    }
    __syncthreads();
    int c = last;
    if (c & 1) {
        step(c, k1, k0, in0);
        --c;
    }
    for (; c >= c_lo; c -= 2) {
        step(c, k0, k1, in1);
        if (c - 1 >= c_lo) step(c - 1, k1, k0, in0);
    }

    if constexpr (CARRY) {
        // this segment's carry from zero, and its summed step sizes (the four
        // token slices of a row added in order)
        const int64_t ri = int64_t(a.segments) - 1 - seg;
        if (row_ok)
            *reinterpret_cast<float4*>(a.rc_state + (ri * rows + row) * kN + n0) =
                make_float4(carry[0], carry[1], carry[2], carry[3]);
        double* red = reinterpret_cast<double*>(&sm.pa[0][0]);
        red[pq * kWave + pr] = lsum_acc;
        __syncthreads();
        if (wv == 0 && row_ok) {
            double sL = 0.0;
#pragma unroll
            for (int g = 0; g < kBG; ++g) sL += red[g * kWave + lane];
            a.rc_lsum[ri * rows + row] = sL;
        }
        return;
    }
    // the adjoint carry leaving the first token is the gradient of the initial state
    if (a.dh0 && seg == 0 && row_ok)
        *reinterpret_cast<float4*>(a.dh0 + row * kN + n0) =
            make_float4(carry[0], carry[1], carry[2], carry[3]);
    // ---- per-row sums over the segment: dA (this wave's states), dD and ddt_bias ----
    const int64_t so = int64_t(seg) * rows + row;
    if (row_ok) {
        *reinterpret_cast<float4*>(a.pA + so * kN + n0) =
            make_float4(dAacc[0], dAacc[1], dAacc[2], dAacc[3]);
    }
    float2* red = reinterpret_cast<float2*>(&sm.pa[0][0]);
    red[pq * kWave + pr] = make_float2(dDacc, dTacc);
    __syncthreads();
    if (wv == 0 && row_ok) {
        float sD = 0.0f, sT = 0.0f;
#pragma unroll
        for (int g = 0; g < kBG; ++g) {
            const float2 v = red[g * kWave + lane];
            sD += v.x;
            sT += v.y;
        }
        a.pD[so] = sD;
        a.pT[so] = sT;
    }
}

// dB[b,n,t] = ln 2 * sum_rb pB[rb,b,t,n] and dC[b,n,t] = sum_rb pC[rb,b,t,n].
template <typename T>
__global__ __launch_bounds__(256) void bwd_reduce_bc(const float* __restrict__ pB,
                                                     const float* __restrict__ pC, T* __restrict__ dB,
                                                     T* __restrict__ dC, int64_t batch, int64_t L,
                                                     int64_t Lp, int32_t row_blocks) {
    // A lane takes one (b, t, 4 states), the state quad fastest, so a wave
    // reads 16 whole 64-byte partial records (1 KiB contiguous) from each row
    // block; the block's 4 waves take a quarter of the row blocks each, summed
    // in order, and wave 0 adds the quarters in order (deterministic).
    __shared__ float4 part[2][3][kWave];
    const int lane = threadIdx.x % kWave, w = threadIdx.x / kWave;
    const int64_t i = int64_t(blockIdx.x) * kWave + lane;
    const bool ok = i < batch * L * 4;
    const int q = int(i % 4);
    const int64_t bt = ok ? i / 4 : 0;
    const int64_t t = bt % L, b = bt / L;
    const int r_lo = int(int64_t(row_blocks) * w / 4), r_hi = int(int64_t(row_blocks) * (w + 1) / 4);
    float4 sb = make_float4(0.0f, 0.0f, 0.0f, 0.0f), sc = sb;
    const int64_t step = batch * Lp * kN;  // floats from one row block to the next
    const float* ob = pB + (b * Lp + t) * kN + 4 * q;
    const float* oc = pC + (b * Lp + t) * kN + 4 * q;
    int r = r_lo;
    if (ok) {
        for (; r + 8 <= r_hi; r += 8) {
            float4 vb[8], vc[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                vb[u] = *reinterpret_cast<const float4*>(ob + (r + u) * step);
                vc[u] = *reinterpret_cast<const float4*>(oc + (r + u) * step);
            }
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                sb.x += vb[u].x; sb.y += vb[u].y; sb.z += vb[u].z; sb.w += vb[u].w;
                sc.x += vc[u].x; sc.y += vc[u].y; sc.z += vc[u].z; sc.w += vc[u].w;
            }
        }
        for (; r < r_hi; ++r) {
            const float4 vb = *reinterpret_cast<const float4*>(ob + r * step);
            const float4 vc = *reinterpret_cast<const float4*>(oc + r * step);
            sb.x += vb.x; sb.y += vb.y; sb.z += vb.z; sb.w += vb.w;
            sc.x += vc.x; sc.y += vc.y; sc.z += vc.z; sc.w += vc.w;
        }
    }
    if (w > 0) {
        part[0][w - 1][lane] = sb;
        part[1][w - 1][lane] = sc;
    }
    __syncthreads();
    if (w > 0 || !ok) return;
#pragma unroll
    for (int g = 0; g < 3; ++g) {
        const float4 vb = part[0][g][lane], vc = part[1][g][lane];
        sb.x += vb.x; sb.y += vb.y; sb.z += vb.z; sb.w += vb.w;
        sc.x += vc.x; sc.y += vc.y; sc.z += vc.z; sc.w += vc.w;
    }
    const float vb4[4] = {sb.x, sb.y, sb.z, sb.w}, vc4[4] = {sc.x, sc.y, sc.z, sc.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        dB[(b * kN + 4 * q + j) * L + t] = from_f32<T>(vb4[j] * kLn2);
        dC[(b * kN + 4 * q + j) * L + t] = from_f32<T>(vc4[j]);
    }
}

// dA[d,n] = ln 2 * sum_e pA[e,d,n]; dD[d] = sum_e pD[e,d]; ddt_bias[d] = sum_e pT[e,d],
// e over the entries (segment x batch entry). A block takes 64 outputs
// (4 channels x 16 states); each of its waves a quarter of the entries,
// summed in order; wave 0 adds the quarters in order (deterministic).
__global__ __launch_bounds__(256) void bwd_reduce_params(const float* __restrict__ pA,
                                                         const float* __restrict__ pD,
                                                         const float* __restrict__ pT,
                                                         float* __restrict__ dA, float* dD,
                                                         float* ddt, int64_t entries, int64_t dim) {
    __shared__ float part[3][3][kWave];
    const int lane = threadIdx.x % kWave, w = threadIdx.x / kWave;
    const int64_t i = int64_t(blockIdx.x) * kWave + lane;  // d * N + n
    const bool ok = i < dim * kN;
    const int64_t d = i / kN;
    const bool first = ok && i % kN == 0;  // this lane also sums dD and ddt_bias of channel d
    const int64_t e_lo = entries * w / 4, e_hi = entries * (w + 1) / 4;
    const int64_t sA = dim * kN;  // floats from one entry to the next
    float s = 0.0f, sD = 0.0f, sT = 0.0f;
    if (ok) {
        int64_t e = e_lo;
        for (; e + 8 <= e_hi; e += 8) {
            float v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) v[u] = pA[(e + u) * sA + i];
#pragma unroll
            for (int u = 0; u < 8; ++u) s += v[u];
        }
        for (; e < e_hi; ++e) s += pA[e * sA + i];
        if (first)
            for (e = e_lo; e < e_hi; ++e) {
                sD += pD[e * dim + d];
                sT += pT[e * dim + d];
            }
    }
    if (w > 0) {
        part[0][w - 1][lane] = s;
        part[1][w - 1][lane] = sD;
        part[2][w - 1][lane] = sT;
    }
    __syncthreads();
    if (w > 0 || !ok) return;
#pragma unroll
    for (int g = 0; g < 3; ++g) {
        s += part[0][g][lane];
        sD += part[1][g][lane];
        sT += part[2][g][lane];
    }
    dA[i] = s * kLn2;
    if (first) {
        if (dD) dD[d] = sD;
        if (ddt) ddt[d] = sT;
    }
}

size_t al256(size_t v) { return (v + 255) & ~size_t(255); }

struct BwdLayout {
    size_t packed, ckpt, pB, pC, pA, pD, pT, seg_state, carry, seg_lsum, total;
};
BwdLayout bwd_layout(int64_t batch, int64_t L, int64_t dim, int32_t segments, bool ckpt_given) {
    const size_t rows = size_t(batch) * size_t(dim);
    const size_t S = size_t(segments);
    const size_t nck = size_t((L + kBCH - 1) / kBCH);
    const size_t Lp = nck * kBCH;
    const size_t Lp32 = size_t((L + kChunk - 1) / kChunk) * kChunk;
    const size_t rbk = size_t((dim + kWave - 1) / kWave);
    BwdLayout o{};
    size_t off = 0;
    o.packed = off; off += al256(size_t(batch) * Lp32 * 2 * kN * 4);
    o.ckpt = off;   off += ckpt_given ? 0 : al256(nck * rows * kN * 4);
    o.pB = off;     off += al256(rbk * size_t(batch) * Lp * kN * 4);
    o.pC = off;     off += al256(rbk * size_t(batch) * Lp * kN * 4);
    o.pA = off;     off += al256(S * rows * kN * 4);
    o.pD = off;     off += al256(S * rows * 4);
    o.pT = off;     off += al256(S * rows * 4);
    // segmented runs: per-segment states and carries (forward, then reused
    // for the reverse carries) and summed step sizes
    const size_t segb = S > 1 ? S : 0;
    o.seg_state = off; off += al256(segb * rows * kN * 4);
    o.carry = off;     off += al256(segb * rows * kN * 4);
    o.seg_lsum = off;  off += al256(segb * rows * 8);
    o.total = off;
    return o;
}

template <typename T, bool CARRY>
hipError_t launch_bwd_kernel(const BwdKArgs& k, bool gate, int64_t blocks, hipStream_t st) {
    const dim3 grid{unsigned(blocks)}, block{256};
    if (gate) hipLaunchKernelGGL((bwd_kernel<T, true, CARRY>), grid, block, 0, st, k);
    else hipLaunchKernelGGL((bwd_kernel<T, false, CARRY>), grid, block, 0, st, k);
    return hipGetLastError();
}

// A segmented backward (S > 1) runs: the forward state pass and carries
// (states entering each segment), the checkpoint pass over all segments from
// those states, the reverse carry pass over segments 1..S-1 (the adjoint
// carry each leaves from zero) and its right-to-left composition (the same
// associative pair as the forward carries: the carry a sweep leaves is
// prod(decays) * carry in + carry from zero), and the reverse pass over all
// segments from the carries entering them from the right. Every per-token
// gradient belongs to one segment; dA, dD and ddt_bias are per-segment
// partial sums added in a fixed order.
template <typename T>
hipError_t bwd_t(const BwdTensors& t, int64_t batch, int64_t L, int64_t dim, int32_t segments,
                 int64_t seg_len, void* ws, hipStream_t st) {
    unsigned char* w = static_cast<unsigned char*>(ws);
    const bool given = t.ckpt != nullptr;
    const BwdLayout lo = bwd_layout(batch, L, dim, segments, given);
    FwdTensors ft{t.x, t.delta, t.z, t.A, t.B, t.C, t.D, t.dt_bias, nullptr, nullptr, t.h0, nullptr};
    FwdShape fs{batch, L, dim, sizeof(T) == 2 ? DType::BF16 : DType::F32};
    float* packed = reinterpret_cast<float*>(w + lo.packed);
    float* ckpt = given ? nullptr : reinterpret_cast<float*>(w + lo.ckpt);
    float* seg_state = segments > 1 ? reinterpret_cast<float*>(w + lo.seg_state) : nullptr;
    float* carry = segments > 1 ? reinterpret_cast<float*>(w + lo.carry) : nullptr;
    double* seg_lsum = segments > 1 ? reinterpret_cast<double*>(w + lo.seg_lsum) : nullptr;
    hipError_t e = launch_fwd_ckpt(ft, ckpt, fs, packed, segments, seg_len, seg_state, seg_lsum,
                                   carry, !given, st);
    if (e != hipSuccess) return e;

    BwdKArgs k{};
    k.x = t.x; k.delta = t.delta; k.z = t.z; k.dy = t.dy; k.A = t.A; k.P = packed;
    k.D = t.D; k.dt_bias = t.dt_bias; k.ckpt = given ? t.ckpt : ckpt; k.dx = t.dx; k.ddelta = t.ddelta; k.dz = t.dz;
    k.pB = reinterpret_cast<float*>(w + lo.pB);
    k.pC = reinterpret_cast<float*>(w + lo.pC);
    k.pA = reinterpret_cast<float*>(w + lo.pA);
    k.pD = reinterpret_cast<float*>(w + lo.pD);
    k.pT = reinterpret_cast<float*>(w + lo.pT);
    k.batch = batch; k.L = L; k.dim = dim;
    k.nck = int32_t((L + kBCH - 1) / kBCH);
    k.Lp = int64_t(k.nck) * kBCH;
    k.psub = ((L + kChunk - 1) / kChunk * kChunk) / kBG;
    k.row_blocks = int32_t((dim + kWave - 1) / kWave);
    k.segments = segments;
    k.seg_len = segments > 1 ? seg_len : int64_t(k.nck) * kBCH;
    const int64_t per_seg = int64_t(k.row_blocks) * batch;
    const bool gate = t.z != nullptr;
    const int64_t rows = batch * dim;
    if (segments > 1) {
        // reverse carries: the forward state buffers are free again
        BwdKArgs kc = k;
        kc.seg0 = 1;
        kc.rc_state = seg_state;
        kc.rc_lsum = seg_lsum;
        e = launch_bwd_kernel<T, true>(kc, gate, per_seg * (segments - 1), st);
        if (e != hipSuccess) return e;
        e = launch_carry(t.A, seg_state, seg_lsum, t.dlast, carry, rows, dim, segments, st);
        if (e != hipSuccess) return e;
        k.carry_in = carry;
    } else {
        k.carry_in = t.dlast;
    }
    k.dh0 = t.dh0;
    e = launch_bwd_kernel<T, false>(k, gate, per_seg * segments, st);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((bwd_reduce_bc<T>), dim3(unsigned((batch * 4 * L + kWave - 1) / kWave)), dim3(256), 0, st,
                       k.pB, k.pC, static_cast<T*>(t.dB), static_cast<T*>(t.dC), batch, L, k.Lp,
                       k.row_blocks);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(bwd_reduce_params, dim3(unsigned((dim * kN + kWave - 1) / kWave)), dim3(256), 0, st,
                       k.pA, k.pD, k.pT, t.dA, t.dD, t.ddt_bias, batch * segments, dim);
    return hipGetLastError();
}

}  // namespace

size_t bwd_workspace_bytes(int64_t batch, int64_t L, int64_t dim, int32_t segments,
                           bool ckpt_given) {
    return bwd_layout(batch, L, dim, segments, ckpt_given).total;
}

hipError_t launch_bwd(const BwdTensors& t, int64_t batch, int64_t L, int64_t dim, DType dtype,
                      int32_t segments, int64_t seg_len, void* workspace, hipStream_t stream) {
    return dtype == DType::BF16 ? bwd_t<bf16_bits>(t, batch, L, dim, segments, seg_len, workspace, stream)
                                : bwd_t<float>(t, batch, L, dim, segments, seg_len, workspace, stream);
}

}  // namespace selscan
