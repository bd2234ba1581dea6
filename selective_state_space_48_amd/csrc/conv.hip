// Causal depthwise convolution of width 4 followed by SiLU, and its one-token
// decode step, for gfx950.
//
// "State Space Models and Mamba" (multigrid.ai), section "What a Mamba block
// actually contains": in front of the selective SSM sits a depthwise conv1d of
// kernel width 4 and a SiLU, which gives the block direct access to the last
// few tokens; "Mamba: Linear-Time Sequence Modeling with Selective State
// Spaces" (azimuth.plus), the block architecture (projection, short 1D
// convolution of size 4, SiLU, selective SSM). Causal, so that the same block
// can run one token at a time. Per (b, d) row and token t:
//     out[t] = silu(bias_d + sum_{k<4} w[d,k] * xx(t - 3 + k))
// where xx(s) is x[s] for s >= 0 and the carried-in input x_prev[3 + s] before
// the start of the call.
//
// The whole operation moves 2 x (element size) bytes per element and does 4
// FMAs and a sigmoid: it is bound by HBM. Each thread takes one 16-byte
// vector of consecutive tokens of one row; consecutive lanes take consecutive
// vectors of the same row, so a wave reads and writes 1 KiB contiguous runs
// with non-temporal 16-byte accesses. A thread also loads the 4 inputs before
// its vector (a hit in cache: the lane below's vector), so that no lane
// waits for another.
#include "common.hpp"
#include "launch.hpp"

namespace selscan {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

template <typename T> struct CElem;
template <> struct CElem<float> { static constexpr int kPer16 = 4; };
template <> struct CElem<bf16_bits> { static constexpr int kPer16 = 8; };

template <typename T>
__device__ __forceinline__ void unpack_vec(const u32x4& v, float* o) {
    if constexpr (sizeof(T) == 4) {
        o[0] = __uint_as_float(v.x); o[1] = __uint_as_float(v.y);
        o[2] = __uint_as_float(v.z); o[3] = __uint_as_float(v.w);
    } else {
        o[0] = bf16_lo(v.x); o[1] = bf16_hi(v.x); o[2] = bf16_lo(v.y); o[3] = bf16_hi(v.y);
        o[4] = bf16_lo(v.z); o[5] = bf16_hi(v.z); o[6] = bf16_lo(v.w); o[7] = bf16_hi(v.w);
    }
}

template <typename T>
__device__ __forceinline__ u32x4 pack_vec(const float* f) {
    u32x4 v;
    if constexpr (sizeof(T) == 4) {
        v.x = __float_as_uint(f[0]); v.y = __float_as_uint(f[1]);
        v.z = __float_as_uint(f[2]); v.w = __float_as_uint(f[3]);
    } else {
        auto p = [](float a, float b) {
            return pack_bf16x2(a, b);
        };
        v.x = p(f[0], f[1]); v.y = p(f[2], f[3]); v.z = p(f[4], f[5]); v.w = p(f[6], f[7]);
    }
    return v;
}

__device__ __forceinline__ float conv4(const float4& w, float b, float x0, float x1, float x2,
                                       float x3) {
    return fmaf(w.w, x3, fmaf(w.z, x2, fmaf(w.y, x1, fmaf(w.x, x0, b))));
}

// 4 consecutive tokens (8 bytes of bf16, 16 of fp32).
template <typename T> struct Halo;  // 4 tokens
template <> struct Halo<float> { typedef u32x4 type; };
template <> struct Halo<bf16_bits> { typedef unsigned int type __attribute__((ext_vector_type(2))); };

template <typename T>
__device__ __forceinline__ void unpack_halo(const typename Halo<T>::type& v, float* o) {
    if constexpr (sizeof(T) == 4) {
        o[0] = __uint_as_float(v.x); o[1] = __uint_as_float(v.y);
        o[2] = __uint_as_float(v.z); o[3] = __uint_as_float(v.w);
    } else {
        o[0] = bf16_lo(v.x); o[1] = bf16_hi(v.x); o[2] = bf16_lo(v.y); o[3] = bf16_hi(v.y);
    }
}

// Bytes [sh, sh + 16) of the 32 bytes lo ++ hi (sh = 0..15).
__device__ __forceinline__ u32x4 bytes16_at(const u32x4& lo, const u32x4& hi, int sh) {
    const bool s4 = sh & 4, s8 = sh & 8;
    const uint32_t e0 = s4 ? lo.y : lo.x, e1 = s4 ? lo.z : lo.y, e2 = s4 ? lo.w : lo.z,
                   e3 = s4 ? hi.x : lo.w, e4 = s4 ? hi.y : hi.x, e5 = s4 ? hi.z : hi.y,
                   e6 = s4 ? hi.w : hi.z;
    const uint32_t f0 = s8 ? e2 : e0, f1 = s8 ? e3 : e1, f2 = s8 ? e4 : e2, f3 = s8 ? e5 : e3,
                   f4 = s8 ? e6 : e4;
    const uint32_t b = uint32_t(sh & 3);
    u32x4 r;
    r.x = __builtin_amdgcn_alignbyte(f1, f0, b);
    r.y = __builtin_amdgcn_alignbyte(f2, f1, b);
    r.z = __builtin_amdgcn_alignbyte(f3, f2, b);
    r.w = __builtin_amdgcn_alignbyte(f4, f3, b);
    return r;
}

// One thread = V consecutive tokens (one 16-byte vector) of one row.
// VEC: L is a multiple of V, so every vector is whole and 16-byte aligned.
template <typename T, bool VEC>
__global__ __launch_bounds__(256) void conv1d_kernel(const T* __restrict__ x,
                                                     const float* __restrict__ w,
                                                     const float* __restrict__ bias,
                                                     const float* __restrict__ x_prev,
                                                     T* __restrict__ out, int64_t rows, int64_t L,
                                                     int64_t dim, int64_t nvec) {
    constexpr int V = CElem<T>::kPer16;
    const int64_t total = rows * nvec;
    const int64_t gid = int64_t(blockIdx.x) * 256 + threadIdx.x;
    const bool active = gid < total;
    const int64_t g = active ? gid : total - 1;  // clamped: every lane reads valid memory
    const int64_t r = g / nvec;
    const int64_t v = g - r * nvec;
    const int64_t t0 = v * V;
    const int64_t d = r % dim;
    const T* xr = x + r * L;

    float xs[V + 3];  // xs[0..2]: the three inputs before t0; xs[3 + e]: token t0 + e
    if constexpr (VEC) {
        // the vector and the 4 inputs before it (cache hits: the lane below's vector)
        typedef typename Halo<T>::type H;
        const H hb = v == 0 ? H{} : *reinterpret_cast<const H*>(xr + t0 - 4);
        unpack_vec<T>(__builtin_nontemporal_load(reinterpret_cast<const u32x4*>(xr + t0)), xs + 3);
        float b4[4];
        unpack_halo<T>(hb, b4);
        xs[0] = b4[1]; xs[1] = b4[2]; xs[2] = b4[3];
    } else {
        // A row off a 16-byte boundary: the three aligned 16-byte blocks that
        // hold the vector and the 16 bytes before it, shifted into place. A
        // block past the tensor's last is read from that last one (it holds
        // only tokens past the row's end, which feed no stored output); the
        // block before the tensor is needed only for v = 0, whose history is
        // x_prev.
        const int64_t bo = (r * L + t0) * int64_t(sizeof(T));
        const int sh = int(bo & 15);
        const int64_t b0 = bo - sh, lastb = (rows * L * int64_t(sizeof(T)) - 1) & ~int64_t(15);
        const char* xb = reinterpret_cast<const char*>(x);
        const u32x4 bm = *reinterpret_cast<const u32x4*>(xb + max(b0 - 16, int64_t(0)));
        const u32x4 bc = *reinterpret_cast<const u32x4*>(xb + min(b0, lastb));
        const u32x4 bn = *reinterpret_cast<const u32x4*>(xb + min(b0 + 16, lastb));
        float before[V];
        unpack_vec<T>(bytes16_at(bm, bc, sh), before);
        unpack_vec<T>(bytes16_at(bc, bn, sh), xs + 3);
        xs[0] = before[V - 3]; xs[1] = before[V - 2]; xs[2] = before[V - 1];
    }
    if (v == 0) {
        xs[0] = x_prev ? x_prev[r * 3 + 0] : 0.0f;
        xs[1] = x_prev ? x_prev[r * 3 + 1] : 0.0f;
        xs[2] = x_prev ? x_prev[r * 3 + 2] : 0.0f;
    }
    const float4 wd = *reinterpret_cast<const float4*>(w + d * 4);
    const float bd = bias ? bias[d] : 0.0f;
    float o[V];
#pragma unroll
    for (int e = 0; e < V; ++e) o[e] = silu(conv4(wd, bd, xs[e], xs[e + 1], xs[e + 2], xs[e + 3]));
    if constexpr (VEC) {
        if (!active) return;
        __builtin_nontemporal_store(pack_vec<T>(o), reinterpret_cast<u32x4*>(out + r * L + t0));
    } else {
        // A row off a 16-byte boundary: the vector as one 16-byte store at its
        // (2- or 4-byte aligned) address when it lies inside the row, which
        // gfx950's global memory path takes whole; element stores at the row's end.
        if (!active) return;
        T* orow = out + r * L;
        if (t0 + V <= L) {
            const u32x4 vo = pack_vec<T>(o);
            __builtin_memcpy(orow + t0, &vo, 16);
        } else {
#pragma unroll
            for (int e = 0; e < V; ++e)
                if (t0 + e < L) orow[t0 + e] = from_f32<T>(o[e]);
        }
    }
}

// x_last[r] = the last three entries of x_prev[r] ++ x[r]; one thread per row.
// Reads everything before writing, so x_last may be x_prev itself.
template <typename T>
__global__ __launch_bounds__(256) void conv_last_kernel(const T* __restrict__ x,
                                                        const float* x_prev, float* x_last,
                                                        int64_t rows, int64_t L) {
    const int64_t r = int64_t(blockIdx.x) * 256 + threadIdx.x;
    if (r >= rows) return;
    float s[3];
#pragma unroll
    for (int k = 0; k < 3; ++k) {
        const int64_t t = L - 3 + k;
        s[k] = t >= 0 ? to_f32(x[r * L + t]) : (x_prev ? x_prev[r * 3 + 3 + t] : 0.0f);
    }
#pragma unroll
    for (int k = 0; k < 3; ++k) x_last[r * 3 + k] = s[k];
}

// One token per row: out = silu(bias + w . (s0, s1, s2, x)), state <- (s1, s2, x).
template <typename T>
__global__ __launch_bounds__(256) void conv_step_kernel(float* __restrict__ state,
                                                        const T* __restrict__ x,
                                                        const float* __restrict__ w,
                                                        const float* __restrict__ bias,
                                                        T* __restrict__ out, int64_t rows,
                                                        int64_t dim) {
    const int64_t r = int64_t(blockIdx.x) * 256 + threadIdx.x;
    if (r >= rows) return;
    const int64_t d = r % dim;
    const float s0 = state[r * 3 + 0], s1 = state[r * 3 + 1], s2 = state[r * 3 + 2];
    const float xv = to_f32(x[r]);
    const float4 wd = *reinterpret_cast<const float4*>(w + d * 4);
    out[r] = from_f32<T>(silu(conv4(wd, bias ? bias[d] : 0.0f, s0, s1, s2, xv)));
    state[r * 3 + 0] = s1;
    state[r * 3 + 1] = s2;
    state[r * 3 + 2] = xv;
}

// ---- gradients ----
//   g[t] = dout[t] silu'(pre[t]),  dx(s) = sum_k w[k] g[s + 3 - k],
//   dw[k] = sum_t g[t] xx(t - 3 + k),  dbias = sum_t g[t]
// A workgroup takes one channel d, a group of batch entries and a piece of
// the sequence (a contiguous range of 16-byte vectors), and walks the rows of
// its batch entries 256 vectors per trip, one vector per thread, with the
// next trip's loads in flight while it computes the current one. Each thread
// loads, beside its vector, the 4 inputs before it and the 4 inputs and
// output gradients after it (cache hits: the neighbouring lanes' vectors).
// dx of a vector needs g of the 3 tokens after it, which the thread holding
// the next vector forms anyway: a lane takes them from the lane above (a
// cross-lane shuffle), lane 63 of a wave from lane 0 of the next wave through
// LDS (one barrier per trip); only where the next vector lies outside the
// trip (the trip's last thread, or the end of a piece inside the row) does a
// thread form them itself, from its own loads; after a row's last vector
// they are 0. The thread's sums for dw and dbias, added over its trips in
// order, then over the workgroup in a fixed order, give one partial per
// (channel, batch group, piece); conv1d_bwd_reduce adds a channel's partials
// in order.
// The raw loads of one trip of one thread (t0 = its vector's first token).
// VEC: x and dout at t0 .. t0+V-1, x at t0-4 .. t0-1 (zero for the row's
// first vector), x and dout at t0+V .. t0+V+3 (zero for its last vector).
// Otherwise element by element: x at t0-3 .. t0+V+2, dout at t0 .. t0+V+2,
// zero outside the row.
template <typename T, bool VEC> struct Trip;
template <typename T> struct Trip<T, true> {
    static constexpr int V = CElem<T>::kPer16;
    u32x4 x, dy;
    typename Halo<T>::type xb, xa, da;
    __device__ __forceinline__ void load(const T* xr, const T* dr, int64_t t0, int64_t, bool first,
                                         bool last, const T*, const T*, int64_t) {
        typedef typename Halo<T>::type H;
        x = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(xr + t0));
        dy = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(dr + t0));
        xb = first ? H{} : *reinterpret_cast<const H*>(xr + t0 - 4);
        xa = last ? H{} : *reinterpret_cast<const H*>(xr + t0 + V);
        da = last ? H{} : *reinterpret_cast<const H*>(dr + t0 + V);
    }
    __device__ __forceinline__ void unpack(float* xs, float* dys, int64_t, int64_t) const {
        float b4[4];
        unpack_halo<T>(xb, b4);
        xs[0] = b4[1]; xs[1] = b4[2]; xs[2] = b4[3];
        unpack_vec<T>(x, xs + 3);
        unpack_vec<T>(dy, dys);
        float a4[4];
        unpack_halo<T>(xa, a4);
        xs[V + 3] = a4[0]; xs[V + 4] = a4[1]; xs[V + 5] = a4[2];
        unpack_halo<T>(da, a4);
        dys[V] = a4[0]; dys[V + 1] = a4[1]; dys[V + 2] = a4[2];
    }
};
template <typename T> struct Trip<T, false> {
    // A row off a 16-byte boundary: the aligned 16-byte blocks around the
    // vector, x at -16, 0, +16, +32 bytes and dout at 0, +16, +32 from the
    // block that holds the vector's first byte (sh bytes into it); a block
    // outside the tensor is read from its first or last block instead (it
    // holds only tokens outside the row, masked in unpack).
    static constexpr int V = CElem<T>::kPer16;
    u32x4 xb[4], db[3];
    int sh;
    __device__ __forceinline__ void load(const T* xr, const T* dr, int64_t t0, int64_t, bool, bool,
                                         const T* x, const T* dout, int64_t lastb) {
        const int64_t bo = reinterpret_cast<const char*>(xr + t0) - reinterpret_cast<const char*>(x);
        sh = int(bo & 15);
        const int64_t b0 = bo - sh;
        const char* xc = reinterpret_cast<const char*>(x);
        const char* dc = reinterpret_cast<const char*>(dout);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int64_t o = min(max(b0 + 16 * (i - 1), int64_t(0)), lastb);
            xb[i] = *reinterpret_cast<const u32x4*>(xc + o);
        }
#pragma unroll
        for (int i = 0; i < 3; ++i)
            db[i] = *reinterpret_cast<const u32x4*>(dc + min(b0 + 16 * i, lastb));
        (void)dr;
    }
    __device__ __forceinline__ void unpack(float* xs, float* dys, int64_t t0, int64_t L) const {
        float pre[V], cur[V], post[V];
        unpack_vec<T>(bytes16_at(xb[0], xb[1], sh), pre);
        unpack_vec<T>(bytes16_at(xb[1], xb[2], sh), cur);
        unpack_vec<T>(bytes16_at(xb[2], xb[3], sh), post);
        xs[0] = pre[V - 3]; xs[1] = pre[V - 2]; xs[2] = pre[V - 1];
#pragma unroll
        for (int e = 0; e < V; ++e) xs[3 + e] = cur[e];
        xs[V + 3] = post[0]; xs[V + 4] = post[1]; xs[V + 5] = post[2];
        unpack_vec<T>(bytes16_at(db[0], db[1], sh), cur);
        unpack_vec<T>(bytes16_at(db[1], db[2], sh), post);
#pragma unroll
        for (int e = 0; e < V; ++e) dys[e] = cur[e];
        dys[V] = post[0]; dys[V + 1] = post[1]; dys[V + 2] = post[2];
#pragma unroll
        for (int i = 0; i < V + 6; ++i) {
            const int64_t t = t0 - 3 + i;
            if (t < 0 || t >= L) xs[i] = 0.0f;
        }
#pragma unroll
        for (int i = 0; i < V + 3; ++i)
            if (t0 + i >= L) dys[i] = 0.0f;
    }
};

// Grid: dim * bgroups * pieces workgroups of 256 threads, blockIdx =
// (d * bgroups + bg) * pieces + piece. part: 5 floats per workgroup.
template <typename T, bool VEC>
__global__ __launch_bounds__(256) void conv1d_bwd_kernel(const T* __restrict__ x,
                                                         const float* __restrict__ w,
                                                         const float* __restrict__ bias,
                                                         const float* __restrict__ x_prev,
                                                         const T* __restrict__ dout,
                                                         T* __restrict__ dx, float* __restrict__ dx_prev,
                                                         float* __restrict__ part, int64_t batch,
                                                         int64_t L, int64_t dim, int64_t nvec,
                                                         int32_t bgroups, int32_t pieces) {
    constexpr int V = CElem<T>::kPer16;
    __shared__ float red[5][4];
    __shared__ float halo[2][4][4];  // by trip parity and wave: g of the wave's lane 0, first 3 tokens
    const int lane = threadIdx.x % 64, wv = threadIdx.x / 64;
    const int64_t d = blockIdx.x / (int64_t(bgroups) * pieces);
    const int bg = int(blockIdx.x / pieces % bgroups);
    const int sg = int(blockIdx.x % pieces);
    const int64_t b_lo = batch * bg / bgroups, b_hi = batch * (bg + 1) / bgroups;
    const int64_t v_lo = nvec * sg / pieces, v_hi = nvec * (sg + 1) / pieces;
    const int64_t per_row = (v_hi - v_lo + 255) / 256;  // trips per row, uniform over the workgroup
    const int64_t trips = (b_hi - b_lo) * per_row;
    const int64_t lastb = (batch * dim * L * int64_t(sizeof(T)) - 1) & ~int64_t(15);  // last 16-byte block
    const float4 wd = *reinterpret_cast<const float4*>(w + d * 4);
    const float bd = bias ? bias[d] : 0.0f;
    auto gof = [&](float pre, float dy) {  // dy * silu'(pre)
        const float s = rcp_hw(1.0f + exp2_hw(-pre * kLog2e));
        return dy * s * fmaf(pre, 1.0f - s, 1.0f);
    };
    // trip i: row (b_lo + i / per_row) * dim + d, vector v_lo + (i % per_row) * 256 + thread
    auto where = [&](int64_t i, int64_t& r, int64_t& v, int64_t& vc) {
        r = (b_lo + i / per_row) * dim + d;
        v = v_lo + (i % per_row) * 256 + threadIdx.x;
        vc = v < v_hi ? v : v_hi - 1;  // clamped: every lane reads valid memory
    };
    float aw[4] = {0.0f, 0.0f, 0.0f, 0.0f}, ab = 0.0f;
    Trip<T, VEC> cur;
    if (trips > 0) {
        int64_t r, v, vc;
        where(0, r, v, vc);
        cur.load(x + r * L, dout + r * L, vc * V, L, vc == 0, vc == nvec - 1, x, dout, lastb);
    }
    for (int64_t i = 0; i < trips; ++i) {
        int64_t r, v, vc;
        where(i, r, v, vc);
        Trip<T, VEC> nxt;
        if (i + 1 < trips) {
            int64_t r1, v1, vc1;
            where(i + 1, r1, v1, vc1);
            nxt.load(x + r1 * L, dout + r1 * L, vc1 * V, L, vc1 == 0, vc1 == nvec - 1, x, dout, lastb);
        }
        const int64_t t0 = vc * V;
        float xs[V + 6], dys[V + 3], gs[V + 3];
        cur.unpack(xs, dys, t0, L);
        if (vc == 0) {
#pragma unroll
            for (int e = 0; e < 3; ++e) xs[e] = x_prev ? x_prev[r * 3 + e] : 0.0f;
        }
#pragma unroll
        for (int e = 0; e < V; ++e) {
            const bool in_row = VEC || t0 + e < L;
            gs[e] = in_row ? gof(conv4(wd, bd, xs[e], xs[e + 1], xs[e + 2], xs[e + 3]), dys[e]) : 0.0f;
        }
        // g of the 3 tokens after the vector: 0 after the row's last vector;
        // else from the thread that holds the next vector when it is in this
        // trip, else formed here
        const bool row_end = VEC ? vc == nvec - 1 : t0 + V >= L;
        const bool from_next = threadIdx.x < 255 && v + 1 < v_hi;
        float hn[3];
#pragma unroll
        for (int e = 0; e < 3; ++e) hn[e] = __shfl_down(gs[e], 1, 64);
        const int hb = int(i & 1);
        if (lane == 0 && wv > 0) {
#pragma unroll
            for (int e = 0; e < 3; ++e) halo[hb][wv][e] = gs[e];
        }
        __syncthreads();
        if (lane == 63) {
#pragma unroll
            for (int e = 0; e < 3; ++e) hn[e] = halo[hb][(wv + 1) & 3][e];
        }
        if (row_end || from_next) {
#pragma unroll
            for (int e = 0; e < 3; ++e) gs[V + e] = row_end ? 0.0f : hn[e];
        } else {
#pragma unroll
            for (int e = V; e < V + 3; ++e) {
                const bool in_row = VEC || t0 + e < L;
                gs[e] = in_row ? gof(conv4(wd, bd, xs[e], xs[e + 1], xs[e + 2], xs[e + 3]), dys[e]) : 0.0f;
            }
        }
        float o[V];
#pragma unroll
        for (int e = 0; e < V; ++e)
            o[e] = fmaf(wd.x, gs[e + 3], fmaf(wd.y, gs[e + 2], fmaf(wd.z, gs[e + 1], wd.w * gs[e])));
        if (v < v_hi) {
            T* orow = dx + r * L;
            if constexpr (VEC) {
                __builtin_nontemporal_store(pack_vec<T>(o), reinterpret_cast<u32x4*>(orow + t0));
            } else if (t0 + V <= L) {
                // a row off a 16-byte boundary: one 16-byte store at the vector's address
                const u32x4 vo = pack_vec<T>(o);
                __builtin_memcpy(orow + t0, &vo, 16);
            } else {
#pragma unroll
                for (int e = 0; e < V; ++e)
                    if (t0 + e < L) orow[t0 + e] = from_f32<T>(o[e]);
            }
#pragma unroll
            for (int e = 0; e < V; ++e) {
                aw[0] = fmaf(gs[e], xs[e], aw[0]);
                aw[1] = fmaf(gs[e], xs[e + 1], aw[1]);
                aw[2] = fmaf(gs[e], xs[e + 2], aw[2]);
                aw[3] = fmaf(gs[e], xs[e + 3], aw[3]);
                ab += gs[e];
            }
            if (vc == 0 && dx_prev) {  // the inputs before token 0: dxx(j - 3) = sum_{k <= j} w[k] g[j - k]
                dx_prev[r * 3 + 0] = wd.x * gs[0];
                dx_prev[r * 3 + 1] = fmaf(wd.x, gs[1], wd.y * gs[0]);
                dx_prev[r * 3 + 2] = fmaf(wd.x, gs[2], fmaf(wd.y, gs[1], wd.z * gs[0]));
            }
        }
        cur = nxt;
    }
    // a fixed tree over the wave's lanes, then the four waves in order
    float v5[5] = {aw[0], aw[1], aw[2], aw[3], ab};
#pragma unroll
    for (int i = 0; i < 5; ++i)
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) v5[i] += __shfl_xor(v5[i], off, 64);
    if (lane == 0) {
#pragma unroll
        for (int i = 0; i < 5; ++i) red[i][threadIdx.x / 64] = v5[i];
    }
    __syncthreads();
    if (threadIdx.x < 5)
        part[int64_t(blockIdx.x) * 5 + threadIdx.x] =
            ((red[threadIdx.x][0] + red[threadIdx.x][1]) + red[threadIdx.x][2]) + red[threadIdx.x][3];
}

// dw[d,k] = sum over the channel's nparts partials part[d nparts + j][k], in
// order of j; dbias likewise from entry 4.
__global__ __launch_bounds__(256) void conv1d_bwd_reduce(const float* __restrict__ part,
                                                         float* __restrict__ dw, float* dbias,
                                                         int64_t dim, int32_t nparts) {
    const int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;
    if (i >= dim * 5) return;
    const int64_t d = i / 5;
    const int k = int(i % 5);
    float s = 0.0f;
    for (int j = 0; j < nparts; ++j) s += part[(d * nparts + j) * 5 + k];
    if (k < 4) dw[d * 4 + k] = s;
    else if (dbias) dbias[d] = s;
}

template <typename T>
hipError_t conv_bwd_t(const ConvBwdTensors& t, int64_t batch, int64_t L, int64_t dim, float* part,
                      ConvBwdPlan plan, hipStream_t st) {
    constexpr int V = CElem<T>::kPer16;
    const int64_t nvec = (L + V - 1) / V;
    const dim3 grid(unsigned(dim * plan.bgroups * plan.pieces)), block(256);
    const T* x = static_cast<const T*>(t.x);
    const T* dy = static_cast<const T*>(t.dout);
    T* dx = static_cast<T*>(t.dx);
    if (L % V == 0)
        hipLaunchKernelGGL((conv1d_bwd_kernel<T, true>), grid, block, 0, st, x, t.w, t.bias, t.x_prev,
                           dy, dx, t.dx_prev, part, batch, L, dim, nvec, plan.bgroups, plan.pieces);
    else
        hipLaunchKernelGGL((conv1d_bwd_kernel<T, false>), grid, block, 0, st, x, t.w, t.bias, t.x_prev,
                           dy, dx, t.dx_prev, part, batch, L, dim, nvec, plan.bgroups, plan.pieces);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(conv1d_bwd_reduce, dim3(unsigned((dim * 5 + 255) / 256)), dim3(256), 0, st, part,
                       t.dw, t.dbias, dim, plan.bgroups * plan.pieces);
    return hipGetLastError();
}

template <typename T>
hipError_t conv_t(const ConvTensors& t, int64_t rows, int64_t L, int64_t dim, hipStream_t st) {
    constexpr int V = CElem<T>::kPer16;
    const T* x = static_cast<const T*>(t.x);
    if (L > 0) {
        const int64_t nvec = (L + V - 1) / V;
        const int64_t blocks = (rows * nvec + 255) / 256;
        if (L % V == 0)
            hipLaunchKernelGGL((conv1d_kernel<T, true>), dim3(unsigned(blocks)), dim3(256), 0, st, x,
                               t.w, t.bias, t.x_prev, static_cast<T*>(t.out), rows, L, dim, nvec);
        else
            hipLaunchKernelGGL((conv1d_kernel<T, false>), dim3(unsigned(blocks)), dim3(256), 0, st, x,
                               t.w, t.bias, t.x_prev, static_cast<T*>(t.out), rows, L, dim, nvec);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (t.x_last) {
        hipLaunchKernelGGL((conv_last_kernel<T>), dim3(unsigned((rows + 255) / 256)), dim3(256), 0, st,
                           x, t.x_prev, t.x_last, rows, L);
        return hipGetLastError();
    }
    return hipSuccess;
}

template <typename T>
hipError_t conv_step_t(const ConvStepTensors& t, int64_t rows, int64_t dim, hipStream_t st) {
    hipLaunchKernelGGL((conv_step_kernel<T>), dim3(unsigned((rows + 255) / 256)), dim3(256), 0, st,
                       t.state, static_cast<const T*>(t.x), t.w, t.bias, static_cast<T*>(t.out),
                       rows, dim);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_conv(const ConvTensors& t, int64_t rows, int64_t L, int64_t dim, DType dtype,
                       hipStream_t stream) {
    return dtype == DType::BF16 ? conv_t<bf16_bits>(t, rows, L, dim, stream)
                                : conv_t<float>(t, rows, L, dim, stream);
}

ConvBwdPlan conv_bwd_plan(int64_t batch, int64_t L, int64_t dim, DType dtype) {
    const int64_t V = dtype == DType::BF16 ? 8 : 4;
    const int64_t nvec = (L + V - 1) / V;
    // Workgroups to fill the chip (kFill): batch groups first (a workgroup
    // keeps at least 2 rows while the batch allows), then pieces of the
    // sequence of at least 256 vectors.
    constexpr int64_t kFill = 8192;
    ConvBwdPlan p{1, 1};
    while (dim * p.bgroups * p.pieces < kFill) {
        if (int64_t(p.bgroups) * 4 <= batch) p.bgroups *= 2;
        else if (nvec / (int64_t(p.pieces) * 2) >= 256) p.pieces *= 2;
        else break;
    }
    return p;
}

hipError_t launch_conv_bwd(const ConvBwdTensors& t, int64_t batch, int64_t L, int64_t dim,
                           DType dtype, float* part, ConvBwdPlan plan, hipStream_t stream) {
    return dtype == DType::BF16 ? conv_bwd_t<bf16_bits>(t, batch, L, dim, part, plan, stream)
                                : conv_bwd_t<float>(t, batch, L, dim, part, plan, stream);
}

hipError_t launch_conv_last(const void* x, const float* x_prev, float* x_last, int64_t rows,
                            int64_t L, DType dtype, hipStream_t stream) {
    const dim3 grid(unsigned((rows + 255) / 256)), block(256);
    if (dtype == DType::BF16)
        hipLaunchKernelGGL((conv_last_kernel<bf16_bits>), grid, block, 0, stream,
                           static_cast<const bf16_bits*>(x), x_prev, x_last, rows, L);
    else
        hipLaunchKernelGGL((conv_last_kernel<float>), grid, block, 0, stream,
                           static_cast<const float*>(x), x_prev, x_last, rows, L);
    return hipGetLastError();
}

hipError_t launch_conv_step(const ConvStepTensors& t, int64_t rows, int64_t dim, DType dtype,
                            hipStream_t stream) {
    return dtype == DType::BF16 ? conv_step_t<bf16_bits>(t, rows, dim, stream)
                                : conv_step_t<float>(t, rows, dim, stream);
}

}  // namespace selscan
