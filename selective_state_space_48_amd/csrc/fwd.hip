// Forward selective scan (S6) kernels for gfx950.
//
// The recurrence per (batch b, channel d) row, from "State Space Models and
// Mamba" (multigrid.ai), section "Selective state: the change that made it
// work on text":
//     delta_t = softplus(delta_raw_t + dt_bias_d)
//     h_n     = exp(delta_t A_dn) h_n + delta_t B_nt x_t
//     y_t     = (sum_n C_nt h_n + D_d x_t) silu(z_t)
// Following the hardware-aware evaluation of "Mamba: Linear-Time Sequence
// Modeling with Selective State Spaces" (azimuth.plus), kernel fusion: every
// input is read from HBM once, the state lives in registers, and only y (and
// the final state) is written back; the (B, L, D, N) state tensor never exists.
//
// Mapping (MI355X-first, not the pages' GPU design):
// * One lane owns one (b, d) row and walks its tokens in order, so the scan is
//   a plain register recurrence with no cross-lane combine at all. The 64 rows
//   of a wave share b, which makes B_t and C_t wave-uniform: they are fed to
//   the VALU as scalar (SGPR) operands, costing no VGPRs, no LDS traffic and
//   no vector-memory instructions.
// * A small pre-pass packs B and C into fp32, ordered so that the operands one
//   wave needs for one sub-block of tokens (its N/G states x G tokens, for B
//   and for C) are 2 x 16 contiguous floats: one s_load_dwordx16 each, loaded
//   one sub-block ahead. This removes all scalar unpacking and address math
//   from the inner loop, and turns B/C reads into one contiguous stream per
//   batch entry (long rows no longer touch 2N distant pages per sub-block).
// * The 16 states of a row are split across the G waves of a workgroup (N/G
//   states each), so that B*d/64*G waves fill the 1024 SIMDs. Per token and
//   state the inner loop is one multiply (l*A), one v_exp_f32, one multiply
//   (w*B), and two FMAs (state, readout): the floor of the method.
// * Per-token work that does not depend on n (softplus, w = delta*x, D*x,
//   silu(z)) is computed once per row and token, split between the waves by
//   token slices and shared through LDS. Partial readouts of the G waves are
//   summed through LDS in a fixed order (deterministic).
// * Time advances in 32-token chunks. Each wave loads its own token slice of
//   x, delta and z straight from HBM in 16-byte vectors, one chunk ahead, so
//   HBM latency hides behind a chunk of arithmetic; the G slices of a chunk
//   tile whole cache lines. Two barriers per chunk, about 54 KB of LDS at G=4.
// * Long sequences with few rows are cut into segments scanned in parallel
//   ("parallel scan" of the same page: the pair (decay, state) composes
//   associatively): a state pass gives each segment's end state from zero and
//   its summed step size, a carry pass composes them in order, and the output
//   pass rescans each segment from its carried-in state.
#include "common.hpp"
#include "launch.hpp"

namespace selscan {
namespace {

template <typename T> struct Elem;
template <> struct Elem<float> { static constexpr int kPer16 = 4; };
template <> struct Elem<bf16_bits> { static constexpr int kPer16 = 8; };

// E elements of T in the low bytes of a 16-byte register quad: E = 4 or 8
// for bf16 (8 or 16 bytes), 4 for fp32.
template <typename T, int E = Elem<T>::kPer16>
__device__ __forceinline__ void unpack16(const uint4& v, float* o) {
    if constexpr (sizeof(T) == 4) {
        o[0] = __uint_as_float(v.x); o[1] = __uint_as_float(v.y);
        o[2] = __uint_as_float(v.z); o[3] = __uint_as_float(v.w);
    } else {
        o[0] = bf16_lo(v.x); o[1] = bf16_hi(v.x); o[2] = bf16_lo(v.y); o[3] = bf16_hi(v.y);
        if constexpr (E == 8) {
            o[4] = bf16_lo(v.z); o[5] = bf16_hi(v.z); o[6] = bf16_lo(v.w); o[7] = bf16_hi(v.w);
        }
    }
}

template <typename T, int E = Elem<T>::kPer16>
__device__ __forceinline__ uint4 pack16(const float* f) {
    uint4 v;
    if constexpr (sizeof(T) == 4) {
        v.x = __float_as_uint(f[0]); v.y = __float_as_uint(f[1]);
        v.z = __float_as_uint(f[2]); v.w = __float_as_uint(f[3]);
    } else {
        auto p = [](float a, float b) {
            return pack_bf16x2(a, b);
        };
        v.x = p(f[0], f[1]); v.y = p(f[2], f[3]);
        if constexpr (E == 8) {
            v.z = p(f[4], f[5]); v.w = p(f[6], f[7]);
        } else {
            v.z = v.w = 0u;
        }
    }
    return v;
}

// Streaming global accesses of 16 (or 8) bytes: x, delta and z are read
// exactly once and y is written exactly once, so they are marked
// non-temporal (no reuse).
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
template <int BYTES = 16>
__device__ __forceinline__ uint4 ldg_stream(const void* p) {
    if constexpr (BYTES == 16) {
        const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
        return make_uint4(v.x, v.y, v.z, v.w);
    } else {
        const u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
        return make_uint4(v.x, v.y, 0u, 0u);
    }
}
template <int BYTES = 16>
__device__ __forceinline__ void stg_stream(void* p, const uint4& v) {
    if constexpr (BYTES == 16) {
        u32x4 w = {v.x, v.y, v.z, v.w};
        __builtin_nontemporal_store(w, reinterpret_cast<u32x4*>(p));
    } else {
        u32x2 w = {v.x, v.y};
        __builtin_nontemporal_store(w, reinterpret_cast<u32x2*>(p));
    }
}

// Bytes [sh, sh + 16) of the 32 bytes lo ++ hi (sh = 0..15): a row that
// does not start on a 16-byte boundary is read with aligned loads and shifted
// into place here.
__device__ __forceinline__ uint4 extract16(const uint4& lo, const uint4& hi, int sh) {
    // dwords sh/4 .. sh/4 + 4 of the 8, then the byte shift within them
    const bool s4 = sh & 4, s8 = sh & 8;
    const uint32_t e0 = s4 ? lo.y : lo.x, e1 = s4 ? lo.z : lo.y, e2 = s4 ? lo.w : lo.z,
                   e3 = s4 ? hi.x : lo.w, e4 = s4 ? hi.y : hi.x, e5 = s4 ? hi.z : hi.y,
                   e6 = s4 ? hi.w : hi.z;
    const uint32_t f0 = s8 ? e2 : e0, f1 = s8 ? e3 : e1, f2 = s8 ? e4 : e2, f3 = s8 ? e5 : e3,
                   f4 = s8 ? e6 : e4;
    const uint32_t b = uint32_t(sh & 3);
    return make_uint4(__builtin_amdgcn_alignbyte(f1, f0, b), __builtin_amdgcn_alignbyte(f2, f1, b),
                      __builtin_amdgcn_alignbyte(f3, f2, b), __builtin_amdgcn_alignbyte(f4, f3, b));
}

// 16 floats through the constant address space: with a wave-uniform address
// the compiler must use one scalar load (s_load_dwordx16) into SGPRs. Going
// through an integer keeps address-space inference from turning it back into
// a global-memory (vector) load.
typedef float f32x16 __attribute__((ext_vector_type(16)));
__device__ __forceinline__ f32x16 sload64(const float* p) {
    using CP = const __attribute__((address_space(4))) f32x16*;
    return *(CP)(reinterpret_cast<uintptr_t>(p));
}

// Packed operand layout (fp32): P[b][s][g][k][j][e] = (k ? C : B ln 2)[b, g*NG + j, s*G + e]
// for sub-block s of G tokens, wave group g, state j < NG = 16/G, token e < G;
// zero for tokens >= L. One (b, s, g) record is 2 x 16 floats.
constexpr int kRec = 32;  // floats per (b, s, g) record

// LDS of one workgroup: the per-token pairs (l, w) of the current chunk and
// the partial readouts of the G waves, accessed 16 bytes (a piece) at a time.
// On gfx950 a 16-byte LDS write is served 8 lanes at a time from 32 banks and
// a 16-byte read 16 lanes at a time from 64 banks, so the 8 lanes of a write
// must hit distinct pieces mod 8 and the 16 lanes of a read distinct pieces
// mod 16.
// * (l, w): rows of 17 pieces; token pair k of a row at piece lw_swizzle(k).
//   The scan reads one pair of 16 consecutive rows (distinct at the odd
//   stride); the G threads of a row write their token slices in the same
//   instruction, and without the swizzle slices 64 bytes apart (G = 4) would
//   share banks. The swizzle keeps the pairs of a sub-block consecutive, so
//   the 8 slices of one row (G = 8: 2 pairs each, of one parity) still meet
//   two to a bank group.
// * partial readouts: rows of 8 pieces (4 tokens each), piece k of row r at
//   k ^ f(r) with f a permutation of r mod 8: the scan writes one piece of 8
//   consecutive rows, and the per-token threads read 4 rows x 4 slices
//   (G = 4), of which rows r and r + 2 share a half of the banks and get
//   pieces of opposite parity. With one wave (a thread per row) rows are 9
//   pieces apart instead.
template <int G>
__device__ __forceinline__ constexpr int lw_swizzle(int k) {
    // flip a bit of the pair index in the upper half of the chunk's 16 pairs:
    // the pieces (mod 8) of the G threads of two rows then all differ
    return k ^ (((k >> 3) & 1) * (G == 2 ? 4 : G == 4 ? 2 : 0));
}
template <int G>
__device__ __forceinline__ int yp_piece(int row, int k) {
    if constexpr (G == 1) return row * (kChunk / 4 + 1) + k;
    else return row * (kChunk / 4) + (k ^ (((row >> 1) & 3) | ((row & 1) << 2)));
}

template <int G, int CH, int MODE>
struct alignas(16) Smem {
    static constexpr int kPairB = CH * 8 + 16;  // float2-per-token row stride (bytes)
    static constexpr int kYB = CH * 4 + (G == 1 ? 16 : 0);  // float-per-token row stride (bytes)
    unsigned char lw[kWave * kPairB];
    static constexpr int kBase = MODE >= 4 ? MODE - 4 : MODE;  // 4, 5: 0, 1 with the conv
    static constexpr bool kReadout = kBase == 0 || kBase == 3;
    unsigned char yp[kReadout ? G : 1][kReadout ? kWave * kYB : 16];
    double lsum[kBase == 1 ? G : 1][kWave];
};

struct FwdKArgs {
    const void* x;
    const void* delta;
    const void* z;
    const float* A;
    const float* P;    // packed B/C
    const float* D;
    const float* dt_bias;
    void* y;
    float* last_state;
    const float* h0;   // [segments][rows][N] carried-in states, or null
    float* seg_state;  // [segments][rows][N] (state pass)
    double* seg_lsum;  // [segments][rows]    (state pass)
    int64_t batch, L, dim, seg_len;
    int64_t psub;      // sub-blocks per batch entry in P
    int32_t segments, row_blocks;
    // MODE 2 and 3 only:
    float* ckpt;       // [ceil(L/16)][batch*dim][N]: the state before every 16th token
    // MODE 4 and 5 only: x is the convolution's input (see below)
    const float* cw;      // [dim][4] taps, tap k on the input 3 - k tokens back
    const float* cb;      // [dim] or null
    const float* cx_prev; // [batch*dim][3] inputs before token 0 (oldest first), or null
    // warp-specialised kernel only: 256 bytes of workspace that the io lanes
    // of rows past dim store to, so that every lane issues the same stores
    void* dump;
};

// MODE 0: output pass (y, and last_state from the final segment).
// MODE 1: state pass (each segment's end state from zero, and its summed l).
// MODE 2: checkpoint pass of the backward: the recurrence alone, storing the
//         state before every 16th token.
// MODE 3: output pass that also stores those checkpoints (a forward whose
//         backward follows).
// MODE 4, 5: MODE 0, 1 with the block's causal depthwise convolution (width
//         4) and SiLU applied to x on the fly, in the per-token phase: the
//         scan's input is silu(cb + sum_k cw[k] x[t - 3 + k]), which is never
//         written to memory.
template <typename T, int G, bool GATE, bool VEC, int MODE>
__global__ __launch_bounds__(kWave* G) void fwd_kernel(FwdKArgs a) {
    constexpr int CH = kChunk;
    constexpr int NG = kN / G;              // states per wave
    constexpr int SB = G;                   // tokens per sub-block (NG * SB = 16)
    constexpr int NSB = CH / SB;            // sub-blocks per chunk
    constexpr int TS = CH / G;              // tokens per wave in the per-token phases
    // elements per vector access: 16 bytes, or 8 when the slice is shorter
    // (bf16 with 8 waves: 4 tokens)
    constexpr int V = Elem<T>::kPer16 < TS ? Elem<T>::kPer16 : TS;
    constexpr int VB = V * int(sizeof(T));  // bytes per vector access
    constexpr int SV = TS / V;              // vectors per row slice
    constexpr bool CONV = MODE >= 4;                  // convolution + SiLU in front
    constexpr int BASE = CONV ? MODE - 4 : MODE;
    constexpr bool READOUT = BASE == 0 || BASE == 3;  // y = C.h + D x, gated
    constexpr bool CKPT = BASE == 2 || BASE == 3;     // states every 16 tokens
    constexpr bool LOADZ = GATE && READOUT;
    static_assert(!CKPT || G == 4, "checkpoints: 4 waves of 4 states");
    static_assert(!CONV || (G == 4 && BASE < 2), "the convolution: 4 waves, output or state pass");
    static_assert(TS % V == 0 && SV >= 1, "tile shape");
    using S = Smem<G, CH, MODE>;
    __shared__ S sm;

    const T* __restrict__ X = static_cast<const T*>(a.x);
    const T* __restrict__ DL = static_cast<const T*>(a.delta);
    const T* __restrict__ Z = static_cast<const T*>(a.z);
    // byte offset of the last 16-byte block of x, delta and z (without VEC)
    const int64_t last_block = (a.batch * a.dim * a.L * int64_t(sizeof(T)) - 1) & ~int64_t(15);

    const int tid = threadIdx.x;
    // The wave index is uniform across the wave; saying so lets every address
    // derived from it (the packed B/C records) live in SGPRs.
    const int wv = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int lane = tid % kWave;

    // block -> (segment, batch entry, 64-row block)
    int64_t blk = xcd_tile(blockIdx.x, gridDim.x);
    const int rb = int(blk % a.row_blocks);
    blk /= a.row_blocks;
    const int64_t b = blk % a.batch;
    const int seg = int(blk / a.batch);

    const int64_t d0 = int64_t(rb) * kWave;
    const int64_t d = d0 + lane;
    const bool row_ok = d < a.dim;
    const int64_t row = b * a.dim + (row_ok ? d : d0);  // clamped for safe reads
    const int64_t t_begin = int64_t(seg) * a.seg_len;
    const int64_t t_end = min(a.L, t_begin + a.seg_len);
    const int nchunks = int((t_end - t_begin + CH - 1) / CH);
    const int n0 = wv * NG;

    // The per-token phases use their own mapping, chosen for memory access:
    // thread (pr, pq) takes row pr of the block and token slice pq, so the G
    // threads of a row are adjacent lanes reading one contiguous row segment.
    const int pr = tid / G, pq = tid % G;
    const int64_t dp = d0 + pr;
    const bool prow_ok = dp < a.dim;
    const int64_t prow = b * a.dim + (prow_ok ? dp : d0);  // clamped for safe reads
    const float biasl = (a.dt_bias && prow_ok) ? a.dt_bias[dp] * kLog2e : 0.0f;  // bias / ln 2
    const float Dd = (a.D && prow_ok) ? a.D[dp] : 0.0f;
    float4 cw4 = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    float cbias = 0.0f;
    if constexpr (CONV) {
        if (prow_ok) cw4 = *reinterpret_cast<const float4*>(a.cw + dp * 4);
        cbias = (a.cb && prow_ok) ? a.cb[dp] : 0.0f;
    }
    float An[NG], h[NG];
#pragma unroll
    for (int j = 0; j < NG; ++j) {
        An[j] = row_ok ? a.A[d * kN + n0 + j] : 0.0f;
        h[j] = (a.h0 && row_ok) ? a.h0[(int64_t(seg) * a.batch * a.dim + b * a.dim + d) * kN + n0 + j]
                                : 0.0f;
    }
    double lsum_acc = 0.0;
    // this wave's NG states of a row, to 16-byte aligned memory
    auto store_state = [&](float* dst, const float* hv) {
        if constexpr (NG >= 4) {
#pragma unroll
            for (int k = 0; k < NG / 4; ++k)
                reinterpret_cast<float4*>(dst)[k] = make_float4(hv[4 * k], hv[4 * k + 1], hv[4 * k + 2], hv[4 * k + 3]);
        } else {
            *reinterpret_cast<float2*>(dst) = make_float2(hv[0], hv[1]);
        }
    };

    // ---- thread (pr, pq)'s token slice [pq*TS, pq*TS+TS) of a chunk, straight from HBM ----
    // The G threads of a row read adjacent slices, so a wave's load covers
    // 64/G rows with CH contiguous tokens each. Two register sets alternate by
    // chunk parity.
    // Without VEC, each vector is read as the two aligned 16-byte blocks
    // that hold it and shifted into place in the prologue (RAW), so that the
    // loads stay in flight a chunk ahead like the VEC ones. With 1 or 2 waves
    // (long token slices) that would take too many registers: there the
    // loads are element by element, converted on arrival.
    constexpr bool RAW = !VEC && G >= 4;
    constexpr int NR = RAW ? 2 : 1;  // 16-byte loads per vector
    struct Slice {
        uint4 x[SV * NR], d[SV * NR], z[LOADZ ? SV * NR : 1];
        uint4 xp[1];  // with the convolution: the 16 bytes of x before the slice
    };
    Slice sl0, sl1;
    // With 16-byte rows (VEC) the loads are issued without any condition: a
    // vector past the end of the row is read from the row's last vector
    // instead (always valid memory) and its values are discarded by the
    // prologue's masked path. Branch-free loads keep the compiler from
    // merging differently-allocated register sets after the loads, which
    // would make it wait for them there. Without VEC, element loads test
    // each token.
    auto load_vec = [&](const T* base, int64_t tk) {
        return ldg_stream<VB>(base + prow * a.L + min(tk, a.L - V));
    };
    // The convolution's history of a slice: the V inputs before it (real
    // data also across a segment boundary; at token 0 the prologue takes the
    // caller's previous inputs instead).
    auto load_hist = [&](int64_t ts, Slice& sl) {
        if constexpr (CONV) {
            if constexpr (VEC) {
                sl.xp[0] = ldg_stream(X + prow * a.L + max(int64_t(0), min(ts - V, a.L - V)));
            } else if constexpr (RAW) {
                // the aligned block before the one that holds the slice's
                // first byte: with that block, it holds the 16 bytes before
                // the slice (shifted in the prologue)
                const int64_t b0 = ((prow * a.L + ts) * int64_t(sizeof(T))) & ~int64_t(15);
                sl.xp[0] = *reinterpret_cast<const uint4*>(reinterpret_cast<const char*>(X) +
                                                           min(max(b0 - 16, int64_t(0)), last_block));
            } else {
                float f[V];
#pragma unroll
                for (int e = 0; e < V; ++e) {
                    const int64_t tk = ts - V + e;
                    f[e] = (tk >= 0 && tk < a.L) ? to_f32(X[prow * a.L + tk]) : 0.0f;
                }
                sl.xp[0] = pack16<T>(f);
            }
        }
    };
    auto load_slice = [&](int c, Slice& sl) {
        const int64_t ts = t_begin + int64_t(c) * CH + pq * TS;
        const int64_t off = prow * a.L + ts;
        load_hist(ts, sl);
#pragma unroll
        for (int k = 0; k < SV; ++k) {
            const int64_t tk = ts + k * V;
            if constexpr (VEC) {
                sl.x[k] = load_vec(X, tk);
                sl.d[k] = load_vec(DL, tk);
                if constexpr (LOADZ) sl.z[k] = load_vec(Z, tk);
            } else if constexpr (RAW) {
                // The 16-byte blocks at and after the vector's start. A block
                // that starts past the tensor's last block is read from that
                // last block instead (always valid memory): it holds only
                // tokens past the row's end, whose values the prologue's
                // masked path discards.
                // Cached loads (not streaming): a row's chunk straddles cache
                // lines that the next chunk's loads touch again.
                const int64_t b0 = ((off + k * V) * int64_t(sizeof(T))) & ~int64_t(15);
                const int64_t b1 = min(b0 + 16, last_block), bb = min(b0, last_block);
                auto ld = [](const T* base, int64_t byte) {
                    return *reinterpret_cast<const uint4*>(reinterpret_cast<const char*>(base) + byte);
                };
                sl.x[2 * k] = ld(X, bb);
                sl.x[2 * k + 1] = ld(X, b1);
                sl.d[2 * k] = ld(DL, bb);
                sl.d[2 * k + 1] = ld(DL, b1);
                if constexpr (LOADZ) {
                    sl.z[2 * k] = ld(Z, bb);
                    sl.z[2 * k + 1] = ld(Z, b1);
                }
            } else {
                float fx[V], fd[V], fz[V];
#pragma unroll
                for (int e = 0; e < V; ++e) {
                    const bool ok = tk + e < t_end;
                    fx[e] = ok ? to_f32(X[off + k * V + e]) : 0.0f;
                    fd[e] = ok ? to_f32(DL[off + k * V + e]) : 0.0f;
                    fz[e] = (LOADZ && ok) ? to_f32(Z[off + k * V + e]) : 0.0f;
                }
                sl.x[k] = pack16<T, V>(fx);
                sl.d[k] = pack16<T, V>(fd);
                if constexpr (LOADZ) sl.z[k] = pack16<T, V>(fz);
            }
        }
    };
    // Two consecutive chunks at once, tensor by tensor, so that when a row's
    // chunk is only half a 128-byte line (bf16: 32 tokens = 64 bytes) both
    // halves are requested back to back and the line is fetched once.
    auto load_pair = [&](int c, Slice& s0, Slice& s1) {
        const int64_t ts = t_begin + int64_t(c) * CH + pq * TS;
        load_hist(ts, s0);
        load_hist(ts + CH, s1);
#pragma unroll
        for (int k = 0; k < SV; ++k) {
            s0.x[k] = load_vec(X, ts + k * V);
            s1.x[k] = load_vec(X, ts + CH + k * V);
        }
#pragma unroll
        for (int k = 0; k < SV; ++k) {
            s0.d[k] = load_vec(DL, ts + k * V);
            s1.d[k] = load_vec(DL, ts + CH + k * V);
        }
        if constexpr (LOADZ) {
#pragma unroll
            for (int k = 0; k < SV; ++k) {
                s0.z[k] = load_vec(Z, ts + k * V);
                s1.z[k] = load_vec(Z, ts + CH + k * V);
            }
        }
    };

    // The swizzled pieces of this thread's token pairs: k = pq TS/2 + jj maps
    // to pq TS/2 + (jj ^ X) with X < TS/2 fixed per thread.
    int lw_piece[TS / 2];
#pragma unroll
    for (int jj = 0; jj < TS / 2; ++jj) lw_piece[jj] = lw_swizzle<G>(pq * (TS / 2) + jj);
    // ---- per-token phase before the scan ----
    // (l, w) go to LDS for all G waves; x (for the D skip) and silu(z) stay
    // in this thread's registers until its epilogue of the same slice. Tokens past the segment
    // end get l = w = 0, which makes their scan step the identity. B was
    // scaled by ln 2 when packed, so w = l * x with l in log2 units.
    auto prologue = [&](int c, const Slice& sl, float* dxo, float* gzo) {
        const int64_t ts = t_begin + int64_t(c) * CH + pq * TS;
        float xs[TS], ds[TS], zs[TS];
#pragma unroll
        for (int k = 0; k < SV; ++k) {
            if constexpr (!RAW) {
                unpack16<T, V>(sl.x[k], xs + k * V);
                unpack16<T, V>(sl.d[k], ds + k * V);
                if constexpr (LOADZ) unpack16<T, V>(sl.z[k], zs + k * V);
            } else {
                const int sh = int(((prow * a.L + ts + k * V) * int64_t(sizeof(T))) & 15);
                unpack16<T, V>(extract16(sl.x[2 * k], sl.x[2 * k + 1], sh), xs + k * V);
                unpack16<T, V>(extract16(sl.d[2 * k], sl.d[2 * k + 1], sh), ds + k * V);
                if constexpr (LOADZ) unpack16<T, V>(extract16(sl.z[2 * k], sl.z[2 * k + 1], sh), zs + k * V);
            }
        }
        if constexpr (CONV) {
            // x <- silu(cb + sum_k cw[k] x[t - 3 + k]) over the window of the
            // 3 inputs before the slice and the slice itself
            float hp[V], win[TS + 3];
            if constexpr (RAW) {
                const int sh = int(((prow * a.L + ts) * int64_t(sizeof(T))) & 15);
                unpack16<T>(extract16(sl.xp[0], sl.x[0], sh), hp);
            } else {
                unpack16<T>(sl.xp[0], hp);
            }
#pragma unroll
            for (int e = 0; e < 3; ++e) win[e] = hp[V - 3 + e];
            if (ts == 0) {
#pragma unroll
                for (int e = 0; e < 3; ++e) win[e] = a.cx_prev ? a.cx_prev[prow * 3 + e] : 0.0f;
            }
#pragma unroll
            for (int e = 0; e < TS; ++e) win[3 + e] = xs[e];
#pragma unroll
            for (int e = 0; e < TS; ++e)
                xs[e] = silu(fmaf(cw4.w, win[e + 3], fmaf(cw4.z, win[e + 2],
                             fmaf(cw4.y, win[e + 1], fmaf(cw4.x, win[e], cbias)))));
        }
        float4* lwrow = reinterpret_cast<float4*>(&sm.lw[pr * S::kPairB]);
        auto body = [&](auto masked) {
            const int nvalid = masked ? int(min(int64_t(TS), max(int64_t(0), t_end - ts))) : TS;
#pragma unroll
            for (int j = 0; j < TS; j += 2) {
                float l[2], w[2];
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    l[u] = softplus_log2_of(fmaf(ds[j + u], kLog2e, biasl));
                    if (masked && j + u >= nvalid) {  // past the end: an identity step
                        l[u] = 0.0f;
                        xs[j + u] = 0.0f;
                    }
                    w[u] = l[u] * xs[j + u];
                    if constexpr (BASE == 1) lsum_acc += double(l[u]);
                    if constexpr (READOUT) {
                        // the D skip: x, multiplied in the epilogue's FMA (with
                        // one wave, whose 32 tokens a thread holds, the product)
                        dxo[j + u] = G == 1 ? Dd * xs[j + u] : xs[j + u];
                        if constexpr (LOADZ) gzo[j + u] = silu(zs[j + u]);
                    }
                }
                lwrow[lw_piece[j / 2]] = make_float4(l[0], w[0], l[1], w[1]);
            }
        };
        if (t_begin + int64_t(c + 1) * CH <= t_end) body(std::false_type{});
        else body(std::true_type{});
    };
    // ---- the scan over one chunk: this wave's NG states, all CH tokens ----
    // Software pipeline, one sub-block ahead: wait for the previous loads,
    // issue the next sub-block's B/C record (scalar) and (l, w) (LDS) loads,
    // then compute from registers only. lgkmcnt covers both kinds of load (and
    // LDS writes), so the wait must come before the next loads are issued; for
    // the same reason a sub-block's partial readouts are written to LDS one
    // sub-block later, right after those loads, so that the next wait does not
    // wait for a write issued just before it.
    auto scan_chunk = [&](int c) {
        const int64_t s0 = (t_begin + int64_t(c) * CH) / SB;          // first sub-block
        const float* rec = a.P + ((b * a.psub + s0) * G + wv) * kRec;  // this wave's record
        const float2* lw2 = reinterpret_cast<const float2*>(&sm.lw[lane * S::kPairB]);
        // the (l, w) of the SB tokens of sub-block sb: SB/2 consecutive token
        // pairs starting at piece lw_swizzle(sb * SB / 2) (the swizzle keeps the
        // pairs of a sub-block together); single tokens for SB = 1
        auto read_lw = [&](int sb, float2* out) {
            if constexpr (SB >= 2) {
                const float4* q4 = reinterpret_cast<const float4*>(lw2) + lw_swizzle<G>(sb * (SB / 2));
#pragma unroll
                for (int e = 0; e < SB / 2; ++e) {
                    const float4 v = q4[e];
                    out[2 * e] = make_float2(v.x, v.y);
                    out[2 * e + 1] = make_float2(v.z, v.w);
                }
            } else {
                out[0] = lw2[sb];
            }
        };
        float* yp = reinterpret_cast<float*>(&sm.yp[READOUT ? wv : 0][0]);
        // Ping-pong operand buffers (two sub-blocks per loop trip), so that no
        // register has to be copied at the loop back-edge.
        f32x16 B0 = sload64(rec), C0, B1, C1;
        if constexpr (READOUT) C0 = sload64(rec + 16);
        float2 l0[SB], l1[SB];
        read_lw(0, l0);
        float yA[SB], yB[SB];
        auto put = [&](int sb, const float* yv) {  // partial readouts of sub-block sb
            if constexpr (SB >= 4) {
#pragma unroll
                for (int k = 0; k < SB / 4; ++k)
                    reinterpret_cast<float4*>(yp)[yp_piece<G>(lane, sb * (SB / 4) + k)] =
                        make_float4(yv[4 * k], yv[4 * k + 1], yv[4 * k + 2], yv[4 * k + 3]);
            } else if constexpr (SB == 2) {
                *reinterpret_cast<float2*>(yp + 4 * yp_piece<G>(lane, sb >> 1) + 2 * (sb & 1)) =
                    make_float2(yv[0], yv[1]);
            } else {
                yp[4 * yp_piece<G>(lane, sb >> 2) + (sb & 3)] = yv[0];
            }
        };
        auto half = [&](int sb, const f32x16& Bc, const f32x16& Cc, const float2* lc, f32x16& Bn,
                        f32x16& Cn, float2* ln, const float* yprev, float* yv) {
            const int sbn = sb + 1 < NSB ? sb + 1 : sb;  // stays inside the chunk
            if constexpr (CKPT) {
                // the state before tokens 0 and 16 of the chunk
                const int64_t k = (t_begin + int64_t(c) * CH + sb * SB) / 16;
                if ((sb * SB) % 16 == 0 && row_ok && k * 16 < t_end)
                    *reinterpret_cast<float4*>(a.ckpt + (k * a.batch * a.dim + row) * kN + n0) =
                        make_float4(h[0], h[1], h[2], h[3]);
            }
            __builtin_amdgcn_s_waitcnt(0xc07f);          // lgkmcnt(0): current operands ready
            __builtin_amdgcn_sched_barrier(0);
            const float* nrec = rec + int64_t(sbn) * (G * kRec);
            Bn = sload64(nrec);
            if constexpr (READOUT) Cn = sload64(nrec + 16);
            read_lw(sbn, ln);
            // The previous sub-block's readouts. At sb = 0 there is none: the
            // write goes to the chunk's last slot, which the final write below
            // overwrites (same wave, LDS accesses in order).
            if constexpr (READOUT) put((sb + NSB - 1) % NSB, yprev);
            __builtin_amdgcn_sched_barrier(0);
            // All decays and input terms first, then the dependent FMAs, so
            // that no FMA is scheduled right behind the exponential it uses.
            float dA[SB][NG], u[SB][NG];
#pragma unroll
            for (int e = 0; e < SB; ++e)
#pragma unroll
                for (int j = 0; j < NG; ++j) dA[e][j] = exp2_hw(lc[e].x * An[j]);
#pragma unroll
            for (int e = 0; e < SB; ++e)
#pragma unroll
                for (int j = 0; j < NG; ++j) u[e][j] = lc[e].y * Bc[j * SB + e];
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int e = 0; e < SB; ++e) {
                float acc = 0.0f;
#pragma unroll
                for (int j = 0; j < NG; ++j) {
                    h[j] = fmaf(dA[e][j], h[j], u[e][j]);
                    if constexpr (READOUT) acc = fmaf(Cc[j * SB + e], h[j], acc);
                }
                yv[e] = acc;
            }
        };
        static_assert(NSB % 2 == 0, "sub-blocks per chunk must be even");
#pragma unroll
        for (int e = 0; e < SB; ++e) yB[e] = 0.0f;
#pragma unroll 1
        for (int sb = 0; sb < NSB; sb += 2) {
            half(sb, B0, C0, l0, B1, C1, l1, yB, yA);
            half(sb + 1, B1, C1, l1, B0, C0, l0, yA, yB);
        }
        if constexpr (READOUT) put(NSB - 1, yB);
    };

    // ---- per-token phase after the scan: sum partial readouts, D skip, gate, store ----
    auto epilogue = [&](int c, const float* dx, const float* gz) {
        const int64_t ts = t_begin + int64_t(c) * CH + pq * TS;
        float yv[TS];
#pragma unroll
        for (int j = 0; j < TS; j += 4) {
            const int yq = yp_piece<G>(pr, (pq * TS + j) / 4);
            float4 acc = reinterpret_cast<const float4*>(&sm.yp[0][0])[yq];
#pragma unroll
            for (int g = 1; g < G; ++g) {
                const float4 q = reinterpret_cast<const float4*>(&sm.yp[g][0])[yq];
                acc.x += q.x; acc.y += q.y; acc.z += q.z; acc.w += q.w;
            }
            yv[j] = acc.x; yv[j + 1] = acc.y; yv[j + 2] = acc.z; yv[j + 3] = acc.w;
        }
#pragma unroll
        for (int j = 0; j < TS; ++j) {
            yv[j] = G == 1 ? yv[j] + dx[j] : fmaf(Dd, dx[j], yv[j]);
            if constexpr (LOADZ) yv[j] *= gz[j];
        }
        T* Y = static_cast<T*>(a.y) + prow * a.L;
        // Rows off a 16-byte boundary (RAW), chunk wholly inside the row: the
        // thread's vectors are stored as they are, as 16-byte stores at
        // 2-byte (bf16) or 4-byte (fp32) aligned addresses, which gfx950's
        // global memory path takes whole (measured: 384 -> 328 us at the
        // headline shape with L 2047, against element stores and the
        // aligned-block shuffle this replaced).
        if constexpr (RAW && VB == 16) {
            if (t_begin + int64_t(c + 1) * CH <= t_end) {
                if (!prow_ok) return;
#pragma unroll
                for (int k = 0; k < SV; ++k) {
                    const uint4 v = pack16<T, V>(yv + k * V);
                    __builtin_memcpy(Y + ts + k * V, &v, 16);
                }
                return;
            }
        }
        if (!prow_ok) return;
        if (VEC && ts + TS <= t_end) {
#pragma unroll
            for (int k = 0; k < SV; ++k)
                stg_stream<VB>(Y + ts + k * V, pack16<T, V>(yv + k * V));
        } else {
#pragma unroll
            for (int j = 0; j < TS; ++j)
                if (ts + j < t_end) Y[ts + j] = from_f32<T>(yv[j]);
        }
    };

    // Per chunk: scan | barrier | prologue(c+1), loads, epilogue(c) | barrier.
    // Loads: with PAIR, chunks c+2 and c+3 at even c (one and two chunks of
    // lead); otherwise chunk c+3 at every c (two chunks of lead). The
    // epilogue's y stores come after the loads, so no wait for loads (vmcnt,
    // which on this chip also counts stores) waits for fresh stores.
    // Register sets: chunk c+1's inputs are in `next`; the D-skip inputs and
    // gate values alternate between two arrays by chunk parity (no copies).
    constexpr bool PAIR = VEC && sizeof(T) * CH < 128;
    float dxA[TS], gzA[TS], dxB[TS], gzB[TS];
    // The scan runs at a raised wave priority and the per-token phases at the
    // base one: with two waves per SIMD from different workgroups, the
    // VALU-bound scan of one then issues ahead of the latency-bound loads,
    // LDS traffic and stores of the other, which fill the gaps (measured:
    // about 7% less time than equal priorities).
    auto step = [&](int c, Slice& next, Slice& other, const float* dxc, const float* gzc,
                    float* dxn, float* gzn) {
        __builtin_amdgcn_s_setprio(1);
        scan_chunk(c);
        __syncthreads();
        __builtin_amdgcn_s_setprio(0);
        if (c + 1 < nchunks) prologue(c + 1, next, dxn, gzn);
        // (VEC loads of chunks past the end read valid memory and are never used)
        if constexpr (PAIR) {
            if ((c & 1) == 0) load_pair(c + 2, other, next);
        } else {
            if (VEC || c + 3 < nchunks) load_slice(c + 3, next);
        }
        if constexpr (READOUT) epilogue(c, dxc, gzc);
        __syncthreads();
    };
    if (nchunks > 0) {
        if constexpr (PAIR) {
            load_pair(0, sl0, sl1);
            prologue(0, sl0, dxA, gzA);
        } else {
            load_slice(0, sl0);
            if (nchunks > 1) load_slice(1, sl1);
            prologue(0, sl0, dxA, gzA);
            if (nchunks > 2) load_slice(2, sl0);
        }
        __syncthreads();
        // chunk c+1's inputs are in sl1 for even c, sl0 for odd c
        for (int c = 0; c < nchunks; c += 2) {
            step(c, sl1, sl0, dxA, gzA, dxB, gzB);
            if (c + 1 < nchunks) step(c + 1, sl0, sl1, dxB, gzB, dxA, gzA);
        }
    }

    if constexpr (READOUT) {
        if (a.last_state && row_ok && seg == a.segments - 1)
            store_state(a.last_state + (b * a.dim + d) * kN + n0, h);
    } else if constexpr (BASE == 1) {
        const int64_t so = (int64_t(seg) * a.batch * a.dim + b * a.dim + d);
        if (row_ok) store_state(a.seg_state + so * kN + n0, h);
        // Step-size sums were accumulated per (row pr, slice pq); add the G
        // slices of each row in a fixed order.
        sm.lsum[pq][pr] = lsum_acc;
        __syncthreads();
        if (wv == 0 && row_ok) {
            double s = 0.0;
#pragma unroll
            for (int g = 0; g < G; ++g) s += sm.lsum[g][lane];
            a.seg_lsum[so] = s;
        }
    }
}

// ---------------------------------------------------------------------------
// Warp-specialised forward: the output pass (MODE 0) and the state pass
// (MODE 1) of fwd_kernel, computing the same recurrence from the same packed
// B/C records, with the two kinds of work on different waves of a 64-row
// block. NS scan waves (16/NS states of every row each) run only the
// register recurrence, fed by the records through SGPRs and by (l, w) from
// LDS; four io waves stream x, delta and z from HBM, form the per-token
// values, sum the scan waves' partial readouts, gate and store y. LDS holds
// two chunks of each hand-off, so one barrier per 16-token chunk separates
// the roles: during chunk c the scan waves read (l, w) of c and write their
// partial readouts of c, while the io waves write (l, w) of c+1 and read the
// partial readouts of c-1. The scan waves never wait on global memory, and
// the io waves' loads, LDS traffic and stores run beside the scans of other
// waves on the same SIMD instead of between them.
//
// Rows must be whole 4-token vectors (L % 4 == 0): an io lane takes 4
// consecutive tokens of one row per chunk (8 bytes of bf16, 16 of fp32), and
// the lanes of a wave load QC consecutive chunks back to back, one 128-byte
// line per row, tensor by tensor.
constexpr int kWsChunk = 16;  // tokens per chunk of the warp-specialised kernel
constexpr int kWsIo = 4;      // io waves per block

// LDS of the warp-specialised kernel. (l, w): row stride 9 x 16 bytes, so the
// scan lanes' 16-byte reads of one token pair on 8 consecutive rows, and the io
// lanes' writes (4 lanes of a row at 32-byte steps, two rows per 8 lanes),
// each fall in 8 distinct 16-byte bank groups. Partial readouts: 64 bytes per
// row, the 16-byte piece k of row r stored at piece k ^ ((r >> 1) & 3), which
// keeps both the scan lanes' writes (one piece, 8 rows) and the io lanes' reads
// (4 pieces of 2 rows) free of bank conflicts.
template <int NS, bool READOUT>
struct alignas(16) WsSmem {
    static constexpr int kLwB = kWsChunk * 8 + 16;
    unsigned char lw[2][kWave * kLwB];
    float yp[READOUT ? 2 : 1][READOUT ? NS : 1][READOUT ? kWave * kWsChunk : 4];
};
__device__ __forceinline__ int yp_index(int row, int piece) {
    return row * kWsChunk + ((piece ^ ((row >> 1) & 3)) << 2);
}

template <typename T, int NS, bool GATE, int MODE, bool PREF>
__global__ __launch_bounds__(kWave*(NS + kWsIo)) void fwd_ws_kernel(FwdKArgs a) {
    constexpr int CH = kWsChunk;
    constexpr int NG = kN / NS;        // states per scan lane
    constexpr int SB = NS;             // tokens per sub-block (NG * SB = 16)
    constexpr int NSB = CH / SB;       // sub-blocks per chunk
    constexpr bool READOUT = MODE == 0;
    constexpr bool LOADZ = GATE && READOUT;
    // chunks per load group: one 128-byte line per row, or two for fp32 rows
    // without a gate and 4 scan waves (registers allow it there; the rows of
    // such grids are long and far apart in memory, and 256-byte runs per row
    // took the million-token output pass from 607 to 573 us)
    constexpr int QC = ((sizeof(T) == 4 && NS == 4 && !LOADZ) ? 256 : 128) / (CH * int(sizeof(T)));
    static_assert(NS == 4 || NS == 8, "4 or 8 scan waves");
    static_assert(NSB % 2 == 0, "sub-blocks per chunk must be even");
    using S = WsSmem<NS, READOUT>;
    __shared__ S sm;

    const int tid = threadIdx.x;
    const int wv = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int lane = tid % kWave;

    int64_t blk = xcd_tile(blockIdx.x, gridDim.x);
    const int rb = int(blk % a.row_blocks);
    blk /= a.row_blocks;
    const int64_t b = blk % a.batch;
    const int seg = int(blk / a.batch);
    const int64_t d0 = int64_t(rb) * kWave;
    const int64_t t_begin = int64_t(seg) * a.seg_len;
    const int64_t t_end = min(a.L, t_begin + a.seg_len);
    const int nchunks = int((t_end - t_begin + CH - 1) / CH);
    // Both roles run a whole number of io iterations (2 QC chunks each):
    // chunks past the segment's end are identity steps (l = w = 0) whose
    // outputs go to the dump area. The io loop then issues the same memory
    // operations in every iteration, which lets the compiler count its
    // waits for prefetched loads exactly.
    const int nch = (nchunks + 2 * QC - 1) / (2 * QC) * (2 * QC);

    if (wv < NS) {
        // ---------------- scan wave: states n0 .. n0+NG-1 of every row ----------------
        const int64_t d = d0 + lane;
        const bool row_ok = d < a.dim;
        const int n0 = wv * NG;
        float An[NG], h[NG];
#pragma unroll
        for (int j = 0; j < NG; ++j) {
            An[j] = row_ok ? a.A[d * kN + n0 + j] : 0.0f;
            h[j] = (a.h0 && row_ok) ? a.h0[(int64_t(seg) * a.batch * a.dim + b * a.dim + d) * kN + n0 + j]
                                    : 0.0f;
        }
        // this wave's records: sub-block s of the segment at rec0 + s * RS;
        // consecutive sub-blocks (also across chunks) are RS floats apart
        constexpr int RS = NS * kRec;
        // With 4 scan waves the first records of a chunk are loaded during
        // the chunk before; with 8 (one sub-block pair per chunk) that leaves
        // the compiler short of SGPRs at the loop back-edge, so they are
        // loaded at the top of each chunk instead.
        constexpr bool XPF = NSB >= 4;
        const float* rec0 = a.P + ((b * a.psub + t_begin / SB) * NS + wv) * kRec;
        f32x16 B0, C0, B1, C1;
        if constexpr (XPF) {
            B0 = sload64(rec0);
            if constexpr (READOUT) C0 = sload64(rec0 + 16);
        }
        float yA[SB], yB[SB];
#pragma unroll
        for (int e = 0; e < SB; ++e) yB[e] = 0.0f;
        __syncthreads();  // (l, w) of chunk 0 written
        for (int c = 0; c < nch; ++c) {
            const int buf = c & 1;
            const float4* lwrow = reinterpret_cast<const float4*>(&sm.lw[buf][lane * S::kLwB]);
            float* yrow = READOUT ? &sm.yp[buf][wv][0] : nullptr;
            // the chunk's records (past the segment's last chunk that one's:
            // their steps are identities), and the furthest one to prefetch:
            // the next chunk's first, or in the last chunk its own last
            const float* recc = rec0 + int64_t(min(c, nchunks - 1)) * NSB * RS;
            const int nmax = XPF && c + 1 < nchunks ? NSB : NSB - 1;
            if constexpr (!XPF) {
                B0 = sload64(recc);
                if constexpr (READOUT) C0 = sload64(recc + 16);
            }
            float4 lq0[SB / 2], lq1[SB / 2];
#pragma unroll
            for (int e = 0; e < SB / 2; ++e) lq0[e] = lwrow[e];
            auto put = [&](int sb, const float* yv) {  // partial readouts of sub-block sb
#pragma unroll
                for (int m = 0; m < SB / 4; ++m)
                    *reinterpret_cast<float4*>(yrow + yp_index(lane, sb * (SB / 4) + m)) =
                        make_float4(yv[4 * m], yv[4 * m + 1], yv[4 * m + 2], yv[4 * m + 3]);
            };
            auto half = [&](int sb, const f32x16& Bc, const f32x16& Cc, const float4* lc, f32x16& Bn,
                            f32x16& Cn, float4* ln, const float* yprev, float* yv) {
                __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): current operands ready
                __builtin_amdgcn_sched_barrier(0);
                // Next sub-block's records (the next chunk's first after the
                // last) and (l, w) (at the last sub-block the chunk's first
                // again: harmless, reloaded after the barrier). The previous
                // sub-block's partial readouts; at sb = 0 that write goes to
                // the chunk's last slot, which the final write overwrites.
                const float* nrec = recc + min(sb + 1, nmax) * RS;
                Bn = sload64(nrec);
                if constexpr (READOUT) Cn = sload64(nrec + 16);
#pragma unroll
                for (int e = 0; e < SB / 2; ++e) ln[e] = lwrow[((sb + 1) & (NSB - 1)) * (SB / 2) + e];
                if constexpr (READOUT) put((sb + NSB - 1) & (NSB - 1), yprev);
                __builtin_amdgcn_sched_barrier(0);
                float dA[SB][NG], u[SB][NG];
#pragma unroll
                for (int e = 0; e < SB; ++e) {
                    const float l = (e & 1) ? lc[e / 2].z : lc[e / 2].x;
#pragma unroll
                    for (int j = 0; j < NG; ++j) dA[e][j] = exp2_hw(l * An[j]);
                }
#pragma unroll
                for (int e = 0; e < SB; ++e) {
                    const float w = (e & 1) ? lc[e / 2].w : lc[e / 2].y;
#pragma unroll
                    for (int j = 0; j < NG; ++j) u[e][j] = w * Bc[j * SB + e];
                }
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int e = 0; e < SB; ++e) {
                    float acc = 0.0f;
#pragma unroll
                    for (int j = 0; j < NG; ++j) {
                        h[j] = fmaf(dA[e][j], h[j], u[e][j]);
                        if constexpr (READOUT) acc = fmaf(Cc[j * SB + e], h[j], acc);
                    }
                    yv[e] = acc;
                }
            };
            // sub-blocks in pairs (ping-pong operand sets, no copies at the
            // back-edge); a loop rather than a full unroll keeps the two
            // record sets of each pair in fixed SGPRs
#pragma unroll 1
            for (int sb = 0; sb < NSB; sb += 2) {
                half(sb, B0, C0, lq0, B1, C1, lq1, yB, yA);
                half(sb + 1, B1, C1, lq1, B0, C0, lq0, yA, yB);
            }
            if constexpr (READOUT) put(NSB - 1, yB);
            __syncthreads();  // partial readouts of c written; (l, w) of c+1 written
        }
        if constexpr (READOUT) {
            if (a.last_state && row_ok && seg == a.segments - 1) {
                float* dst = a.last_state + (b * a.dim + d) * kN + n0;
#pragma unroll
                for (int k = 0; k < NG / 2; ++k)
                    reinterpret_cast<float2*>(dst)[k] = make_float2(h[2 * k], h[2 * k + 1]);
            }
        } else {
            const int64_t so = int64_t(seg) * a.batch * a.dim + b * a.dim + d;
            if (row_ok) {
                float* dst = a.seg_state + so * kN + n0;
#pragma unroll
                for (int k = 0; k < NG / 2; ++k)
                    reinterpret_cast<float2*>(dst)[k] = make_float2(h[2 * k], h[2 * k + 1]);
            }
        }
        return;
    }

    // ---------------- io wave: 16 rows x 16 tokens per chunk ----------------
    // At a raised priority: the scan waves wait at each chunk's barrier for
    // the io waves' (l, w), so these latency-bound waves issue first and the
    // VALU-bound scans fill their gaps.
    __builtin_amdgcn_s_setprio(1);
    const int io = tid - NS * kWave;  // 0..255
    const int r = io >> 2, q = io & 3;
    const int64_t dp = d0 + r;
    const bool prow_ok = dp < a.dim;
    const int64_t prow = b * a.dim + (prow_ok ? dp : d0);  // clamped for safe reads
    const float biasl = (a.dt_bias && prow_ok) ? a.dt_bias[dp] * kLog2e : 0.0f;
    const float Dd = (a.D && prow_ok) ? a.D[dp] : 0.0f;
    // this lane's row of each tensor; token indices within a row fit in 32 bits
    const T* __restrict__ Xr = static_cast<const T*>(a.x) + prow * a.L;
    const T* __restrict__ DLr = static_cast<const T*>(a.delta) + prow * a.L;
    const T* __restrict__ Zr = LOADZ ? static_cast<const T*>(a.z) + prow * a.L : nullptr;
    T* __restrict__ Yr = READOUT ? static_cast<T*>(a.y) + prow * a.L : nullptr;
    const int tb = int(t_begin), te = int(t_end), L32 = int(a.L);
    using V = typename std::conditional<sizeof(T) == 4, uint4, uint2>::type;
    struct Group {
        V x[QC], d[QC], z[LOADZ ? QC : 1];
    };
    // The lane's 4 tokens of chunk c: a vector past the row's end is read
    // from the row's last vector instead (valid memory, values discarded).
    auto ld = [&](const T* row, int c) -> V {
        const T* p = row + min(tb + c * CH + q * 4, L32 - 4);
        if constexpr (sizeof(T) == 4) {
            const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
            return make_uint4(v.x, v.y, v.z, v.w);
        } else {
            const u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
            return make_uint2(v.x, v.y);
        }
    };
    auto load_group = [&](int k, Group& g) {
#pragma unroll
        for (int j = 0; j < QC; ++j) g.x[j] = ld(Xr, k * QC + j);
#pragma unroll
        for (int j = 0; j < QC; ++j) g.d[j] = ld(DLr, k * QC + j);
        if constexpr (LOADZ) {
#pragma unroll
            for (int j = 0; j < QC; ++j) g.z[j] = ld(Zr, k * QC + j);
        }
    };
    auto unpack4 = [](const V& v, float* o) {
        if constexpr (sizeof(T) == 4) {
            o[0] = __uint_as_float(v.x); o[1] = __uint_as_float(v.y);
            o[2] = __uint_as_float(v.z); o[3] = __uint_as_float(v.w);
        } else {
            o[0] = bf16_lo(v.x); o[1] = bf16_hi(v.x); o[2] = bf16_lo(v.y); o[3] = bf16_hi(v.y);
        }
    };
    double lsum_acc = 0.0;
    uint32_t sink = 0;
    // per-token phase of chunk c (tokens past the segment end: identity
    // steps). Whether the chunk lies wholly inside the segment is the same for
    // the whole wave: only the last chunks take the masking.
    auto prologue = [&](int c, const V& xv, const V& dv, const V& zv, float* dxo, float* gzo) {
        float xs[4], ds[4], zs[4];
        unpack4(xv, xs);
        unpack4(dv, ds);
        if constexpr (LOADZ) unpack4(zv, zs);
        auto body = [&](auto masked) {
            const int nvalid = masked ? min(4, max(0, te - (tb + c * CH + q * 4))) : 4;
            float l[4], w[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                l[e] = softplus_log2_of(fmaf(ds[e], kLog2e, biasl));
                if (masked && e >= nvalid) {
                    l[e] = 0.0f;
                    xs[e] = 0.0f;
                }
                w[e] = l[e] * xs[e];
                if constexpr (MODE == 1) lsum_acc += double(l[e]);
                if constexpr (READOUT) {
                    dxo[e] = Dd * xs[e];
                    if constexpr (LOADZ) gzo[e] = silu(zs[e]);
                }
            }
            float4* dst = reinterpret_cast<float4*>(&sm.lw[c & 1][r * S::kLwB + q * 32]);
            dst[0] = make_float4(l[0], w[0], l[1], w[1]);
            dst[1] = make_float4(l[2], w[2], l[3], w[3]);
        };
        if (tb + (c + 1) * CH <= te) body(std::false_type{});
        else body(std::true_type{});
    };
    // The B/C records of chunk c (2 KB per block: NSB sub-blocks x NS scan
    // waves x 128 bytes) are brought into the scalar data cache, which the
    // CU's waves share, by scalar loads of one dword per 64-byte line from
    // the io waves (a quarter each), one chunk ahead of the scan waves' own
    // loads: those then hit that cache instead of waiting on L2.
    auto prefetch_records = [&](int c) {
        if constexpr (PREF) {
            const int iw = wv - NS;
            const float* base = a.P + ((b * a.psub + (t_begin + int64_t(c) * CH) / SB) * NS) * kRec + iw * 128;
            using CP = const __attribute__((address_space(4))) uint32_t*;
            uint32_t acc = 0;
#pragma unroll
            for (int k = 0; k < 8; ++k) acc ^= *(CP)(reinterpret_cast<uintptr_t>(base + 16 * k));
            sink ^= acc;
        }
    };
    // Chunk c's outputs: every lane issues exactly one vector store, to y
    // when its 4 tokens are inside the segment (t_begin, t_end and ts are
    // multiples of 4: they are all inside or all past it) and its row exists,
    // else to the dump area. With a fixed number of memory operations per
    // chunk the compiler's waits for the next chunks' loads count past the
    // fresh stores instead of draining them.
    auto epilogue = [&](int c, const float* dx, const float* gz) {
        const int ts = tb + c * CH + q * 4;
        float4 acc = *reinterpret_cast<const float4*>(&sm.yp[c & 1][0][yp_index(r, q)]);
#pragma unroll
        for (int g = 1; g < NS; ++g) {
            const float4 v = *reinterpret_cast<const float4*>(&sm.yp[c & 1][g][yp_index(r, q)]);
            acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
        }
        float yv[4] = {acc.x, acc.y, acc.z, acc.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            yv[e] += dx[e];
            if constexpr (LOADZ) yv[e] *= gz[e];
        }
        const bool real = prow_ok && c >= 0 && ts < te;
        T* dst = real ? Yr + ts : static_cast<T*>(a.dump) + 4 * (io & 15);
        if constexpr (sizeof(T) == 4) {
            u32x4 v = {__float_as_uint(yv[0]), __float_as_uint(yv[1]), __float_as_uint(yv[2]),
                       __float_as_uint(yv[3])};
            __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(dst));
        } else {
            const uint4 p = pack16<T, 4>(yv);
            u32x2 v = {p.x, p.y};
            __builtin_nontemporal_store(v, reinterpret_cast<u32x2*>(dst));
        }
    };

    Group g0, g1;
    float dx0[4], gz0[4], dx1[4], gz1[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) dx1[e] = gz1[e] = 0.0f;
    prefetch_records(0);
    load_group(0, g0);
    load_group(1, g1);
    prologue(0, g0.x[0], g0.d[0], LOADZ ? g0.z[0] : g0.x[0], dx0, gz0);
    __syncthreads();
    // Chunk c's inputs are slot c % QC of group (c / QC) % 2; group k + 2 is
    // loaded into the set of group k once its last chunk has been formed
    // (addresses past the row's end read its last vector). The loop is
    // unrolled over 2 QC chunks so that every slot index is a compile-time
    // constant, and every iteration issues the same loads and stores.
    for (int c0 = 0; c0 < nch; c0 += 2 * QC) {
#pragma unroll
        for (int j = 0; j < 2 * QC; ++j) {
            const int c = c0 + j;
            prefetch_records(min(c + 1, nchunks - 1));
            // chunk c - 1's outputs first (chunk -1: a store to the dump
            // area): its D x and gate values share a buffer with chunk c + 1's,
            // which the prologue below overwrites
            if constexpr (READOUT)
                epilogue(c - 1, j & 1 ? dx0 : dx1, j & 1 ? gz0 : gz1);
            Group& gn = ((j + 1) / QC) % 2 == 0 ? g0 : g1;  // set of chunk c + 1
            constexpr int QCc = QC;
            const int sn = (j + 1) % QCc;
            prologue(c + 1, gn.x[sn], gn.d[sn], LOADZ ? gn.z[sn] : gn.x[sn], j & 1 ? dx0 : dx1,
                     j & 1 ? gz0 : gz1);
            if (sn == QC - 1) load_group((c + 1) / QC + 2, gn);
            __syncthreads();
        }
    }
    if constexpr (READOUT) epilogue(nch - 1, dx1, gz1);
    if constexpr (MODE == 1) {
        // step-size sum of the row: the 4 lanes of a row (a quad) add their
        // sums in a fixed order
        double v = lsum_acc;
        const double v1 = __shfl_xor(v, 1, 64);
        v = q & 1 ? v1 + v : v + v1;          // (q0 + q1), (q2 + q3)
        const double v2 = __shfl_xor(v, 2, 64);
        v = q & 2 ? v2 + v : v + v2;          // (q0 + q1) + (q2 + q3)
        if (q == 0 && prow_ok) a.seg_lsum[int64_t(seg) * a.batch * a.dim + b * a.dim + dp] = v;
    }
    if (PREF && a.dim < 0) static_cast<uint32_t*>(a.y)[0] = sink;  // never true: keeps the prefetch loads
}

template <typename T, int NS, int MODE, bool PREF>
hipError_t launch_ws_t(const FwdKArgs& k, bool gate, int64_t blocks, hipStream_t st) {
    const dim3 grid{unsigned(blocks)}, block{unsigned(kWave * (NS + kWsIo))};
    if (gate && MODE == 0)
        hipLaunchKernelGGL((fwd_ws_kernel<T, NS, true, MODE, PREF>), grid, block, 0, st, k);
    else
        hipLaunchKernelGGL((fwd_ws_kernel<T, NS, false, MODE, PREF>), grid, block, 0, st, k);
    return hipGetLastError();
}

template <int MODE>
hipError_t launch_ws(DType dt, const FwdKArgs& k, int ns, bool pref, bool gate, int64_t blocks,
                     hipStream_t st) {
    if (dt == DType::BF16) {
        if (ns == 8) return pref ? launch_ws_t<bf16_bits, 8, MODE, true>(k, gate, blocks, st)
                                 : launch_ws_t<bf16_bits, 8, MODE, false>(k, gate, blocks, st);
        return pref ? launch_ws_t<bf16_bits, 4, MODE, true>(k, gate, blocks, st)
                    : launch_ws_t<bf16_bits, 4, MODE, false>(k, gate, blocks, st);
    }
    if (ns == 8) return pref ? launch_ws_t<float, 8, MODE, true>(k, gate, blocks, st)
                             : launch_ws_t<float, 8, MODE, false>(k, gate, blocks, st);
    return pref ? launch_ws_t<float, 4, MODE, true>(k, gate, blocks, st)
                : launch_ws_t<float, 4, MODE, false>(k, gate, blocks, st);
}

// Pack B and C ([batch, 16, L] of T) into the fp32 record layout above, for
// Lp >= L tokens (a multiple of the chunk), zero past L. One thread writes one
// float4 of a 16-float half-record (B or C of one (b, s, g)), so a wave
// writes 1 KiB contiguously; with G = 4 a float4 is 4 consecutive tokens of
// one row, read as one 8-byte (bf16) or 16-byte (fp32) load when whole.
template <typename T, int G>
__global__ __launch_bounds__(256) void pack_bc_kernel(const T* __restrict__ B, const T* __restrict__ C,
                                                      float* __restrict__ P, int64_t batch, int64_t L,
                                                      int64_t Lp) {
    constexpr int NG = kN / G;
    const int64_t psub = Lp / G;
    const int64_t f = int64_t(blockIdx.x) * 256 + threadIdx.x;  // float4 index
    if (f >= batch * psub * G * 2 * 4) return;
    const int q = int(f % 4);
    const int64_t i = f / 4;                                      // half-record index
    const int k = int(i % 2);
    const int g = int((i / 2) % G);
    const int64_t s = (i / (2 * G)) % psub;
    const int64_t b = i / (2 * G * psub);
    const T* src = (k ? C : B) + (b * kN + g * NG) * L;
    // B is stored times ln 2, so that the scan's input term is (l x) B' with
    // l the step size in log2 units (l ln 2 x B = l x (B ln 2)).
    const float scale = k ? 1.0f : kLn2;
    float v[4];
    if (G == 4 && L % 4 == 0 && s * 4 + 3 < L) {  // row q, tokens 4s..4s+3, aligned and whole
        const T* p = src + q * L + s * 4;
        if constexpr (sizeof(T) == 4) {
            const float4 u = *reinterpret_cast<const float4*>(p);
            v[0] = u.x; v[1] = u.y; v[2] = u.z; v[3] = u.w;
        } else {
            const uint2 u = *reinterpret_cast<const uint2*>(p);
            v[0] = bf16_lo(u.x); v[1] = bf16_hi(u.x); v[2] = bf16_lo(u.y); v[3] = bf16_hi(u.y);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] *= scale;
    } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int idx = 4 * q + e;  // element of the half-record: state row j, token within sub-block
            const int j = idx / G;
            const int64_t t = s * G + idx % G;
            v[e] = t < L ? to_f32(src[j * L + t]) * scale : 0.0f;
        }
    }
    reinterpret_cast<float4*>(P)[f] = make_float4(v[0], v[1], v[2], v[3]);
}

// The same packing for G = 4 and rows of whole 4-token vectors, as a tile
// transpose: a workgroup takes 64 sub-blocks (256 tokens) of one batch entry,
// reads its B and C rows with whole-line loads (consecutive threads on
// consecutive 4-token vectors of one row), places each vector at its record
// position in LDS (padded by one float4 per 32 so that the writes spread
// over the banks), and writes the 2,048 float4s of its records contiguously.
// Each float4 of a record is one 4-token vector of one state row, so the
// tile is a permutation of whole vectors.
template <typename T>
__global__ __launch_bounds__(256) void pack_bc4_kernel(const T* __restrict__ B, const T* __restrict__ C,
                                                      float* __restrict__ P, int64_t L, int64_t Lp) {
    constexpr int kSub = 64;                  // sub-blocks per workgroup
    constexpr int kRecs = kSub * 32;          // float4s of their records (4 groups x 2 x 4)
    __shared__ float4 tile[kRecs + kRecs / 32];
    const int64_t psub = Lp / 4;
    const int64_t tiles = (psub + kSub - 1) / kSub;
    const int64_t b = blockIdx.x / tiles;
    const int64_t s0 = (blockIdx.x % tiles) * kSub;
    const int tid = threadIdx.x;
#pragma unroll
    for (int m = 0; m < kRecs / 256; ++m) {
        const int i = tid + 256 * m;
        const int k = i / (kN * kSub), n = (i / kSub) % kN, sq = i % kSub;
        const int64_t t = (s0 + sq) * 4;
        float v[4] = {0.0f, 0.0f, 0.0f, 0.0f};
        if (t < L) {  // whole: L is a multiple of 4
            const T* p = (k ? C : B) + (b * kN + n) * L + t;
            if constexpr (sizeof(T) == 4) {
                const float4 u = *reinterpret_cast<const float4*>(p);
                v[0] = u.x; v[1] = u.y; v[2] = u.z; v[3] = u.w;
            } else {
                const uint2 u = *reinterpret_cast<const uint2*>(p);
                v[0] = bf16_lo(u.x); v[1] = bf16_hi(u.x); v[2] = bf16_lo(u.y); v[3] = bf16_hi(u.y);
            }
            // B is stored times ln 2 (the scan's input term is (l x) B' with l in log2 units)
            if (k == 0) {
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] *= kLn2;
            }
        }
        const int o = sq * 32 + (n / 4) * 8 + k * 4 + n % 4;  // position among the tile's records
        tile[o + o / 32] = make_float4(v[0], v[1], v[2], v[3]);
    }
    __syncthreads();
    float4* dst = reinterpret_cast<float4*>(P) + (b * psub + s0) * 32;
    const int64_t left = (psub - s0) * 32;  // float4s of this batch entry's records from s0 on
#pragma unroll
    for (int m = 0; m < kRecs / 256; ++m) {
        const int o = tid + 256 * m;
        if (o < left) dst[o] = tile[o + o / 32];
    }
}

// Carry pass: for each (row, n), compose the segments in order,
//   H_{s+1} = 2^(A_n * lsum_s) H_s + state_s,  H_0 = h0 (or 0),
// and write the state entering every segment. 2^(A * sum of l) is the
// product of the per-token decays of the segment.
__global__ __launch_bounds__(256) void carry_kernel(const float* __restrict__ A,
                                                    const float* __restrict__ seg_state,
                                                    const double* __restrict__ seg_lsum,
                                                    const float* __restrict__ h0,
                                                    float* __restrict__ carry, int64_t rows,
                                                    int64_t dim, int32_t segments) {
    const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i >= rows * kN) return;
    const int64_t r = i / kN;
    const int n = int(i % kN);
    const double An = A[(r % dim) * kN + n];
    float H = h0 ? h0[i] : 0.0f;
    carry[i] = H;
    constexpr int U = 8;
    int s = 0;
    for (; s + U <= segments - 1; s += U) {
        float st[U];
        double ls[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            st[u] = seg_state[int64_t(s + u) * rows * kN + i];
            ls[u] = seg_lsum[int64_t(s + u) * rows + r];
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            H = fmaf(exp2_hw(float(An * ls[u])), H, st[u]);
            carry[int64_t(s + u + 1) * rows * kN + i] = H;
        }
    }
    for (; s < segments - 1; ++s) {
        H = fmaf(exp2_hw(float(An * seg_lsum[int64_t(s) * rows + r])), H,
                 seg_state[int64_t(s) * rows * kN + i]);
        carry[int64_t(s + 1) * rows * kN + i] = H;
    }
}

// The same carries for many segments and few chains: a workgroup takes 64
// chains (one per lane) and kCarryW waves, each wave a run of consecutive
// segments. A wave first composes its run from a zero state (the run's decay
// 2^(A_n * its summed steps) and its end state), the runs are then chained in
// order through LDS to give each run its entering state, and each wave
// rescans its run from that state, writing the state entering every segment.
// Chain length: two runs plus the number of waves, instead of all segments.
constexpr int kCarryW = 16;
__global__ __launch_bounds__(64 * kCarryW) void carry_runs_kernel(const float* __restrict__ A,
                                                                 const float* __restrict__ seg_state,
                                                                 const double* __restrict__ seg_lsum,
                                                                 const float* __restrict__ h0,
                                                                 float* __restrict__ carry, int64_t rows,
                                                                 int64_t dim, int32_t segments) {
    __shared__ float agg_a[kCarryW][64], agg_b[kCarryW][64];
    const int lane = threadIdx.x % 64;
    const int w = threadIdx.x / 64;
    const int64_t chains = rows * kN;
    const int64_t i = int64_t(blockIdx.x) * 64 + lane;
    const bool ok = i < chains;
    const int64_t r = ok ? i / kN : 0;
    const int n = int(i % kN);
    const double An = ok ? double(A[(r % dim) * kN + n]) : 0.0;
    const int steps = segments - 1;  // transitions s -> s + 1
    const int per = (steps + kCarryW - 1) / kCarryW;
    const int s0 = min(steps, w * per), s1 = min(steps, s0 + per);
    // 1) the run from zero (loads issued U at a time, ahead of their use)
    constexpr int U = 8;
    float beta = 0.0f;
    double lsum = 0.0;
    if (ok) {
        for (int s = s0; s < s1; s += U) {
            float st[U];
            double ls[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int q = min(s + u, s1 - 1);
                st[u] = seg_state[int64_t(q) * chains + i];
                ls[u] = seg_lsum[int64_t(q) * rows + r];
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                if (s + u < s1) {
                    beta = fmaf(exp2_hw(float(An * ls[u])), beta, st[u]);
                    lsum += ls[u];
                }
            }
        }
    }
    agg_a[w][lane] = exp2_hw(float(An * lsum));
    agg_b[w][lane] = beta;
    __syncthreads();
    // 2) the state entering this wave's run
    float H = (ok && h0) ? h0[i] : 0.0f;
    for (int v = 0; v < w; ++v) H = fmaf(agg_a[v][lane], H, agg_b[v][lane]);
    // 3) rescan the run from it
    if (ok) {
        if (w == 0) carry[i] = H;
        for (int s = s0; s < s1; s += U) {
            float st[U];
            double ls[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int q = min(s + u, s1 - 1);
                st[u] = seg_state[int64_t(q) * chains + i];
                ls[u] = seg_lsum[int64_t(q) * rows + r];
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                if (s + u < s1) {
                    H = fmaf(exp2_hw(float(An * ls[u])), H, st[u]);
                    carry[int64_t(s + u + 1) * chains + i] = H;
                }
            }
        }
    }
}

template <typename T, int G, bool GATE, bool VEC, int MODE>
hipError_t launch_one(const FwdKArgs& k, int64_t blocks, hipStream_t st) {
    hipLaunchKernelGGL((fwd_kernel<T, G, GATE, VEC, MODE>), dim3(unsigned(blocks)),
                       dim3(kWave * G), 0, st, k);
    return hipGetLastError();
}

template <typename T, int G, int MODE>
hipError_t dispatch_gv(const FwdKArgs& k, bool gate, bool vec, int64_t blocks, hipStream_t st) {
    static_assert(MODE < 2 || G == 4, "checkpoints: 4 waves");
    if (MODE == 1 || MODE == 2 || MODE == 5) gate = false;  // no readout: z is never read
    if (gate) return vec ? launch_one<T, G, true, true, MODE>(k, blocks, st)
                         : launch_one<T, G, true, false, MODE>(k, blocks, st);
    return vec ? launch_one<T, G, false, true, MODE>(k, blocks, st)
               : launch_one<T, G, false, false, MODE>(k, blocks, st);
}

template <typename T, int MODE>
hipError_t dispatch(const FwdKArgs& k, int groups, bool gate, bool vec, int64_t blocks,
                    hipStream_t st) {
    switch (groups) {
        case 1: return dispatch_gv<T, 1, MODE>(k, gate, vec, blocks, st);
        case 2: return dispatch_gv<T, 2, MODE>(k, gate, vec, blocks, st);
        case 4: return dispatch_gv<T, 4, MODE>(k, gate, vec, blocks, st);
        case 8: return dispatch_gv<T, 8, MODE>(k, gate, vec, blocks, st);
        default: return hipErrorInvalidValue;
    }
}

template <int MODE>
hipError_t dispatch_dtype(DType dt, const FwdKArgs& k, int groups, bool gate, bool vec,
                          int64_t blocks, hipStream_t st) {
    return dt == DType::BF16 ? dispatch<bf16_bits, MODE>(k, groups, gate, vec, blocks, st)
                             : dispatch<float, MODE>(k, groups, gate, vec, blocks, st);
}

template <typename T>
hipError_t launch_pack(const void* B, const void* C, float* P, int64_t batch, int64_t L,
                       int64_t Lp, int groups, hipStream_t st) {
    const int64_t n = batch * Lp * 2 * 4;  // float4s: batch * (Lp / G) * G * 2 half-records of 4
    const dim3 grid(unsigned((n + 255) / 256)), block(256);
    const T* b = static_cast<const T*>(B);
    const T* c = static_cast<const T*>(C);
    switch (groups) {
        case 1: hipLaunchKernelGGL((pack_bc_kernel<T, 1>), grid, block, 0, st, b, c, P, batch, L, Lp); break;
        case 2: hipLaunchKernelGGL((pack_bc_kernel<T, 2>), grid, block, 0, st, b, c, P, batch, L, Lp); break;
        case 4:
            if (L % 4 == 0) {
                const int64_t tiles = (Lp / 4 + 63) / 64;
                hipLaunchKernelGGL((pack_bc4_kernel<T>), dim3(unsigned(batch * tiles)), block, 0, st, b, c, P, L, Lp);
            } else {
                hipLaunchKernelGGL((pack_bc_kernel<T, 4>), grid, block, 0, st, b, c, P, batch, L, Lp);
            }
            break;
        case 8: hipLaunchKernelGGL((pack_bc_kernel<T, 8>), grid, block, 0, st, b, c, P, batch, L, Lp); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

// The output pass, bracketed by the plan's timing events when it has them;
// with checkpoints wanted (k.ckpt), the 4-wave variant that also stores them.
hipError_t output_pass(DType dt, const FwdKArgs& k, const FwdPlan& p, bool gate, int64_t blocks,
                       hipStream_t st) {
    if (p.ev_begin && hipEventRecord(p.ev_begin, st) != hipSuccess) return hipGetLastError();
    hipError_t e;
    if (p.ws) {
        if (k.cw || k.ckpt) return hipErrorInvalidValue;
        e = launch_ws<0>(dt, k, p.groups, p.pref, gate, blocks, st);
    } else if (k.cw) {
        if (p.groups != 4 || k.ckpt) return hipErrorInvalidValue;
        e = dt == DType::BF16 ? dispatch_gv<bf16_bits, 4, 4>(k, gate, p.vec, blocks, st)
                              : dispatch_gv<float, 4, 4>(k, gate, p.vec, blocks, st);
    } else if (k.ckpt) {
        if (p.groups != 4) return hipErrorInvalidValue;
        e = dt == DType::BF16 ? dispatch_gv<bf16_bits, 4, 3>(k, gate, p.vec, blocks, st)
                              : dispatch_gv<float, 4, 3>(k, gate, p.vec, blocks, st);
    } else {
        e = dispatch_dtype<0>(dt, k, p.groups, gate, p.vec, blocks, st);
    }
    if (e != hipSuccess) return e;
    if (p.ev_end && hipEventRecord(p.ev_end, st) != hipSuccess) return hipGetLastError();
    return hipSuccess;
}

size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

// Padded token count of the packed B/C: whole chunks.
int64_t padded_len(int64_t L) { return (L + kChunk - 1) / kChunk * kChunk; }

__global__ __launch_bounds__(256) void fill_zero_kernel(float* __restrict__ p, int64_t n) {
    const int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;
    if (i < n) p[i] = 0.0f;
}

__global__ __launch_bounds__(256) void copy_f32_kernel(float* __restrict__ dst,
                                                      const float* __restrict__ src, int64_t n) {
    const int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;
    if (i < n) dst[i] = src[i];
}

}  // namespace

// A fill kernel rather than a memset, so that the call stays capturable.
hipError_t launch_fill_zero(float* p, int64_t n, hipStream_t st) {
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(fill_zero_kernel, dim3(unsigned((n + 255) / 256)), dim3(256), 0, st, p, n);
    return hipGetLastError();
}

hipError_t launch_copy_f32(float* dst, const float* src, int64_t n, hipStream_t st) {
    if (n <= 0 || dst == src) return hipSuccess;
    hipLaunchKernelGGL(copy_f32_kernel, dim3(unsigned((n + 255) / 256)), dim3(256), 0, st, dst, src, n);
    return hipGetLastError();
}

// Workspace: packed B/C records; with segments, the segment states, carries
// and step sums; with the warp-specialised kernel, 256 bytes of dump area.
size_t fwd_workspace_bytes(const FwdShape& s, const FwdPlan& p) {
    const size_t packed = size_t(s.batch) * size_t(padded_len(s.L)) * 2 * kN * sizeof(float);
    const size_t dump = p.ws ? 256 : 0;
    if (p.segments <= 1) return align256(packed) + dump;
    const size_t rows = size_t(s.batch) * size_t(s.dim);
    const size_t states = size_t(p.segments) * rows * kN * sizeof(float);
    return align256(packed) + 2 * align256(states) +
           align256(size_t(p.segments) * rows * sizeof(double)) + dump;
}

hipError_t launch_fwd(const FwdTensors& t, const FwdShape& s, const FwdPlan& p, void* workspace,
                      hipStream_t stream) {
    const int64_t Lp = padded_len(s.L);
    unsigned char* ws = static_cast<unsigned char*>(workspace);
    float* P = reinterpret_cast<float*>(ws);
    const size_t packed = size_t(s.batch) * size_t(Lp) * 2 * kN * sizeof(float);
    hipError_t e = s.dtype == DType::BF16
                       ? launch_pack<bf16_bits>(t.B, t.C, P, s.batch, s.L, Lp, p.groups, stream)
                       : launch_pack<float>(t.B, t.C, P, s.batch, s.L, Lp, p.groups, stream);
    if (e != hipSuccess) return e;

    FwdKArgs k{};
    k.x = t.x; k.delta = t.delta; k.z = t.z; k.A = t.A; k.P = P;
    k.D = t.D; k.dt_bias = t.dt_bias; k.y = t.y; k.last_state = t.last_state; k.ckpt = t.ckpt;
    k.cw = t.conv_w; k.cb = t.conv_b; k.cx_prev = t.conv_x_prev;
    k.batch = s.batch; k.L = s.L; k.dim = s.dim;
    k.seg_len = p.segments > 1 ? p.seg_len : s.L;
    k.psub = Lp / p.groups;
    k.segments = p.segments;
    k.row_blocks = int32_t((s.dim + kWave - 1) / kWave);
    if (p.ws) k.dump = ws + fwd_workspace_bytes(s, p) - 256;
    const bool gate = t.z != nullptr;
    const int64_t per_seg = int64_t(k.row_blocks) * s.batch;

    // the convolution's last inputs, after the pass that reads x_prev
    auto conv_last = [&]() -> hipError_t {
        if (!t.conv_w || !t.conv_x_last) return hipSuccess;
        return launch_conv_last(t.x, t.conv_x_prev, t.conv_x_last, s.batch * s.dim, s.L, s.dtype, stream);
    };
    if (p.segments <= 1) {
        k.h0 = t.h0;
        e = output_pass(s.dtype, k, p, gate, per_seg, stream);
        return e != hipSuccess ? e : conv_last();
    }
    const size_t rows = size_t(s.batch) * size_t(s.dim);
    const size_t states = size_t(p.segments) * rows * kN * sizeof(float);
    float* seg_state = reinterpret_cast<float*>(ws + align256(packed));
    float* carry = reinterpret_cast<float*>(ws + align256(packed) + align256(states));
    double* seg_lsum = reinterpret_cast<double*>(ws + align256(packed) + 2 * align256(states));

    // 1) state pass over every segment but the last
    FwdKArgs k1 = k;
    k1.seg_state = seg_state;
    k1.seg_lsum = seg_lsum;
    k1.h0 = nullptr;
    k1.ckpt = nullptr;
    if (p.ws) {
        e = launch_ws<1>(s.dtype, k1, p.groups, p.pref, false, per_seg * (p.segments - 1), stream);
    } else if (t.conv_w) {
        if (p.groups != 4) return hipErrorInvalidValue;
        e = s.dtype == DType::BF16
                ? dispatch_gv<bf16_bits, 4, 5>(k1, false, p.vec, per_seg * (p.segments - 1), stream)
                : dispatch_gv<float, 4, 5>(k1, false, p.vec, per_seg * (p.segments - 1), stream);
    } else {
        e = dispatch_dtype<1>(s.dtype, k1, p.groups, false, p.vec, per_seg * (p.segments - 1), stream);
    }
    if (e != hipSuccess) return e;
    // 2) carries
    e = launch_carry(t.A, seg_state, seg_lsum, t.h0, carry, int64_t(rows), s.dim, p.segments, stream);
    if (e != hipSuccess) return e;
    // 3) output pass from the carried-in states
    k.h0 = carry;
    e = output_pass(s.dtype, k, p, gate, per_seg * p.segments, stream);
    return e != hipSuccess ? e : conv_last();
}

hipError_t launch_carry(const float* A, const float* seg_state, const double* seg_lsum,
                        const float* h0, float* carry, int64_t rows, int64_t dim, int32_t segments,
                        hipStream_t stream) {
    const int64_t nthreads = rows * kN;
    // Many segments over few chains (the long-sequence plans): runs per wave,
    // so that the sequential chain is short; otherwise one thread per chain.
    if (segments > 4 * kCarryW && nthreads <= 65536)
        hipLaunchKernelGGL(carry_runs_kernel, dim3(unsigned((nthreads + 63) / 64)), dim3(64 * kCarryW), 0,
                           stream, A, seg_state, seg_lsum, h0, carry, rows, dim, segments);
    else
        hipLaunchKernelGGL(carry_kernel, dim3(unsigned((nthreads + 255) / 256)), dim3(256), 0, stream,
                           A, seg_state, seg_lsum, h0, carry, rows, dim, segments);
    return hipGetLastError();
}

hipError_t launch_fwd_ckpt(const FwdTensors& t, float* ckpt, const FwdShape& s, float* packed,
                           int32_t segments, int64_t seg_len, float* seg_state, double* seg_lsum,
                           float* carry, bool recompute, hipStream_t stream) {
    const int64_t Lp = padded_len(s.L);
    constexpr int G = 4;
    hipError_t e = s.dtype == DType::BF16
                       ? launch_pack<bf16_bits>(t.B, t.C, packed, s.batch, s.L, Lp, G, stream)
                       : launch_pack<float>(t.B, t.C, packed, s.batch, s.L, Lp, G, stream);
    if (e != hipSuccess) return e;
    if (!recompute) return hipSuccess;
    FwdKArgs k{};
    k.x = t.x; k.delta = t.delta; k.z = t.z; k.A = t.A; k.P = packed;
    k.D = t.D; k.dt_bias = t.dt_bias; k.y = nullptr; k.last_state = nullptr; k.h0 = t.h0;
    k.batch = s.batch; k.L = s.L; k.dim = s.dim;
    k.seg_len = segments > 1 ? seg_len : s.L;
    k.psub = Lp / G; k.segments = segments > 1 ? segments : 1;
    k.row_blocks = int32_t((s.dim + kWave - 1) / kWave);
    k.ckpt = ckpt;
    const int64_t per_seg = int64_t(k.row_blocks) * s.batch;
    const bool vec = (s.L * (s.dtype == DType::BF16 ? 2 : 4)) % 16 == 0;
    if (segments > 1) {
        // the states entering the segments: state pass over all but the last,
        // then the carries
        FwdKArgs k1 = k;
        k1.seg_state = seg_state;
        k1.seg_lsum = seg_lsum;
        k1.h0 = nullptr;  // every segment from zero; h0 enters through the carries
        k1.ckpt = nullptr;
        e = s.dtype == DType::BF16
                ? dispatch_gv<bf16_bits, G, 1>(k1, false, vec, per_seg * (segments - 1), stream)
                : dispatch_gv<float, G, 1>(k1, false, vec, per_seg * (segments - 1), stream);
        if (e != hipSuccess) return e;
        e = launch_carry(t.A, seg_state, seg_lsum, t.h0, carry, s.batch * s.dim, s.dim, segments,
                         stream);
        if (e != hipSuccess) return e;
        k.h0 = carry;
    }
    const int64_t blocks = per_seg * k.segments;
    return s.dtype == DType::BF16 ? dispatch_gv<bf16_bits, G, 2>(k, false, vec, blocks, stream)
                                  : dispatch_gv<float, G, 2>(k, false, vec, blocks, stream);
}

}  // namespace selscan
